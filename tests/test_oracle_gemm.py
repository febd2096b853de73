"""Pins of the oracle GEMM (CPU only).

* exact brute force (rational sums, Python big ints) on tiny shapes covering
  every layout pair, padded leading dimensions, batches with strides, a C
  operand, and each (input, output) type pair;
* the worked values of the layout experiment (tests/golden);
* closed forms of the structured workloads, including the ragged K tail of the
  5000 x 3000 x 2050 problem and the batch-dependent attention-shaped pair;
* int8 extremes; selected-element evaluation equal to the full product.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_oracle(p, nthreads=None):
    return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, in_type=p.in_type,
                       out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                       batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, C=p.C,
                       ldc=p.ldc, stride_c=p.stride_c, ldd=p.ldd, stride_d=p.stride_d,
                       nthreads=nthreads)


def tiny(in_t, out_t, la, lb, M, N, K, batch, seed, with_c, pad):
    cfg = "c5" if in_t == "i8" else "c1"
    p = workloads.make(cfg, "random", seed, M=M, N=N, K=K, batch=batch, pad=pad, with_c=with_c)
    if in_t != "i8":
        # re-type the draw: same seeded values rounded to the requested input type
        rng = np.random.default_rng([seed, M, N, K])
        lda, ldb, sa, sb = workloads._layout_params(M, N, K, la, lb, pad)
        a = workloads.to_bits(rng.uniform(-1, 1, (batch, M, K)).reshape(-1), in_t).reshape(batch, M, K)
        b = workloads.to_bits(rng.uniform(-1, 1, (batch, K, N)).reshape(-1), in_t).reshape(batch, K, N)
        p.A, p.B = workloads._storage(a, la, lda), workloads._storage(b, lb, ldb)
        p.lda, p.ldb = lda, ldb
        p.stride_a, p.stride_b = (sa, sb) if batch > 1 else (0, 0)
        p.in_type, p.out_type = in_t, out_t
        p.layout_a, p.layout_b = la, lb
        if with_c:
            p.C = workloads.to_bits(rng.uniform(-1, 1, batch * M * p.ldd), out_t)
            p.ldc, p.stride_c = p.ldd, (M * p.ldd if batch > 1 else 0)
        else:
            p.C = None
    else:
        lda, ldb, sa, sb = workloads._layout_params(M, N, K, la, lb, pad)
        rng = np.random.default_rng([seed, M, N, K])
        a = rng.integers(-128, 128, (batch, M, K)).astype(np.int8)
        b = rng.integers(-128, 128, (batch, K, N)).astype(np.int8)
        p.A, p.B = workloads._storage(a, la, lda), workloads._storage(b, lb, ldb)
        p.lda, p.ldb, p.layout_a, p.layout_b = lda, ldb, la, lb
        p.stride_a, p.stride_b = (sa, sb) if batch > 1 else (0, 0)
    return p


TYPE_PAIRS = [("f16", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("bf16", "f32"), ("i8", "i32")]
LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")]


@pytest.mark.parametrize("in_t,out_t", TYPE_PAIRS)
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_brute_force_tiny(in_t, out_t, la, lb):
    cases = [(3, 5, 7, 1, False, 0), (8, 8, 8, 2, True, 3), (5, 2, 17, 1, True, 1),
             (1, 4, 1, 3, False, 2), (4, 3, 2, 1, True, 0)]
    for n, (M, N, K, batch, with_c, pad) in enumerate(cases):
        p = tiny(in_t, out_t, la, lb, M, N, K, batch, seed=100 + n, with_c=with_c, pad=pad)
        got = run_oracle(p, nthreads=3)
        want = exact.brute_gemm(p)
        if out_t == "f32":
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (M, N, K)
        else:
            assert np.array_equal(got, want), (M, N, K)


def test_layout_experiment_golden():
    """The two cells the layout experiment works out by hand (16 x 8 x 16, D = 16*i*j)."""
    lines = [l.split() for l in open(os.path.join(GOLDEN, "layout_experiment_16x8x16.txt"))
             if l.strip() and not l.startswith("#")]
    M, N, K = map(int, lines[0])
    a = np.repeat(np.arange(M, dtype=np.float64)[:, None], K, axis=1)  # A[i][k] = i
    b = np.repeat(np.arange(N, dtype=np.float64)[None, :], K, axis=0)  # B[k][j] = j
    for t in ("f16", "bf16"):
        D = oracle.gemm(M, N, K, workloads.to_bits(a.reshape(-1), t), K,
                        workloads.to_bits(b.reshape(-1), t), N, in_type=t, out_type="f32")
        D = D.reshape(M, N)
        for i, j, v in lines[1:]:
            assert D[int(i), int(j)] == float(v)
        assert np.array_equal(D, 16.0 * np.outer(np.arange(M), np.arange(N)))


def test_structured_closed_form_c1_c2_c5():
    for cfg, kw in (("c1", {}), ("c2", dict(M=96, N=40, K=4096)), ("c5", dict(M=48, N=24, K=8192))):
        p = workloads.make(cfg, "structured", **kw)
        D = run_oracle(p).reshape(p.M, p.ldd)[:, : p.N].astype(np.float64)
        if p.out_type == "bf16":
            D = exact.bf16_values(D.astype(np.uint16)).reshape(p.M, p.N)
        want = p.K * np.outer(np.arange(p.M) % 16, np.arange(p.N) % 8)
        assert np.array_equal(D, want), cfg


def test_structured_c3_ragged_k_tail():
    """A[i][k] = [k%16 == i%16], B = j%8 over K = 2050: rows with i%16 in {0,1} see the
    two tail values k = 2048, 2049 and get 129*(j%8); the rest get 128*(j%8)."""
    p = workloads.make("c3", "structured", M=40, N=24)
    D = exact.f16_values(run_oracle(p)).reshape(p.M, p.ldd)[:, : p.N]
    n_i = np.where(np.arange(p.M) % 16 < 2, 129, 128)
    assert np.array_equal(D, np.outer(n_i, np.arange(p.N) % 8))


def test_structured_attention_pair():
    p = workloads.make("c4s", "structured", M=64, N=24, batch=3)
    S = run_oracle(p).reshape(p.batch, p.M, p.ldd)[:, :, : p.N]
    bi = (np.arange(p.M)[None, :, None] + np.arange(p.batch)[:, None, None]) % 16
    assert np.array_equal(S, 128.0 * bi * (np.arange(p.N) % 8)[None, None, :])

    q = workloads.make("c4o", "structured", M=40, N=16, K=256, batch=3)
    O = run_oracle(q).reshape(q.batch, q.M, q.ldd)[:, :, : q.N]
    b = np.arange(q.batch)[:, None, None]
    src = (np.arange(q.M)[None, :, None] + b) % q.K
    want = ((src + 3 * b + np.arange(q.N)[None, None, :]) % 64) - 32.0
    assert np.array_equal(O, want)


def test_int8_extremes():
    K = 8192
    A = np.full(2 * K, -128, dtype=np.int8)
    B = np.full(K * 3, -128, dtype=np.int8)
    D = oracle.gemm(2, 3, K, A, K, B, K, in_type="i8", out_type="i32", layout_b="col")
    assert np.all(D == 8192 * 16384)
    B[:] = 127
    D = oracle.gemm(2, 3, K, A, K, B, K, in_type="i8", out_type="i32", layout_b="col")
    assert np.all(D == -128 * 127 * 8192)
    # wrap-around narrowing of the int64 sum (2^17 * 2^14 = 2^31 -> -2^31)
    K = 1 << 17
    A = np.full(K, -128, dtype=np.int8)
    B = np.full(K, -128, dtype=np.int8)
    D = oracle.gemm(1, 1, K, A, K, B, 1, in_type="i8", out_type="i32")
    assert D[0] == -(2 ** 31)


@pytest.mark.parametrize("cfg,batch", [("c3", 1), ("c5", 3), ("c4s", 2)])
def test_gemm_at_matches_full_product(cfg, batch):
    p = workloads.make(cfg, "random", 3, M=70, N=33, K=130, batch=batch, with_c=True)
    full = run_oracle(p)
    rng = np.random.default_rng(0)
    bij = np.stack([rng.integers(0, p.batch, 300), rng.integers(0, p.M, 300),
                    rng.integers(0, p.N, 300)], axis=1)
    got = oracle.gemm_at(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, bij, in_type=p.in_type,
                         out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                         batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b,
                         C=p.C, ldc=p.ldc, stride_c=p.stride_c)
    want = full[bij[:, 0] * p.stride_d + bij[:, 1] * p.ldd + bij[:, 2]]
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_thread_count_does_not_change_result():
    p = workloads.make("c2", "random", 1, M=67, N=45, K=300)
    a = run_oracle(p, nthreads=1)
    b = run_oracle(p, nthreads=7)
    assert np.array_equal(a, b)


def test_empty_and_k_zero():
    p = workloads.make("c1", "random", 0, M=4, N=5, K=0, with_c=True)
    D = run_oracle(p)
    assert np.array_equal(D.view(np.uint32), p.C.view(np.uint32))  # K = 0 => D = C
    z = oracle.gemm(0, 5, 3, np.zeros(0, np.uint16), 3, np.zeros(15, np.uint16), 5,
                    in_type="f16", out_type="f32")
    assert z.size == 0


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):  # integer output takes no epilogue
        oracle.gemm(2, 2, 2, np.zeros(4, np.int8), 2, np.zeros(4, np.int8), 2,
                    in_type="i8", out_type="i32", act="relu")
    with pytest.raises(ValueError):
        oracle.gemm(2, 2, 2, np.zeros(4, np.int8), 2, np.zeros(4, np.int8), 2,
                    in_type="i8", out_type="i32", bias=np.zeros(2, np.float32))
    with pytest.raises(ValueError):  # fp16 inputs cannot give int32 output
        oracle.gemm(2, 2, 2, np.zeros(4, np.uint16), 2, np.zeros(4, np.uint16), 2,
                    in_type="f16", out_type="i32")
    with pytest.raises(ValueError):  # buffer too small for the stated shape
        oracle.gemm(4, 4, 4, np.zeros(8, np.uint16), 4, np.zeros(16, np.uint16), 4,
                    in_type="f16", out_type="f32")


@pytest.mark.parametrize("t,terms,want", [
    # bf16: 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7; the 2^-30 term puts the
    # exact sum above it (round up), but an fp32 intermediate would drop that term
    # (fp32 spacing at 1 is 2^-23) and round the tie to even (down to 1).
    ("bf16", [1.0, 2.0 ** -8, 2.0 ** -30], 0x3F81),
    # fp16: 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10; 2^-24 is itself a tie
    # of fp32 at 1 and would be lost through an fp32 intermediate.
    ("f16", [1.0, 2.0 ** -11, 2.0 ** -24], 0x3C01),
])
def test_single_rounding_of_the_fp64_sum(t, terms, want):
    """The sum is rounded once, from fp64, to the 16-bit output type (no fp32 stage)."""
    K = len(terms)
    A = workloads.to_bits(np.array(terms), t)
    B = workloads.to_bits(np.ones(K), t)
    assert np.array_equal(oracle.decode(t, A), terms)  # the terms are exact in t
    D = oracle.gemm(1, 1, K, A, K, B, 1, in_type=t, out_type=t)
    assert int(D[0]) == want
    # and with the k order reversed the result is the same (the fp64 sum is exact here)
    D = oracle.gemm(1, 1, K, A[::-1].copy(), K, B, 1, in_type=t, out_type=t)
    assert int(D[0]) == want
