"""Pins of the oracle's FP8 e4m3 input path (CPU only).

"Tensor Cores, CUTLASS and CuTe" lists FP8 e4m3 inputs with an fp32 accumulator
(section 2.1) and builds FP8 GEMMs in its CUTLASS section (6.5).  The oracle
decodes e4m3 to exact fp64 and reuses the fp64 GEMM path.  Pinned here by:

* all 256 codes against torch's float8_e4m3fn conversion (a library routine);
* landmark values of the format's definition (largest finite 448, smallest
  subnormal 2^-9, smallest normal 2^-6, no infinities, S.1111.111 is NaN);
* exact brute force (rational sums) on tiny shapes for every layout pair and
  every output type, with batches, padding and C;
* the structured closed form D = K (i mod 16)(j mod 8) and the all-448 extreme;
* NaN inputs reaching exactly the outputs whose sums contain them.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests import exact
from tests.test_oracle_gemm import LAYOUTS, run_oracle


def test_decode_matches_library_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e4m3", codes)
    want = exact.e4m3_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))  # -0 included


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0xB8, -1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x77, 240.0), (0x78, 256.0),
])
def test_decode_landmarks(code, value):
    got = oracle.decode("e4m3", np.array([code], dtype=np.uint8))[0]
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value), (hex(code), got)


@pytest.mark.parametrize("code", [0x7F, 0xFF])
def test_decode_nan(code):
    assert np.isnan(oracle.decode("e4m3", np.array([code], dtype=np.uint8))[0])


def test_no_infinities():
    vals = oracle.decode("e4m3", np.arange(256, dtype=np.uint8))
    assert not np.any(np.isinf(vals))
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0


def tiny_f8(out_t, la, lb, M, N, K, batch, seed, with_c, pad, lo=-4.0, hi=4.0):
    p = workloads.make("c1", "random", seed, M=M, N=N, K=K, batch=batch, pad=pad, with_c=False)
    rng = np.random.default_rng([seed, M, N, K, 8])
    lda, ldb, sa, sb = workloads._layout_params(M, N, K, la, lb, pad)
    a = workloads.to_bits(rng.uniform(lo, hi, batch * M * K), "e4m3").reshape(batch, M, K)
    b = workloads.to_bits(rng.uniform(lo, hi, batch * K * N), "e4m3").reshape(batch, K, N)
    p.A, p.B = workloads._storage(a, la, lda), workloads._storage(b, lb, ldb)
    p.lda, p.ldb, p.layout_a, p.layout_b = lda, ldb, la, lb
    p.stride_a, p.stride_b = (sa, sb) if batch > 1 else (0, 0)
    p.in_type, p.out_type = "e4m3", out_t
    if out_t != "f32":
        p.ldd = N
        p.stride_d = M * N if batch > 1 else M * N
    if with_c:
        p.C = workloads.to_bits(rng.uniform(-1, 1, batch * M * p.ldd), out_t)
        p.ldc, p.stride_c = p.ldd, (M * p.ldd if batch > 1 else 0)
    else:
        p.C = None
    return p


@pytest.mark.parametrize("out_t", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_brute_force_tiny(out_t, la, lb):
    cases = [(3, 5, 7, 1, False, 0), (8, 8, 8, 2, True, 3), (5, 2, 17, 1, True, 1),
             (1, 4, 1, 3, False, 2), (4, 3, 33, 1, True, 0)]
    for n, (M, N, K, batch, with_c, pad) in enumerate(cases):
        p = tiny_f8(out_t, la, lb, M, N, K, batch, seed=300 + n, with_c=with_c, pad=pad)
        got = run_oracle(p, nthreads=2)
        want = exact.brute_gemm(p)
        if out_t == "f32":
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (M, N, K)
        else:
            assert np.array_equal(got, want), (M, N, K)


def test_subnormal_products_are_exact():
    """Products of e4m3 subnormals (down to 2^-18) summed exactly and rounded once."""
    M, N, K = 4, 3, 9
    p = tiny_f8("f32", "row", "col", M, N, K, 1, seed=9, with_c=False, pad=0, lo=-0.01, hi=0.01)
    vals = oracle.decode("e4m3", p.A)
    assert np.any((vals != 0) & (np.abs(vals) < 2.0 ** -6))  # subnormals present
    got = run_oracle(p)
    assert np.array_equal(got.view(np.uint32), exact.brute_gemm(p).view(np.uint32))


def test_structured_closed_form():
    """A = i mod 16, B = j mod 8 (exact in e4m3): D = K (i mod 16)(j mod 8)."""
    M, N, K = 40, 24, 200
    i = np.arange(M) % 16
    j = np.arange(N) % 8
    A = workloads.to_bits(np.repeat(i[:, None], K, axis=1).astype(np.float64).ravel(), "e4m3")
    Bt = workloads.to_bits(np.repeat(j[:, None], K, axis=1).astype(np.float64).ravel(), "e4m3")
    D = oracle.gemm(M, N, K, A, K, Bt, K, in_type="e4m3", out_type="f32", layout_a="row", layout_b="col")
    assert np.array_equal(D.reshape(M, N), (K * np.outer(i, j)).astype(np.float32))


def test_largest_values():
    """All entries 448 (and -448 in B): D = -K 448^2, exact in fp32."""
    M, N, K = 3, 5, 64
    A = np.full(M * K, 0x7E, dtype=np.uint8)
    B = np.full(K * N, 0xFE, dtype=np.uint8)
    D = oracle.gemm(M, N, K, A, K, B, N, in_type="e4m3", out_type="f32")
    assert np.all(D == np.float32(-K * 448.0 * 448.0))


def test_nan_reaches_exactly_its_row_and_column():
    M, N, K = 4, 5, 6
    A = workloads.to_bits(np.ones(M * K), "e4m3")
    B = workloads.to_bits(np.ones(K * N), "e4m3")
    A[2 * K + 3] = 0x7F  # A(2, 3) is NaN
    D = oracle.gemm(M, N, K, A, K, B, N, in_type="e4m3", out_type="f32").reshape(M, N)
    assert np.all(np.isnan(D[2])) and not np.any(np.isnan(np.delete(D, 2, axis=0)))
    assert np.all(np.delete(D, 2, axis=0) == K)


def test_gemm_at_matches_full_product():
    p = tiny_f8("bf16", "row", "col", 9, 7, 45, 2, seed=11, with_c=True, pad=1)
    full = run_oracle(p)
    bij = np.array([(b, i, j) for b in range(2) for i in range(9) for j in range(7)], dtype=np.int64)
    sel = oracle.gemm_at(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, bij, in_type="e4m3", out_type="bf16",
                         layout_a="row", layout_b="col", batch=2, stride_a=p.stride_a, stride_b=p.stride_b,
                         C=p.C, ldc=p.ldc, stride_c=p.stride_c)
    idx = bij[:, 0] * p.stride_d + bij[:, 1] * p.ldd + bij[:, 2]
    assert np.array_equal(sel, full[idx])


def test_rejects_integer_output():
    A = np.zeros(4, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm(2, 2, 2, A, 2, A, 2, in_type="e4m3", out_type="i32")
