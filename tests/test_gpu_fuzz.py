"""A seeded sweep over the call space: random sizes (ragged and aligned), every type triple, all four
layout pairs, padded leading dimensions, batches (an operand shared by every slice at stride 0 now
and then), an optional C (sometimes the same buffer as D) and an optional fused epilogue --
each case against the oracle over every output.  Where the operands qualify for the tiled kernels,
the default choice, a tile configuration drawn at random, and the persistent form are also held bit
for bit against the fallback kernel (every one issues the same MFMA instructions on the same
fragments in the same K order), and the stream-K schedule, whose partial sums are added in another
order, against the oracle.  The cases are a fixed function of their index, so a failure names a
reproducible call."""
import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TYPES = [("f16", "f32", "f32"), ("f16", "f32", "f16"), ("f16", "f16", "f16"), ("bf16", "f32", "bf16"),
         ("bf16", "f32", "f32"), ("i8", "i32", "i32"), ("i8", "i32", "f32"), ("i8", "i32", "bf16"),
         ("e4m3", "f32", "f32"), ("e4m3", "f32", "bf16")]
TILES = ["256x256", "256x256w4", "256x128", "128x128", "64x128"]
CASES = 160


def random_problem(i: int):
    rng = np.random.default_rng([97, i])
    in_t, acc_t, out_t = TYPES[i % len(TYPES)]
    M, N, K = (int(x) for x in rng.integers(1, 600, 3))
    if rng.random() < 0.5:  # aligned sizes reach the tiled kernels' fast operand modes
        M, N, K = (-(-v // 16) * 16 for v in (M, N, K))
    batch = int(rng.choice([1, 1, 1, 2, 3]))
    la, lb = (str(x) for x in rng.choice(["row", "col"], 2))
    pad_a, pad_b, pad_d = (int(x) for x in rng.choice([0, 0, 1, 8, 16], 3))

    def draw(shape):
        if in_t == "i8":
            return rng.integers(-128, 128, shape).astype(np.float64)
        if in_t == "e4m3":
            return rng.standard_normal(shape)
        return rng.uniform(-1, 1, shape)

    A, lda = workloads.store(draw((batch, M, K)), in_t, la, pad_a)
    B, ldb = workloads.store(draw((batch, K, N)), in_t, lb, pad_b)
    ldd = N + pad_d
    p = workloads.Problem(f"fuzz{i}", M, N, K, batch, in_t, acc_t, out_t, la, lb,
                          A, lda, ((M if la == "row" else K) * lda) if batch > 1 else 0,
                          B, ldb, ((K if lb == "row" else N) * ldb) if batch > 1 else 0,
                          ldd=ldd, stride_d=M * ldd, meta={"cfg": "fuzz", "seed": i})
    if rng.random() < 0.5:
        n = batch * M * ldd
        cv = rng.integers(-1000, 1000, n) if out_t == "i32" else rng.uniform(-1, 1, n)
        p.C = workloads.to_bits(cv, out_t)
        p.ldc, p.stride_c = ldd, (M * ldd if batch > 1 else 0)
    ep = None
    if out_t != "i32" and rng.random() < 0.35:
        ep = workloads.make_epilogue(p, i, act=str(rng.choice(["none", "relu", "gelu_tanh"])),
                                     row=bool(rng.random() < 0.7), col=bool(rng.random() < 0.7),
                                     bias=bool(rng.random() < 0.7))
    tile = str(rng.choice(TILES))
    # drawn apart, so that the draws above stay those of the earlier cases: one operand shared by
    # every batch slice (stride 0), and C == D (in place)
    rng2 = np.random.default_rng([99, i])
    if batch > 1 and rng2.random() < 0.3:
        p.A, p.stride_a = p.A[: (M if la == "row" else K) * lda].copy(), 0
    if batch > 1 and rng2.random() < 0.3:
        p.B, p.stride_b = p.B[: (K if lb == "row" else N) * ldb].copy(), 0
    in_place = p.C is not None and rng2.random() < 0.3
    if in_place:
        p.stride_c = p.stride_d
    return p, ep, tile, in_place


def check(got, want, p, ep):
    if ep is None:
        gu.assert_close(got, want, p, where=gu.valid_mask(p))
    else:
        bij = gu.all_bij(p)
        idx = gu.flat_index(p, bij)
        gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("i", range(CASES))
def test_random_call(i, monkeypatch):
    p, ep, tile, in_place = random_problem(i)
    print(f"case {i}: {p.in_type}->{p.out_type} M={p.M} N={p.N} K={p.K} batch={p.batch} "
          f"{p.layout_a}/{p.layout_b} lda={p.lda} ldb={p.ldb} ldd={p.ldd} C={p.C is not None} "
          f"strides a/b={p.stride_a}/{p.stride_b} in_place={in_place} ep={ep.act if ep else None} "
          f"tile={tile}", flush=True)
    got, name = gu.run_dmu(p, ep=ep, return_name=True, in_place=in_place)
    want = gu.run_oracle(p, ep=ep)
    check(got, want, p, ep)
    if "generic" in name:
        return
    mask = gu.valid_mask(p)
    ref = gu.run_dmu(p, ep=ep, force="generic", in_place=in_place)
    gu.assert_bits_equal(got, ref, where=mask)
    forced, fname = gu.run_dmu(p, ep=ep, force=tile, return_name=True, in_place=in_place)
    gu.assert_bits_equal(forced, ref, where=mask)
    monkeypatch.setenv("DMU_PERSIST", "always")
    gu.assert_bits_equal(gu.run_dmu(p, ep=ep, in_place=in_place), ref, where=mask)
    monkeypatch.setenv("DMU_PERSIST", "never")
    monkeypatch.setenv("DMU_STREAMK", "always")
    sk, skname, _ = gu.run_streamk(p, ep=ep)
    check(sk, want, p, ep)
    if p.in_type == "i8" and p.out_type == "i32":
        gu.assert_bits_equal(sk, ref, where=mask)  # integer sums: exact in any order


ATT_TYPES = [("f16", "f32"), ("bf16", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"), ("bf16", "f16")]
ATT_CASES = 24


def random_attention(i: int):
    from tests.test_gpu_attention import Att

    rng = np.random.default_rng([98, i])
    in_t, out_t = ATT_TYPES[i % len(ATT_TYPES)]
    sq, sk = (int(x) for x in rng.integers(1, 700, 2))
    batch = int(rng.choice([1, 1, 2, 3]))
    pad = int(rng.choice([0, 8, 16]))
    scale = float(rng.choice([128 ** -0.5, 0.5, 2.0, -0.3, 0.0]))
    lo, hi = [(-1.0, 1.0), (-3.0, 3.0), (0.0, 1.0)][int(rng.integers(0, 3))]
    return Att(batch, sq, sk, in_t, out_t, 1000 + i, pad=pad, scale=scale, lo=lo, hi=hi)


@pytest.mark.parametrize("i", range(ATT_CASES))
def test_random_attention(i):
    """Fused attention over random query and key counts (ragged around the 256-query and 64-key
    blocks), batches, padded strides, every type pair, scales of either sign (zero included) and
    score ranges that make the running maximum rise often, against the oracle's rows."""
    from tests.test_gpu_attention import check

    att = random_attention(i)
    print(f"attention case {i}: {att.in_t}->{att.out_t} batch={att.batch} sq={att.sq} sk={att.sk} "
          f"ld={att.ldq} scale={att.scale}", flush=True)
    check(att, att.run(), att.want())
