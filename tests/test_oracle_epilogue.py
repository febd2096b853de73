"""Pins of the oracle's fused epilogue (CPU only).

D = round_out(act(rs(i) * cs(j) * P + bias(j) + C(i, j))), with P the product sum
(the int32 accumulator for int8 inputs).  Pinned against:

* exact brute force (rational arithmetic; the tanh-GELU through Python's decimal
  module, no libm) on tiny shapes for every type pair, activation and batch
  layout of the epilogue vectors;
* closed forms of the structured problems with power-of-two scales and integer
  bias, where every step is exact (row and column orientation at full tile width);
* properties of the tanh-GELU that hold exactly: gelu(x) - gelu(-x) = x,
  gelu(0) = 0, and its limits;
* the int32 wrap-around of the accumulator before dequantisation.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import exact
from tests.test_oracle_gemm import run_oracle, tiny

PAIRS = [("f16", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("bf16", "f32"),
         ("i8", "f32"), ("i8", "bf16"), ("i8", "f16")]
ACTS = ["none", "relu", "gelu_tanh"]


def run_oracle_ep(p, ep, nthreads=None):
    return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, in_type=p.in_type,
                       out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                       batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, C=p.C,
                       ldc=p.ldc, stride_c=p.stride_c, ldd=p.ldd, stride_d=p.stride_d,
                       nthreads=nthreads, **ep.kwargs())


def tiny_ep(in_t, out_t, M, N, K, batch, seed, with_c, pad, la="row", lb="col"):
    p = tiny(in_t, "i32" if in_t == "i8" else out_t, la, lb, M, N, K, batch, seed=seed,
             with_c=with_c and in_t != "i8", pad=pad)
    if in_t == "i8":
        p = workloads.with_output(p, out_t)
        if with_c:
            rng = np.random.default_rng([seed, 5])
            p.C = workloads.to_bits(rng.uniform(-4, 4, batch * M * p.ldd), out_t)
            p.ldc, p.stride_c = p.ldd, (M * p.ldd if batch > 1 else 0)
    return p


def same_bits(got, want, out_t):
    if out_t == "f32":
        return np.array_equal(got.view(np.uint32), want.view(np.uint32))
    return np.array_equal(got, want)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("in_t,out_t", PAIRS)
def test_brute_force_epilogue(in_t, out_t, act):
    cases = [(3, 5, 7, 1, False, 0, (True, True, True)), (4, 6, 9, 2, True, 2, (True, True, True)),
             (5, 3, 4, 3, True, 0, (False, True, True)), (2, 4, 5, 2, False, 1, (True, False, False)),
             (3, 3, 6, 1, True, 0, (False, False, True))]
    for n, (M, N, K, batch, with_c, pad, (r, c, b)) in enumerate(cases):
        p = tiny_ep(in_t, out_t, M, N, K, batch, 300 + n, with_c, pad)
        ep = workloads.make_epilogue(p, n, act=act, row=r, col=c, bias=b)
        got = run_oracle_ep(p, ep, nthreads=2)
        want = exact.brute_gemm(p, ep)
        assert same_bits(got, want, out_t), (M, N, K, batch, act, got[:8], want[:8])


@pytest.mark.parametrize("cfg,out_t", [("c1", "f32"), ("c2", "bf16"), ("c5", "f32"), ("c5", "bf16")])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_structured_closed_form(cfg, out_t, act):
    """A = i mod 16, B = j mod 8: P = K (i mod 16)(j mod 8); power-of-two scales and
    integer bias keep every step exact, so D has a closed form at any size."""
    M, N, K, batch = 300, 200, 256, 2
    p = workloads.make(cfg, "structured", 0, M=M, N=N, K=K, batch=batch)
    p.C = None
    if p.out_type != out_t:
        p = workloads.with_output(p, out_t)
    ep = workloads.make_epilogue(p, 4, act=act, exact=True)
    got = run_oracle_ep(p, ep).reshape(batch, M, p.ldd)[:, :, :N]
    b = np.arange(batch)[:, None, None]
    i = np.arange(M)[None, :, None]
    j = np.arange(N)[None, None, :]
    rs = ep.row_scale[b * ep.stride_rs + i].astype(np.float64)
    cs = ep.col_scale[b * ep.stride_cs + j].astype(np.float64)
    bias = ep.bias[b * ep.stride_bias + j].astype(np.float64)
    v = rs * cs * (K * (i % 16) * (j % 8)) + bias
    if act == "relu":
        v = np.where(v > 0, v, 0.0)
    want = workloads.to_bits(v.reshape(-1), out_t).reshape(v.shape)
    assert np.all(np.abs(v) < 2 ** 24)  # exact in fp32: one rounding to the output type
    assert same_bits(np.ascontiguousarray(got), want, out_t)


def test_gelu_properties():
    """gelu(x) - gelu(-x) = x exactly; gelu(0) = 0; gelu(x) -> x and -> 0 in the tails."""
    xs = np.array([0.0, 0.25, 1.0, 1.5, 3.0, 6.0, 12.0, 40.0], dtype=np.float64)
    K = 1
    A = np.concatenate([xs, -xs]).astype(np.float32)  # rows x and -x, as fp16 values
    A16 = workloads.to_bits(A, "f16")
    B16 = workloads.to_bits(np.ones(1), "f16")
    D = oracle.gemm(len(A), 1, K, A16, 1, B16, 1, in_type="f16", out_type="f32", act="gelu_tanh")
    g_pos, g_neg = D[: len(xs)].astype(np.float64), D[len(xs):].astype(np.float64)
    assert g_pos[0] == 0.0 and g_neg[0] == 0.0
    # each value is within half an fp32 ulp of the true one, so the identity holds to 1 ulp
    ulp = np.spacing(np.maximum(np.abs(g_pos), 1e-30).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs((g_pos - g_neg) - xs) <= 2 * ulp + 1e-37)
    assert g_pos[-1] == 40.0 and g_neg[-1] == 0.0  # saturated tails
    assert np.all(np.signbit(g_neg[1:])) and np.all(np.diff(g_pos) > 0)  # negative or -0


def test_int8_dequant_uses_the_wrapped_int32_accumulator():
    K = 1 << 17
    A = np.full(K, -128, dtype=np.int8)
    B = np.full(K, -128, dtype=np.int8)
    D = oracle.gemm(1, 1, K, A, K, B, 1, in_type="i8", out_type="f32")
    assert D[0] == np.float32(-(2.0 ** 31))
    D = oracle.gemm(1, 1, K, A, K, B, 1, in_type="i8", out_type="f32",
                    row_scale=np.array([0.5], np.float32), bias=np.array([3.0], np.float32))
    assert D[0] == np.float32(-(2.0 ** 30) + 3)


@pytest.mark.parametrize("in_t,out_t,act", [("f16", "f32", "gelu_tanh"), ("i8", "bf16", "relu"),
                                            ("bf16", "bf16", "gelu_tanh")])
def test_gemm_at_with_epilogue_matches_full_product(in_t, out_t, act):
    p = tiny_ep(in_t, out_t, 40, 33, 70, 3, 9, True, 1)
    ep = workloads.make_epilogue(p, 2, act=act)
    full = run_oracle_ep(p, ep)
    rng = np.random.default_rng(1)
    bij = np.stack([rng.integers(0, p.batch, 200), rng.integers(0, p.M, 200),
                    rng.integers(0, p.N, 200)], axis=1)
    got = oracle.gemm_at(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, bij, in_type=p.in_type,
                         out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                         batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, C=p.C,
                         ldc=p.ldc, stride_c=p.stride_c, **ep.kwargs())
    want = full[bij[:, 0] * p.stride_d + bij[:, 1] * p.ldd + bij[:, 2]]
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_no_epilogue_equals_plain_product():
    p = tiny_ep("f16", "f32", 7, 9, 11, 2, 4, True, 0)
    ep = workloads.Epilogue(None, 0, None, 0, None, 0, "none")
    assert np.array_equal(run_oracle_ep(p, ep).view(np.uint32), run_oracle(p).view(np.uint32))
