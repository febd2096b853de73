"""Parity of the fused epilogue (dmu_gemm_ex) with the oracle's epilogue.

D = round_out(act(rs(i) * cs(j) * P + bias(j) + C(i, j))) -- per-row and
per-column scales (int8 dequantisation), per-column bias, ReLU / tanh-GELU --
through the C ABI, element by element against the oracle on reduced sizes
(several tiles and ragged tails, every kernel family), bit for bit where every
step is exact (integer-valued data, power-of-two scales), on sampled outputs of
the full-size int8 and bf16 problems, batched with per-batch and shared
vectors, and in place (C == D).
"""
import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

COMBOS = [("c1", "f32"), ("c3", "f16"), ("c2", "bf16"), ("c2", "f32"),
          ("c5", "f32"), ("c5", "f16"), ("c5", "bf16")]
SHAPES = {"c1": dict(M=300, N=270, K=200), "c2": dict(M=520, N=264, K=200),
          "c3": dict(M=300, N=270, K=130), "c5": dict(M=300, N=260, K=384)}


def problem(cfg, out_t, seed, with_c=True, **kw):
    p = workloads.make(cfg, "random", seed, with_c=with_c, **{**SHAPES[cfg], **kw})
    if p.out_type != out_t:
        p = workloads.with_output(p, out_t, seed)
    return p


@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh"])
@pytest.mark.parametrize("cfg,out_t", COMBOS)
@pytest.mark.parametrize("kernel", [None, "generic"])
def test_reduced_parity(cfg, out_t, act, kernel):
    p = problem(cfg, out_t, 11)
    ep = workloads.make_epilogue(p, 3, act=act)
    got = gu.run_dmu(p, force=kernel, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("tile", ["256x256", "256x256w4", "256x128", "128x128", "64x128"])
@pytest.mark.parametrize("cfg,out_t", [("c2", "bf16"), ("c5", "f32")])
def test_every_form_on_every_tile(tile, cfg, out_t):
    """The store code has one instantiation per epilogue form (C or not, scales and bias or
    not, no activation / ReLU / GELU) for wavefront blocks inside D and another path for
    blocks on the M/N edge: every form, on each tiled configuration, on a problem with
    both kinds of block, element by element against the oracle."""
    if tile == "256x256w4" and cfg == "c5":
        pytest.skip("the four-wavefront tile is built for 16-bit inputs")
    for with_c in (False, True):
        p = problem(cfg, out_t, 21, with_c=with_c, M=600, N=560, K=192)
        for vectors in (False, True):
            for act in ("none", "relu", "gelu_tanh"):
                ep = None
                if vectors or act != "none":
                    ep = workloads.make_epilogue(p, 7, act=act, row=vectors, col=vectors, bias=vectors)
                got, name = gu.run_dmu(p, force=tile, ep=ep, return_name=True)
                assert tile in name, name
                want = gu.run_oracle(p, ep=ep)
                bij = gu.all_bij(p)
                idx = gu.flat_index(p, bij)
                if ep is None:
                    gu.assert_close(got[idx], want[idx], p)
                else:
                    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("parts", [(True, False, False), (False, True, False), (False, False, True),
                                   (True, True, False)])
@pytest.mark.parametrize("cfg,out_t", [("c5", "bf16"), ("c2", "f32")])
def test_each_part_alone(cfg, out_t, parts):
    row, col, bias = parts
    p = problem(cfg, out_t, 12, with_c=False)
    ep = workloads.make_epilogue(p, 5, act="none", row=row, col=col, bias=bias)
    got = gu.run_dmu(p, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("cfg", ["c2", "c5"])
def test_exact_epilogue_bit_for_bit(cfg, act):
    """Integer-valued products, power-of-two scales and integer bias and C: every step is
    exact in fp32, so the fp32 output must match the oracle bit for bit."""
    p = workloads.make(cfg, "structured", M=300, N=260, K=256, with_c=True)
    p = workloads.with_output(p, "f32")
    ep = workloads.make_epilogue(p, 4, act=act, exact=True)
    got = gu.run_dmu(p, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    gu.assert_bits_equal(got, want, where=gu.valid_mask(p))


def test_tiled_equals_generic_with_epilogue():
    for cfg, out_t in [("c2", "bf16"), ("c5", "f16"), ("c3", "f16")]:
        p = problem(cfg, out_t, 13)
        ep = workloads.make_epilogue(p, 6, act="gelu_tanh")
        a = gu.run_dmu(p, ep=ep)
        b = gu.run_dmu(p, ep=ep, force="generic")
        gu.assert_bits_equal(a, b, where=gu.valid_mask(p))


@pytest.mark.parametrize("shared", [False, True])
def test_batched_vectors(shared):
    """Per-batch vectors at a padded stride, or one vector shared by every batch (stride 0)."""
    p = workloads.make("c4s", "random", 14, M=200, N=136, K=128, batch=3, with_c=True)
    ep = workloads.make_epilogue(p, 7, act="relu")
    if shared:
        ep.stride_rs = ep.stride_cs = ep.stride_bias = 0
    got = gu.run_dmu(p, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


def test_in_place_c_is_d():
    p = problem("c2", "f32", 15)
    p.ldc, p.stride_c = p.ldd, p.stride_d
    ep = workloads.make_epilogue(p, 8, act="gelu_tanh")
    got = gu.run_dmu(p, ep=ep, in_place=True)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (33, 17, 65), (257, 129, 300)])
def test_ragged_dequantisation(M, N, K):
    p = problem("c5", "bf16", 16, M=M, N=N, K=K)
    ep = workloads.make_epilogue(p, 9, act="gelu_tanh")
    got = gu.run_dmu(p, ep=ep)
    want = gu.run_oracle(p, ep=ep)
    bij = gu.all_bij(p)
    idx = gu.flat_index(p, bij)
    gu.assert_close_epilogue(got[idx], want[idx], p, ep, bij)


@pytest.mark.parametrize("cfg,out_t,act", [("c5", "bf16", "gelu_tanh"), ("c2", "bf16", "relu")])
def test_full_size_sampled(cfg, out_t, act):
    """The full-size int8 and bf16 problems with the whole epilogue, on sampled outputs
    evaluated one by one by the oracle."""
    p = workloads.make(cfg, "random", 0)
    if p.out_type != out_t:
        p = workloads.with_output(p, out_t)
    ep = workloads.make_epilogue(p, 10, act=act)
    got = gu.run_dmu(p, ep=ep)
    bij = gu.sample_bij(p, n=384)
    want = gu.oracle_at(p, bij, ep=ep)
    gu.assert_close_epilogue(got[gu.flat_index(p, bij)], want, p, ep, bij)


def test_no_epilogue_matches_plain_call():
    """dmu_gemm_ex with an empty epilogue is dmu_gemm, bit for bit."""
    p = problem("c2", "bf16", 17)
    a = gu.run_dmu(p)
    b = gu.run_dmu(p, ep=workloads.Epilogue(None, 0, None, 0, None, 0, "none"))
    gu.assert_bits_equal(a, b)
