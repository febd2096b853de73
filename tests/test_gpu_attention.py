"""Parity of the fused attention forward (dmu_attention) with the oracle.

O = softmax(scale Q K^T) V through the C ABI, against the oracle's fp64 rows:
element by element at reduced sizes (ragged query and key counts around the
256-query and 64-key blocks, batch strides, padded leading dimensions, every
type pair), on sampled rows of the full batch-32 4096 x 4096 x 128 problem, and
bit for bit where the softmax is exactly one-hot.

Tolerance (the products' bar moved through the softmax):
    |O - ref| <= max|V| (2 u + 2 |scale| e_S + 1e-5)  [+ 2e-2 |ref| for 16-bit O]
with u the unit roundoff of the input type (P is rounded to it for the P V
product: 2^-11 fp16, 2^-8 bf16) and e_S = 1e-3 sqrt(d) max|Q| max|K| the bound
on the scores S = Q K^T.
"""
import math

import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HD = 128
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


class Att:
    """One attention problem as raw element bits plus the call parameters."""

    def __init__(self, batch, sq, sk, in_t, out_t, seed, pad=0, scale=None, lo=-1.0, hi=1.0):
        rng = np.random.default_rng([91, seed, batch, sq, sk])
        self.batch, self.sq, self.sk, self.in_t, self.out_t = batch, sq, sk, in_t, out_t
        self.ldq = self.ldk = self.ldv = HD + pad
        self.ldo = HD + pad
        self.sqs, self.sks = sq * self.ldq + (8 if pad else 0), sk * self.ldk + (8 if pad else 0)
        self.sos = sq * self.ldo + (8 if pad else 0)
        self.scale = 1.0 / math.sqrt(HD) if scale is None else scale
        self.Q = workloads.to_bits(rng.uniform(lo, hi, batch * self.sqs), in_t)
        self.K = workloads.to_bits(rng.uniform(lo, hi, batch * self.sks), in_t)
        self.V = workloads.to_bits(rng.uniform(-1, 1, batch * self.sks), in_t)

    def oracle_args(self):
        return (self.batch, self.sq, self.sk, HD, HD, self.Q, self.ldq, self.sqs, self.K, self.ldk, self.sks,
                self.V, self.ldv, self.sks)

    def run(self):
        import torch
        dQ, dK, dV = gu.to_dev(self.Q), gu.to_dev(self.K), gu.to_dev(self.V)
        dO = torch.zeros(max(self.batch * self.sos, 1), dtype=gu.out_dtype(self.out_t), device="cuda:0")
        a = dmu.attention_args(self.batch, self.sq, self.sk, HD, dQ, self.ldq, dK, self.ldk, dV, self.ldv, dO,
                               self.ldo, in_type=self.in_t, out_type=self.out_t, scale=self.scale,
                               stride_q=self.sqs, stride_k=self.sks, stride_v=self.sks, stride_o=self.sos)
        dmu.dmu_attention(a)
        torch.cuda.synchronize()
        out = gu.from_dev(dO, self.out_t)
        return np.stack([out[b * self.sos: b * self.sos + self.sq * self.ldo].reshape(self.sq, self.ldo)[:, :HD]
                         for b in range(self.batch)])

    def want(self):
        full = oracle.attention(*self.oracle_args(), in_type=self.in_t, out_type=self.out_t, scale=self.scale,
                                ldo=HD, stride_o=self.sq * HD)
        return full.reshape(self.batch, self.sq, HD)

    def want_rows(self, rows):
        return oracle.attention_rows(*self.oracle_args(), rows, in_type=self.in_t, out_type=self.out_t,
                                     scale=self.scale)

    def tolerance(self, ref_vals):
        q = np.abs(gu.values(self.Q, self.in_t)).max()
        k = np.abs(gu.values(self.K, self.in_t)).max()
        v = np.abs(gu.values(self.V, self.in_t)).max()
        e_s = 1e-3 * math.sqrt(HD) * q * k
        tol = v * (2 * UNIT[self.in_t] + 2 * abs(self.scale) * e_s + 1e-5)  # the scores' error scales by |scale|
        if self.out_t != "f32":
            tol = tol + 2e-2 * np.abs(ref_vals)
        return tol


def check(att, got, want):
    g, w = gu.values(got.reshape(-1), att.out_t), gu.values(want.reshape(-1), att.out_t)
    tol = att.tolerance(w)
    err = np.abs(g - w)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{bad.size}/{g.size} outside tolerance; worst {np.nanmax(err):.3e}; first {bad[:5]}: "
                           f"got {g[bad[:5]]} want {w[bad[:5]]}")


@pytest.mark.parametrize("in_t,out_t", [("f16", "f32"), ("bf16", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                        ("f16", "bf16"), ("bf16", "f16")])
def test_reduced_parity(in_t, out_t):
    att = Att(2, 300, 200, in_t, out_t, 1)
    check(att, att.run(), att.want())


@pytest.mark.parametrize("sq,sk", [(1, 1), (1, 64), (255, 63), (256, 65), (257, 129), (513, 1), (40, 300)])
def test_ragged_sizes(sq, sk):
    att = Att(1, sq, sk, "f16", "f32", 2)
    check(att, att.run(), att.want())


def test_padded_and_strided():
    att = Att(3, 130, 70, "bf16", "f32", 3, pad=8)
    check(att, att.run(), att.want())


def test_large_scores_stay_finite():
    """Scores of several hundred: the running maximum keeps every exponent <= 8 (it is raised
    whenever a block's maximum passes it by more than that), so nothing overflows."""
    att = Att(1, 64, 150, "f16", "f32", 4, scale=40.0)
    got = att.run()
    assert np.all(np.isfinite(got))
    check(att, got, att.want())


def test_one_hot_softmax_is_exact():
    """Query i's key (5 i + 3) mod sk dominates by 300 after scaling: the softmax is
    exactly one-hot and O(i) is that key's row of V, bit for bit."""
    sq, sk = 70, 130
    att = Att(1, sq, sk, "f16", "f16", 5, scale=300.0)
    Qv = np.zeros((sq, HD))
    Kv = np.zeros((sk, HD))
    for j in range(sk):
        Kv[j, j % HD] = 1.0 if j < HD else 0.0
    for j in range(HD, sk):  # keys past d: a second coordinate, half weight
        Kv[j, (j - HD) % HD] = 0.5
    for i in range(sq):
        Qv[i, (5 * i + 3) % HD] = 1.0
    att.Q = workloads.to_bits(Qv.ravel(), "f16")
    att.K = workloads.to_bits(Kv.ravel(), "f16")
    got = att.run()
    want = att.want()
    assert np.array_equal(got, want)
    Vm = att.V.reshape(sk, HD)
    for i in range(sq):
        assert np.array_equal(got[0, i], Vm[(5 * i + 3) % HD]), i


def test_full_size_sampled_rows():
    """The batch-32 attention-shaped problem (4096 queries, 4096 keys, d = 128, fp16 in,
    fp32 out), fused, on sampled rows evaluated one by one by the oracle."""
    att = Att(32, 4096, 4096, "f16", "f32", 6)
    got = att.run()
    rng = np.random.default_rng(7)
    rows = np.array(sorted({(0, 0), (31, 4095), (5, 255), (5, 256), (17, 4095)} |
                           {(int(rng.integers(32)), int(rng.integers(4096))) for _ in range(120)}))
    want = att.want_rows(rows)
    check(att, np.stack([got[b, i] for b, i in rows]), want)


@pytest.mark.parametrize("scale", [-0.25, -1.0 / math.sqrt(HD)])
def test_negative_scale(scale):
    """A negative scale: the kernel negates Q (exactly) and uses |scale|."""
    att = Att(2, 100, 150, "bf16", "f32", 8, scale=scale)
    check(att, att.run(), att.want())


def test_zero_scale_is_mean_of_v():
    """scale = 0: every key gets the same weight, so O(i) is the mean of V's rows for every query."""
    att = Att(1, 40, 130, "f16", "f32", 9, scale=0.0)
    got = att.run()
    check(att, got, att.want())
    mean = gu.values(att.V, "f16").reshape(130, HD).mean(axis=0)
    assert np.max(np.abs(got[0] - mean)) <= 2 * UNIT["f16"] + 1e-6


@pytest.mark.parametrize("batch,sq", [(13, 20), (5, 600)])
def test_grid_not_a_multiple_of_eight(batch, sq):
    """Workgroup counts of 13 and 15 cover every query row once after the XCD renumbering."""
    att = Att(batch, sq, 70, "f16", "f16", 10)
    check(att, att.run(), att.want())
