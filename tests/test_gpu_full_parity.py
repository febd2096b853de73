"""Every output of the full-size problems against the oracle (the page's own practice in
"Tensor Cores, CUTLASS and CuTe" section 4.4: the whole 4096^3 result is compared with a
reference), through the C ABI, in the launch configuration the benchmark times:

* 4096^3 bf16 (A, B row-major, bf16 out) and 5000 x 3000 x 2050 fp16 (B column-major, fp16
  out): all outputs against the full oracle product, to the stated tolerance;
* the batched attention-shaped pair (batch 32): the whole batched call, then one full batch
  slice (the last, whose operands sit furthest from the base pointers) against the oracle;
* 8192^3 int8 (B column- and row-major): bit-exact by an exact Freivalds check -- D x = A (B x) in int64 for three
  random integer vectors x, which a single wrong element fails with probability at least
  1 - 1/2048 per vector (the full oracle product, 1.1 T multiply-adds, would take minutes).

The oracle's full outputs are cached per input digest (tests/oracle_cache.py)."""
import dataclasses

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu
from tests import oracle_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", ["c2", "c3"])
def test_every_output_at_full_size(cfg):
    p = workloads.make(cfg, "random", 0)
    got = gu.run_dmu(p)
    want = oracle_cache.full_output(p, gu.run_oracle)
    gu.assert_close(got, want, p, where=gu.valid_mask(p))


def slice_problem(p, b):
    """Batch slice b of a batched problem as a problem of its own."""
    ea = (p.M - 1) * p.lda + p.K if p.layout_a == "row" else (p.K - 1) * p.lda + p.M
    eb = (p.K - 1) * p.ldb + p.N if p.layout_b == "row" else (p.N - 1) * p.ldb + p.K
    return dataclasses.replace(p, batch=1, A=p.A[b * p.stride_a: b * p.stride_a + ea], stride_a=0,
                               B=p.B[b * p.stride_b: b * p.stride_b + eb], stride_b=0, C=None, stride_c=0,
                               stride_d=p.M * p.ldd, meta=dict(p.meta, slice=b))


@pytest.mark.parametrize("cfg", ["c4s", "c4o"])
def test_last_batch_slice_every_output(cfg):
    import torch

    p = workloads.make(cfg, "random", 0)
    assert p.C is None
    dA, dB = gu.to_dev(p.A), gu.to_dev(p.B)
    dD = torch.zeros(p.batch * p.stride_d, dtype=gu.out_dtype(p.out_type), device="cuda:0")
    import dense_matrix_unit_tiled_amd as dmu

    dmu.dmu_gemm(gu.make_args(p, dA, dB, dD))
    torch.cuda.synchronize()
    b = p.batch - 1
    got = gu.from_dev(dD[b * p.stride_d: (b + 1) * p.stride_d], p.out_type)
    del dD
    s = slice_problem(p, b)
    want = oracle_cache.full_output(s, gu.run_oracle)
    gu.assert_close(got, want, s, where=gu.valid_mask(s))


@pytest.mark.parametrize("cfg", ["c5", "c5nn"])
def test_int8_full_size_freivalds(cfg):
    p = workloads.make(cfg, "random", 0)
    got = gu.run_dmu(p).astype(np.int64).reshape(p.M, p.ldd)[:, : p.N]
    A = p.A.reshape(p.M, p.lda)[:, : p.K].astype(np.int64)   # row-major M x K
    if p.layout_b == "col":
        Bt = p.B.reshape(p.N, p.ldb)[:, : p.K].astype(np.int64)  # column-major B: row j holds B(:, j)
    else:
        Bt = p.B.reshape(p.K, p.ldb)[:, : p.N].astype(np.int64).T  # row-major B
    rng = np.random.default_rng([5, 99])
    for _ in range(3):
        x = rng.integers(-1024, 1024, p.N).astype(np.int64)
        # |B x| < 2^30 and |A (B x)| < 2^50: exact in int64
        want = A @ (Bt.T @ x)
        lhs = got @ x
        bad = np.nonzero(lhs != want)[0]
        assert bad.size == 0, f"D x != A (B x) in {bad.size} rows, first {bad[:8]}"
