"""dmu_gemm_streamk_noalloc (the stream-K schedule on the library's own scratch, no allocation)
against dmu_gemm_streamk with a caller-owned workspace, through the C ABI: the same kernels
on the same workspace layout, so the outputs must agree bit for bit, and both meet the
oracle's bar.  Two calls in a row on the shared scratch, the second with a smaller problem
(so stale partial sums or flags of the first would show), then a third with the first again."""
import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_noalloc(p):
    import torch

    dA, dB = gu.to_dev(p.A), gu.to_dev(p.B)
    dC = gu.to_dev(p.C) if p.C is not None else None
    dD = torch.zeros(max(p.batch * p.stride_d, 1), dtype=gu.out_dtype(p.out_type), device="cuda:0")
    args = gu.make_args(p, dA, dB, dD, dC)
    assert dmu.dmu_gemm_streamk_workspace_size(args) > 0, "the problem must take the stream-K schedule"
    dmu.dmu_gemm_streamk_noalloc(args, None)
    torch.cuda.synchronize()
    assert dmu.dmu_gemm_streamk_error(None, check=False) is False
    return gu.from_dev(dD, p.out_type)[: p.batch * p.stride_d]


def problems():
    big = workloads.make("c1", "random", 31, M=256, N=256, K=8192)   # 4 tiles, each split over 64 workers
    big.C = None
    small = workloads.make("c3", "random", 32, M=700, N=500, K=1030)  # fp16 -> fp16, masked K tail
    return big, small


def test_noalloc_matches_workspace_entry_point_twice():
    big, small = problems()
    for p in (big, small, big):
        got = run_noalloc(p)
        ref, name, ws = gu.run_streamk(p)
        assert "generic" not in name
        gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))
        gu.assert_close(got, gu.run_oracle(p), p, where=gu.valid_mask(p))


def test_noalloc_with_epilogue_and_batches():
    p = workloads.make("c4s", "random", 33, M=300, N=136, K=1024, batch=3, with_c=True)
    ep = workloads.make_epilogue(p, 7, act="relu")
    import torch

    dA, dB, dC = gu.to_dev(p.A), gu.to_dev(p.B), gu.to_dev(p.C)
    keep = [gu.to_dev(x) for x in (ep.row_scale, ep.col_scale, ep.bias)]
    e = dmu.epilogue_args(row_scale=keep[0], stride_row_scale=ep.stride_rs, col_scale=keep[1],
                          stride_col_scale=ep.stride_cs, bias=keep[2], stride_bias=ep.stride_bias, act=ep.act)
    dD = torch.zeros(p.batch * p.stride_d, dtype=gu.out_dtype(p.out_type), device="cuda:0")
    args = gu.make_args(p, dA, dB, dD, dC)
    assert dmu.dmu_gemm_streamk_workspace_size(args) > 0
    dmu.dmu_gemm_streamk_noalloc(args, e)
    torch.cuda.synchronize()
    got = gu.from_dev(dD, p.out_type)[: p.batch * p.stride_d]
    ref, _, _ = gu.run_streamk(p, ep=ep)
    gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))


def test_noalloc_data_parallel_choice_and_empty():
    """Problems the schedule leaves to the data-parallel kernel need no scratch and match dmu_gemm;
    an empty problem launches nothing."""
    import torch

    p = workloads.make("c2", "random", 34, M=1024, N=1024, K=256)  # 64 tiles of 128 x 128 (128 of 64 x 128), 4 K-tiles
    dA, dB = gu.to_dev(p.A), gu.to_dev(p.B)
    dD = torch.zeros(p.stride_d, dtype=gu.out_dtype(p.out_type), device="cuda:0")
    args = gu.make_args(p, dA, dB, dD)
    dmu.dmu_gemm_streamk_noalloc(args, None)
    torch.cuda.synchronize()
    got = gu.from_dev(dD, p.out_type)[: p.stride_d]
    if dmu.dmu_gemm_streamk_workspace_size(args) == 0:
        gu.assert_bits_equal(got, gu.run_dmu(p), where=gu.valid_mask(p))
    else:
        ref, _, _ = gu.run_streamk(p)
        gu.assert_bits_equal(got, ref, where=gu.valid_mask(p))
    args.M = 0
    assert dmu.dmu_gemm_streamk_noalloc(args, None) == dmu.DMU_OK
