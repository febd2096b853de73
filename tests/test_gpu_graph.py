"""Entry points recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Callers that capture their launches record the library's kernels once and replay them with the
same pointers and fresh data.  For each entry point -- dmu_gemm on the data-parallel tiles and
in its persistent form, dmu_gemm_ex with the fused epilogue, dmu_gemm_streamk with a caller
workspace, dmu_gemm_streamk_noalloc on the library's scratch, and dmu_attention -- the call is
made once eagerly (set-up), captured, and the graph replayed four times; before each replay the
inputs are overwritten with new values and the output with a fill pattern by ordinary eager
work, and after it the replayed output must equal, bit for bit, that of an eager call on the
same inputs (which the other GPU tests hold against the oracle), and must differ from the
previous replay's (the replay recomputed rather than left old results).  The library records no
memset node: the stream-K scratch and flags are cleared by a kernel.
"""
import pytest

import dense_matrix_unit_tiled_amd as dmu
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t):
    import torch

    return t.view(torch.int32) if t.dtype == torch.float32 else t


def check_replays(launch, inputs, fresh, out):
    """launch(): the call under test (writes ``out``); inputs: device tensors the call reads;
    fresh(r): new contents for each of them."""
    import torch

    launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    prev = None
    for r in range(REPLAYS):
        for t, v in zip(inputs, fresh(r)):
            t.copy_(v)
        _bits(out).fill_(0x5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _bits(out).fill_(-1)
        launch()
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(out)), f"replay {r} differs from the eager call"
        if prev is not None:
            assert not torch.equal(_bits(got), _bits(prev)), f"replay {r} left the previous output"
        prev = got


def gemm_case(cfg, seed, with_c=False, **shape):
    """A seeded problem on the device: (args, [dA, dB, (dC)], fresh, dD)."""
    import torch

    p = workloads.make(cfg, "random", seed, with_c=with_c, **shape)
    dA, dB = gu.to_dev(p.A), gu.to_dev(p.B)
    dC = gu.to_dev(p.C) if p.C is not None else None
    dD = torch.zeros(max(p.batch * p.stride_d, 1), dtype=gu.out_dtype(p.out_type), device="cuda:0")
    args = gu.make_args(p, dA, dB, dD, dC)
    inputs = [dA, dB] + ([dC] if dC is not None else [])

    def fresh(r):
        q = workloads.make(cfg, "random", seed + 100 + r, with_c=with_c, **shape)
        return [gu.to_dev(q.A), gu.to_dev(q.B)] + ([gu.to_dev(q.C)] if dC is not None else [])

    return p, args, inputs, fresh, dD


@pytest.mark.parametrize("cfg,shape,kernel", [
    ("c2", dict(M=4096, N=4096, K=256), "256x256"),
    ("c3", dict(M=700, N=500, K=1030), "64x128"),
    ("c5", dict(M=1536, N=1536, K=512), "128x128"),
    ("c1", dict(M=300, N=270, K=130), "generic"),
])
def test_gemm_replays(cfg, shape, kernel):
    p, args, inputs, fresh, dD = gemm_case(cfg, 1, with_c=cfg != "c5", **shape)
    assert kernel in dmu.dmu_gemm_kernel_name(args)
    check_replays(lambda: dmu.dmu_gemm(args), inputs, fresh, dD)


def test_persistent_form_replays(monkeypatch):
    monkeypatch.setenv("DMU_PERSIST", "always")
    p, args, inputs, fresh, dD = gemm_case("c2", 2, M=2048, N=2048, K=512)
    check_replays(lambda: dmu.dmu_gemm(args), inputs, fresh, dD)


def test_epilogue_replays():
    p, args, inputs, fresh, dD = gemm_case("c5", 3, M=1024, N=768, K=512)
    p = workloads.with_output(p, "bf16", 3)
    import torch

    dD = torch.zeros(max(p.batch * p.stride_d, 1), dtype=gu.out_dtype(p.out_type), device="cuda:0")
    args = gu.make_args(p, inputs[0], inputs[1], dD)
    ep = workloads.make_epilogue(p, 4, act="gelu_tanh")
    keep = [gu.to_dev(ep.row_scale), gu.to_dev(ep.col_scale), gu.to_dev(ep.bias)]
    e = dmu.epilogue_args(row_scale=keep[0], stride_row_scale=ep.stride_rs, col_scale=keep[1],
                          stride_col_scale=ep.stride_cs, bias=keep[2], stride_bias=ep.stride_bias, act=ep.act)
    check_replays(lambda: dmu.dmu_gemm_ex(args, e), inputs, fresh, dD)


def test_streamk_workspace_replays():
    import torch

    p, args, inputs, fresh, dD = gemm_case("c1", 5, M=512, N=512, K=8192)
    nbytes = dmu.dmu_gemm_streamk_workspace_size(args)
    assert nbytes > 0, "the problem must take the stream-K schedule"
    ws = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device="cuda:0")
    check_replays(lambda: dmu.dmu_gemm_streamk(args, None, ws, 4 * ws.numel()), inputs, fresh, dD)
    assert not dmu.dmu_gemm_streamk_error(ws, check=False)


def test_streamk_noalloc_replays():
    p, args, inputs, fresh, dD = gemm_case("c3", 6, M=700, N=500, K=8200)
    assert dmu.dmu_gemm_streamk_workspace_size(args) > 0, "the problem must take the stream-K schedule"
    check_replays(lambda: dmu.dmu_gemm_streamk_noalloc(args, None), inputs, fresh, dD)
    assert dmu.dmu_gemm_streamk_error(None, check=False) is False


@pytest.mark.parametrize("in_t,out_t", [("f16", "f32"), ("bf16", "bf16")])
def test_attention_replays(in_t, out_t):
    import torch

    B, S, D = 2, 700, 128
    dt = torch.float16 if in_t == "f16" else torch.bfloat16
    gen = torch.Generator(device="cuda:0").manual_seed(7)
    q, k, v = (torch.rand(B * S * D, device="cuda:0", generator=gen).to(dt) for _ in range(3))
    o = torch.zeros(B * S * D, device="cuda:0", dtype=torch.float32 if out_t == "f32" else torch.int16)
    a = dmu.attention_args(B, S, S, D, q, D, k, D, v, D, o, D, in_type=in_t, out_type=out_t, scale=D ** -0.5,
                           stride_q=S * D, stride_k=S * D, stride_v=S * D, stride_o=S * D)

    def fresh(r):
        g = torch.Generator(device="cuda:0").manual_seed(100 + r)
        return [(torch.rand(B * S * D, device="cuda:0", generator=g) * 2 - 1).to(dt) for _ in range(3)]

    check_replays(lambda: dmu.dmu_attention(a), [q, k, v], fresh, o)
