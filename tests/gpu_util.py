"""Helpers of the GPU tests: move seeded workloads to the device, call the HIP
library through its C ABI, and compare with the oracle to the stated bar.

Tolerances (floating point, random inputs):
  fp32 output:       |D - ref| <= 1e-3 * sqrt(K) * max|A| * max|B|
  fp16/bf16 output:  |D - ref| <= 2e-2 * |ref| + 1e-3 * sqrt(K) * max|A| * max|B|
The first is the bound ``1e-3 * sqrt(K)`` for inputs in [-1, 1] rescaled to the
inputs' actual range (never looser than that bound); the second adds the
relative 2e-2 allowance for a 16-bit output.  Integer-valued inputs whose sums
are exact in fp32, and int8, must match bit for bit.
"""
from __future__ import annotations

import math
import os

import numpy as np

import dense_matrix_unit_tiled_amd as dmu
import oracle
from tests import exact
from workloads import to_bits as workloads_to_bits  # noqa: F401

_TORCH_DT = None


def _torch():
    import torch

    return torch


def to_dev(arr: np.ndarray):
    """Raw element bits on cuda:0 (uint16 patterns travel as int16)."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def out_dtype(t: str):
    torch = _torch()
    return {"f32": torch.float32, "f16": torch.int16, "bf16": torch.int16, "i32": torch.int32}[t]


def from_dev(t, out_t: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if out_t in ("f16", "bf16") else a


def make_args(p, dA, dB, dD, dC=None):
    return dmu.gemm_args(p.M, p.N, p.K, dA, p.lda, dB, p.ldb, dD, p.ldd, in_type=p.in_type,
                         out_type=p.out_type, acc_type=p.acc_type, layout_a=p.layout_a,
                         layout_b=p.layout_b, batch=p.batch, stride_a=p.stride_a,
                         stride_b=p.stride_b, C=dC, ldc=p.ldc, stride_c=p.stride_c,
                         stride_d=p.stride_d)


class force_kernel:
    """Context manager selecting a kernel family through DMU_FORCE_KERNEL."""

    def __init__(self, name):
        self.name = name

    def __enter__(self):
        self.old = os.environ.get("DMU_FORCE_KERNEL")
        if self.name is None:
            os.environ.pop("DMU_FORCE_KERNEL", None)
        else:
            os.environ["DMU_FORCE_KERNEL"] = self.name

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("DMU_FORCE_KERNEL", None)
        else:
            os.environ["DMU_FORCE_KERNEL"] = self.old


def run_dmu(p, force=None, fill=None, return_name=False, ep=None, in_place=False):
    """Run one workload on the GPU through dmu_gemm (dmu_gemm_ex when an epilogue
    ``ep`` is given); D as raw bits (oracle format).

    fill: optional bit pattern written to D before the call (to see untouched cells).
    in_place: D starts as a copy of C and the call passes C == D.
    """
    torch = _torch()
    dA, dB = to_dev(p.A), to_dev(p.B)
    dC = to_dev(p.C) if p.C is not None else None
    n = max(p.batch * p.stride_d, 1)
    dD = torch.zeros(n, dtype=out_dtype(p.out_type), device="cuda:0")
    if fill is not None:
        dD.fill_(fill)
    if in_place:
        assert p.C is not None and p.ldc == p.ldd and p.stride_c == p.stride_d
        dD[: dC.numel()].copy_(dC)
        dC = dD
    args = make_args(p, dA, dB, dD, dC)
    keep = []
    with force_kernel(force):
        name = dmu.dmu_gemm_kernel_name(args)
        if ep is None:
            dmu.dmu_gemm(args)
        else:
            vec = lambda x: None if x is None else keep.append(to_dev(x)) or keep[-1]
            e = dmu.epilogue_args(row_scale=vec(ep.row_scale), stride_row_scale=ep.stride_rs,
                                  col_scale=vec(ep.col_scale), stride_col_scale=ep.stride_cs,
                                  bias=vec(ep.bias), stride_bias=ep.stride_bias, act=ep.act)
            dmu.dmu_gemm_ex(args, e)
    torch.cuda.synchronize()
    out = from_dev(dD, p.out_type)[: p.batch * p.stride_d]
    return (out, name) if return_name else out


def run_streamk(p, ep=None, workspace=None, calls=1, check_error=True):
    """Run one workload through dmu_gemm_streamk (``calls`` times with the same
    workspace); returns (D bits, kernel name, workspace tensor or None).  With
    ``check_error`` the workspace's error word (dmu_gemm_streamk_error) must be clear."""
    torch = _torch()
    dA, dB = to_dev(p.A), to_dev(p.B)
    dC = to_dev(p.C) if p.C is not None else None
    dD = torch.zeros(max(p.batch * p.stride_d, 1), dtype=out_dtype(p.out_type), device="cuda:0")
    args = make_args(p, dA, dB, dD, dC)
    nbytes = dmu.dmu_gemm_streamk_workspace_size(args)
    if workspace is None and nbytes:
        workspace = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device="cuda:0")
    keep = []
    e = None
    if ep is not None:
        vec = lambda x: None if x is None else keep.append(to_dev(x)) or keep[-1]
        e = dmu.epilogue_args(row_scale=vec(ep.row_scale), stride_row_scale=ep.stride_rs,
                              col_scale=vec(ep.col_scale), stride_col_scale=ep.stride_cs,
                              bias=vec(ep.bias), stride_bias=ep.stride_bias, act=ep.act)
    for _ in range(calls):
        dmu.dmu_gemm_streamk(args, e, workspace, 4 * workspace.numel() if workspace is not None else 0)
    torch.cuda.synchronize()
    if workspace is not None and check_error:
        assert not dmu.dmu_gemm_streamk_error(workspace, check=False), "a stream-K wait gave up"
    return from_dev(dD, p.out_type)[: p.batch * p.stride_d], dmu.dmu_gemm_kernel_name(args), workspace


def run_oracle(p, nthreads=None, ep=None):
    return oracle.gemm(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, in_type=p.in_type,
                       out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                       batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, C=p.C,
                       ldc=p.ldc, stride_c=p.stride_c, ldd=p.ldd, stride_d=p.stride_d,
                       nthreads=nthreads, **(ep.kwargs() if ep is not None else {}))


def oracle_at(p, bij, ep=None):
    return oracle.gemm_at(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, bij, in_type=p.in_type,
                          out_type=p.out_type, layout_a=p.layout_a, layout_b=p.layout_b,
                          batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b, C=p.C,
                          ldc=p.ldc, stride_c=p.stride_c, **(ep.kwargs() if ep is not None else {}))


def product_at(p, bij):
    """|P| (the plain product, no C, no epilogue) at (b, i, j), from the oracle in fp64 terms."""
    q_out = "f32"
    return np.abs(oracle.gemm_at(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, bij, in_type=p.in_type,
                                 out_type=q_out, layout_a=p.layout_a, layout_b=p.layout_b,
                                 batch=p.batch, stride_a=p.stride_a, stride_b=p.stride_b).astype(np.float64))


def assert_close_epilogue(got: np.ndarray, want: np.ndarray, p, ep, bij: np.ndarray):
    """The parity bar with a fused epilogue, at the elements (b, i, j) of ``bij`` (got/want
    hold those elements).  The product's bound moves through the scales, the epilogue's
    fp32 steps add a relative 1e-5 of the magnitudes summed, the activation is at most
    1.2-Lipschitz, and a 16-bit output adds its 2e-2 relative allowance:
      |D - ref| <= 1.2 (e_P |rs_i cs_j| + 1e-5 (|rs_i cs_j P_ij| + |bias_j| + |C_ij|)) [+ 2e-2 |ref|]
    with e_P = 1e-3 sqrt(K) max|A| max|B| for fp16/bf16 inputs and 0 for int8 (exact sums)."""
    b, i, j = bij[:, 0], bij[:, 1], bij[:, 2]
    rs = ep.row_scale[b * ep.stride_rs + i].astype(np.float64) if ep.row_scale is not None else 1.0
    cs = ep.col_scale[b * ep.stride_cs + j].astype(np.float64) if ep.col_scale is not None else 1.0
    bias = np.abs(ep.bias[b * ep.stride_bias + j].astype(np.float64)) if ep.bias is not None else 0.0
    cmag = np.abs(values(p.C[b * p.stride_c + i * p.ldc + j], p.out_type)) if p.C is not None else 0.0
    P = product_at(p, bij)
    if p.in_type == "i8":
        e_p = 0.0
    else:
        amax, bmax = input_absmax(p)
        e_p = 1e-3 * math.sqrt(max(p.K, 1)) * amax * bmax
    s = np.abs(rs * cs)
    tol = 1.2 * (e_p * s + 1e-5 * (s * P + bias + cmag)) + 1e-30
    g, w = values(got, p.out_type), values(want, p.out_type)
    if p.out_type != "f32":
        tol = tol + 2e-2 * np.abs(w)
    err = np.abs(g - w)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{bad.size}/{g.size} outside tolerance; first {bad[:5]} at {bij[bad[:5]].tolist()}: "
                           f"got {g[bad[:5]]} want {w[bad[:5]]} tol {np.broadcast_to(tol, g.shape)[bad[:5]]}")


def all_bij(p) -> np.ndarray:
    """Every (b, i, j) of the product, in the order of the flat D buffer's valid cells."""
    b, i, j = np.meshgrid(np.arange(p.batch), np.arange(p.M), np.arange(p.N), indexing="ij")
    return np.stack([b.ravel(), i.ravel(), j.ravel()], axis=1).astype(np.int64)


def values(bits: np.ndarray, t: str) -> np.ndarray:
    if t == "e4m3":
        return exact.e4m3_values(bits)
    if t == "f16":
        return exact.f16_values(bits)
    if t == "bf16":
        return exact.bf16_values(bits)
    return np.asarray(bits, dtype=np.float64)


def input_absmax(p) -> tuple[float, float]:
    if p.in_type == "i8":
        return 128.0, 128.0
    return float(np.nanmax(np.abs(values(p.A, p.in_type)))), float(np.nanmax(np.abs(values(p.B, p.in_type))))


def valid_mask(p) -> np.ndarray:
    """Elements of the flat D buffer that are part of the product (not ld padding)."""
    m = np.zeros(max(p.batch * p.stride_d, 1), dtype=bool)
    for b in range(p.batch):
        base = b * p.stride_d
        v = m[base: base + p.M * p.ldd].reshape(p.M, p.ldd)
        v[:, : p.N] = True
    return m[: p.batch * p.stride_d]


def assert_close(got: np.ndarray, want: np.ndarray, p, where=None):
    """The parity bar for one workload (see the module docstring)."""
    if where is not None:
        got, want = got[where], want[where]
    if p.out_type == "i32":
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} int32 mismatches, first at {bad[:5]}: {got[bad[:5]]} vs {want[bad[:5]]}"
        return
    g, w = values(got, p.out_type), values(want, p.out_type)
    amax, bmax = input_absmax(p)
    floor = 1e-3 * math.sqrt(max(p.K, 1)) * amax * bmax
    tol = floor if p.out_type == "f32" else 2e-2 * np.abs(w) + floor
    err = np.abs(g - w)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{bad.size}/{g.size} outside tolerance; worst err {np.nanmax(err):.3e} "
                           f"(floor {floor:.3e}); first {bad[:5]}: got {g[bad[:5]]} want {w[bad[:5]]}")


def assert_bits_equal(got: np.ndarray, want: np.ndarray, where=None):
    if where is not None:
        got, want = got[where], want[where]
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{bad.size} bit mismatches, first at {bad[:8]}: {got[bad[:8]]} vs {want[bad[:8]]}"


def sample_bij(p, n=512, seed=0) -> np.ndarray:
    """Sampled (b, i, j) covering the corners, tile edges and random interior points."""
    rng = np.random.default_rng(seed)
    pts = set()
    for b in {0, p.batch - 1}:
        for i in {0, p.M - 1, min(p.M - 1, 255), min(p.M - 1, 256), min(p.M - 1, 127)}:
            for j in {0, p.N - 1, min(p.N - 1, 255), min(p.N - 1, 256), min(p.N - 1, 31)}:
                pts.add((b, i, j))
    while len(pts) < n:
        pts.add((int(rng.integers(0, p.batch)), int(rng.integers(0, p.M)), int(rng.integers(0, p.N))))
    return np.array(sorted(pts), dtype=np.int64)


def flat_index(p, bij: np.ndarray) -> np.ndarray:
    return bij[:, 0] * p.stride_d + bij[:, 1] * p.ldd + bij[:, 2]
