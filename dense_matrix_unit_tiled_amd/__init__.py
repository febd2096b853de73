"""Python binding of ``libdmu.so`` (the gfx950 GEMM library, C ABI in include/dmu.h).

Argument marshalling only: every step of the product runs in the library's HIP
kernels.  The functions keep the C names (``dmu_gemm``, ``dmu_gemm_check``,
``dmu_gemm_ex``, ``dmu_gemm_ex_check``, ``dmu_attention``, ``dmu_attention_check``,
``dmu_gemm_streamk``, ``dmu_gemm_streamk_workspace_size``, ``dmu_gemm_streamk_error``,
``dmu_gemm_streamk_noalloc``,
``dmu_gemm_kernel_name``,
``dmu_device_info``, ``dmu_status_string``, ``dmu_last_error``, ``dmu_probe``, ``dmu_probe_info``);
``gemm_args`` and ``epilogue_args`` fill the argument structs from torch tensors
(or raw integer device addresses).  PyTorch supplies device
memory and streams only.

If ``libdmu.so`` has not been built, the first call raises ``RuntimeError``:
there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# The library this binding loads: the in-tree build, or another build of the same sources named by
# the environment variable DMU_LIBRARY (the LDS-poisoning debug build, a build kept for comparison).
LIB_PATH = os.environ.get("DMU_LIBRARY") or os.path.join(HERE, "libdmu.so")

DMU_F16, DMU_BF16, DMU_F32, DMU_I8, DMU_I32, DMU_E4M3 = 1, 2, 3, 4, 5, 6
DMU_ROW_MAJOR, DMU_COL_MAJOR = 0, 1
DMU_OK, DMU_ERR_INVALID_ARG, DMU_ERR_UNSUPPORTED, DMU_ERR_HIP = 0, -1, -2, -3

DMU_PROBE_MFMA_32x32x16_BF16 = 1
DMU_PROBE_MFMA_32x32x16_F16 = 2
DMU_PROBE_MFMA_16x16x32_BF16 = 3
DMU_PROBE_MFMA_16x16x32_F16 = 4
DMU_PROBE_MFMA_32x32x32_I8 = 5
DMU_PROBE_MFMA_16x16x64_I8 = 6
DMU_PROBE_MFMA_16x16x128_E4M3 = 7
DMU_PROBE_LDS_READ_B128 = 10
DMU_PROBE_LDS_READ_TR16 = 11
DMU_PROBE_LDS_FRAG = 12
DMU_PROBE_LDS_FRAG_T = 13
DMU_PROBE_LANE_SWAP = 14
DMU_PROBE_LDS_READ_TR8 = 15
DMU_PROBE_CVT_BF16 = 30
DMU_PROBE_CVT_F16 = 31

DTYPES = {"f16": DMU_F16, "bf16": DMU_BF16, "f32": DMU_F32, "i8": DMU_I8, "i32": DMU_I32, "e4m3": DMU_E4M3}
LAYOUTS = {"row": DMU_ROW_MAJOR, "col": DMU_COL_MAJOR}


class dmu_gemm_args(ctypes.Structure):
    """Mirror of ``struct dmu_gemm_args`` (include/dmu.h)."""

    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("batch", ctypes.c_int64),
        ("in_type", ctypes.c_int32), ("acc_type", ctypes.c_int32), ("out_type", ctypes.c_int32),
        ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("stride_a", ctypes.c_int64),
        ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("stride_c", ctypes.c_int64),
        ("D", ctypes.c_void_p), ("ldd", ctypes.c_int64), ("stride_d", ctypes.c_int64),
    ]


DMU_ACT_NONE, DMU_ACT_RELU, DMU_ACT_GELU_TANH = 0, 1, 2
ACTS = {"none": DMU_ACT_NONE, "relu": DMU_ACT_RELU, "gelu_tanh": DMU_ACT_GELU_TANH}


class dmu_epilogue(ctypes.Structure):
    """Mirror of ``struct dmu_epilogue`` (include/dmu.h)."""

    _fields_ = [
        ("row_scale", ctypes.c_void_p), ("stride_row_scale", ctypes.c_int64),
        ("col_scale", ctypes.c_void_p), ("stride_col_scale", ctypes.c_int64),
        ("bias", ctypes.c_void_p), ("stride_bias", ctypes.c_int64),
        ("act", ctypes.c_int32),
    ]


class dmu_attention_args(ctypes.Structure):
    """Mirror of ``struct dmu_attention_args`` (include/dmu.h)."""

    _fields_ = [
        ("batch", ctypes.c_int64), ("seq_q", ctypes.c_int64), ("seq_k", ctypes.c_int64),
        ("head_dim", ctypes.c_int64), ("in_type", ctypes.c_int32), ("out_type", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("Q", ctypes.c_void_p), ("ldq", ctypes.c_int64), ("stride_q", ctypes.c_int64),
        ("K", ctypes.c_void_p), ("ldk", ctypes.c_int64), ("stride_k", ctypes.c_int64),
        ("V", ctypes.c_void_p), ("ldv", ctypes.c_int64), ("stride_v", ctypes.c_int64),
        ("O", ctypes.c_void_p), ("ldo", ctypes.c_int64), ("stride_o", ctypes.c_int64),
    ]


class DmuError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{dmu_status_string(status)}: {detail}")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with dense_matrix_unit_tiled_amd.build.build()")
    # PyTorch ships its own HIP runtime.  Importing it first makes the library's
    # libamdhip64 dependency resolve to that already-loaded copy, so the process
    # holds one HIP runtime and torch's device pointers and streams are valid here.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(dmu_gemm_args)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.dmu_gemm.argtypes, lib.dmu_gemm.restype = [P, vp], i32
    lib.dmu_gemm_check.argtypes, lib.dmu_gemm_check.restype = [P], i32
    PA = ctypes.POINTER(dmu_attention_args)
    lib.dmu_attention.argtypes, lib.dmu_attention.restype = [PA, vp], i32
    lib.dmu_attention_check.argtypes, lib.dmu_attention_check.restype = [PA], i32
    PE = ctypes.POINTER(dmu_epilogue)
    lib.dmu_gemm_ex.argtypes, lib.dmu_gemm_ex.restype = [P, PE, vp], i32
    lib.dmu_gemm_ex_check.argtypes, lib.dmu_gemm_ex_check.restype = [P, PE], i32
    lib.dmu_gemm_streamk.argtypes, lib.dmu_gemm_streamk.restype = [P, PE, vp, ctypes.c_size_t, vp], i32
    lib.dmu_gemm_streamk_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.dmu_gemm_streamk_workspace_size.restype = i32
    lib.dmu_gemm_streamk_noalloc.argtypes, lib.dmu_gemm_streamk_noalloc.restype = [P, PE, vp], i32
    lib.dmu_gemm_streamk_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int)]
    lib.dmu_gemm_streamk_error.restype = i32
    lib.dmu_gemm_kernel_name.argtypes, lib.dmu_gemm_kernel_name.restype = [P], ctypes.c_char_p
    lib.dmu_device_info.argtypes = [i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.dmu_device_info.restype = i32
    lib.dmu_status_string.argtypes, lib.dmu_status_string.restype = [i32], ctypes.c_char_p
    lib.dmu_last_error.argtypes, lib.dmu_last_error.restype = [], ctypes.c_char_p
    lib.dmu_mfma_ceiling.argtypes, lib.dmu_mfma_ceiling.restype = [i32, i32, i32, vp, vp], i32
    lib.dmu_phase_log.argtypes, lib.dmu_phase_log.restype = [vp, ctypes.c_size_t], i32
    lib.dmu_phase_log_last.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int)]
    lib.dmu_phase_log_last.restype = i32
    lib.dmu_probe.argtypes, lib.dmu_probe.restype = [i32, vp, vp, vp, vp], i32
    ip = ctypes.POINTER(ctypes.c_int)
    lib.dmu_probe_info.argtypes, lib.dmu_probe_info.restype = [i32, ip, ip, ip, ip, ip], i32
    return lib


@contextlib.contextmanager
def library_override(path):
    """Route every call of this binding to another build of the library (for example the
    LDS-poisoning debug build) for the duration of a ``with`` block."""
    global _lib
    saved = _load()
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = saved


def library():
    """The loaded ctypes library (raises RuntimeError when it is not built)."""
    return _load()


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_args(M, N, K, A, lda, B, ldb, D, ldd, *, in_type, out_type, acc_type=None,
              layout_a="row", layout_b="row", batch=1, stride_a=0, stride_b=0, C=None, ldc=0,
              stride_c=0, stride_d=0) -> dmu_gemm_args:
    """Fill a dmu_gemm_args from tensors/addresses and type/layout names."""
    if acc_type is None:
        acc_type = "i32" if in_type == "i8" else "f32"
    a = dmu_gemm_args()
    a.M, a.N, a.K, a.batch = M, N, K, batch
    a.in_type, a.acc_type, a.out_type = DTYPES[in_type], DTYPES[acc_type], DTYPES[out_type]
    a.layout_a, a.layout_b = LAYOUTS[layout_a], LAYOUTS[layout_b]
    a.A, a.lda, a.stride_a = _addr(A), lda, stride_a
    a.B, a.ldb, a.stride_b = _addr(B), ldb, stride_b
    a.C, a.ldc, a.stride_c = _addr(C), ldc, stride_c
    a.D, a.ldd, a.stride_d = _addr(D), ldd, stride_d
    return a


def dmu_gemm(args: dmu_gemm_args, stream=None, check: bool = True) -> int:
    """Launch D = A*B + C on ``stream`` (default: torch's current stream)."""
    st = _load().dmu_gemm(ctypes.byref(args), _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def epilogue_args(row_scale=None, stride_row_scale=0, col_scale=None, stride_col_scale=0, bias=None,
                  stride_bias=0, act="none") -> dmu_epilogue:
    """Fill a dmu_epilogue from float32 tensors/addresses and an activation name."""
    e = dmu_epilogue()
    e.row_scale, e.stride_row_scale = _addr(row_scale), stride_row_scale
    e.col_scale, e.stride_col_scale = _addr(col_scale), stride_col_scale
    e.bias, e.stride_bias = _addr(bias), stride_bias
    e.act = ACTS[act] if isinstance(act, str) else act
    return e


def dmu_gemm_ex(args: dmu_gemm_args, ep: dmu_epilogue | None, stream=None, check: bool = True) -> int:
    """Launch D = epilogue(A*B + C) on ``stream`` (default: torch's current stream)."""
    st = _load().dmu_gemm_ex(ctypes.byref(args), None if ep is None else ctypes.byref(ep), _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def dmu_gemm_ex_check(args: dmu_gemm_args, ep: dmu_epilogue | None) -> int:
    return _load().dmu_gemm_ex_check(ctypes.byref(args), None if ep is None else ctypes.byref(ep))


def dmu_gemm_streamk_workspace_size(args: dmu_gemm_args) -> int:
    """Workspace bytes dmu_gemm_streamk needs on the current device (0: none)."""
    n = ctypes.c_size_t(0)
    st = _load().dmu_gemm_streamk_workspace_size(ctypes.byref(args), ctypes.byref(n))
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return n.value


def dmu_gemm_streamk(args: dmu_gemm_args, ep: dmu_epilogue | None, workspace, workspace_bytes: int,
                     stream=None, check: bool = True) -> int:
    """Launch the stream-K schedule of D = epilogue(A*B + C) with a caller-owned, zero-filled workspace."""
    st = _load().dmu_gemm_streamk(ctypes.byref(args), None if ep is None else ctypes.byref(ep), _addr(workspace),
                                  workspace_bytes, _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


# Bytes of the scratch array the library holds on each GPU for dmu_gemm_streamk_noalloc.
DMU_STREAMK_SCRATCH_BYTES = 33 * 1024 * 1024


def dmu_gemm_streamk_noalloc(args: dmu_gemm_args, ep: dmu_epilogue | None, stream=None, check: bool = True) -> int:
    """The stream-K schedule of D = epilogue(A*B + C) on the library's own scratch (no workspace,
    no allocation; calls that overlap in time on one GPU race)."""
    st = _load().dmu_gemm_streamk_noalloc(ctypes.byref(args), None if ep is None else ctypes.byref(ep),
                                          _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def dmu_gemm_streamk_error(workspace, stream=None, check: bool = True) -> bool:
    """Whether a wait inside an earlier dmu_gemm_streamk call on ``workspace`` gave up (that
    call's D is then wrong, and the workspace must be zero-filled again); ``workspace`` None
    asks about the last dmu_gemm_streamk_noalloc call on the current device.  Waits for
    ``stream``.  With ``check`` a failed wait raises DmuError."""
    failed = ctypes.c_int(0)
    st = _load().dmu_gemm_streamk_error(_addr(workspace), _stream(stream), ctypes.byref(failed))
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    if check and failed.value:
        raise DmuError(DMU_ERR_HIP, "a stream-K wait ran past its limit: D is wrong; zero-fill the workspace")
    return bool(failed.value)


def attention_args(batch, seq_q, seq_k, head_dim, Q, ldq, K, ldk, V, ldv, O, ldo, *, in_type, out_type, scale,
                   stride_q=0, stride_k=0, stride_v=0, stride_o=0) -> dmu_attention_args:
    """Fill a dmu_attention_args from tensors/addresses and type names."""
    a = dmu_attention_args()
    a.batch, a.seq_q, a.seq_k, a.head_dim = batch, seq_q, seq_k, head_dim
    a.in_type, a.out_type, a.scale = DTYPES[in_type], DTYPES[out_type], scale
    a.Q, a.ldq, a.stride_q = _addr(Q), ldq, stride_q
    a.K, a.ldk, a.stride_k = _addr(K), ldk, stride_k
    a.V, a.ldv, a.stride_v = _addr(V), ldv, stride_v
    a.O, a.ldo, a.stride_o = _addr(O), ldo, stride_o
    return a


def dmu_attention(args: dmu_attention_args, stream=None, check: bool = True) -> int:
    """Launch O = softmax(scale Q K^T) V on ``stream`` (default: torch's current stream)."""
    st = _load().dmu_attention(ctypes.byref(args), _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def dmu_attention_check(args: dmu_attention_args) -> int:
    return _load().dmu_attention_check(ctypes.byref(args))


def dmu_gemm_check(args: dmu_gemm_args) -> int:
    return _load().dmu_gemm_check(ctypes.byref(args))


def dmu_gemm_kernel_name(args: dmu_gemm_args) -> str | None:
    r = _load().dmu_gemm_kernel_name(ctypes.byref(args))
    return None if r is None else r.decode()


def dmu_device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) of a HIP device; raises DmuError on failure."""
    cu, khz = ctypes.c_int(), ctypes.c_int()
    st = _load().dmu_device_info(device, ctypes.byref(cu), ctypes.byref(khz))
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return cu.value, khz.value


def dmu_mfma_ceiling(in_type: str, rounds: int, workgroups: int, stamps=None, stream=None, check: bool = True) -> int:
    """Launch the matrix-core ceiling microbenchmark (register-only MFMA chains on a grid shaped
    like the tiled kernels'); the caller times it.  ``stamps``: None or a device buffer of
    workgroups x 4 uint64."""
    st = _load().dmu_mfma_ceiling(DTYPES[in_type], rounds, workgroups, _addr(stamps), _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def dmu_phase_log(log, records: int) -> None:
    """Point every following GEMM or attention launch of the process at a phase log: a device buffer of
    ``records`` x 8 uint64 (tensor or address), or None and 0 to turn it off.  Raises DmuError."""
    st = _load().dmu_phase_log(_addr(log), records)
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())


def dmu_phase_log_last():
    """(records, kind) of the last launch's phase log; kind 0 none, 1 one record per
    workgroup, 2 one per tile of the persistent kernel, 3 one per stream-K worker, 4 one per
    workgroup of the attention kernel."""
    n, kind = ctypes.c_size_t(), ctypes.c_int()
    st = _load().dmu_phase_log_last(ctypes.byref(n), ctypes.byref(kind))
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return n.value, kind.value


def dmu_status_string(status: int) -> str:
    return _load().dmu_status_string(status).decode()


def dmu_last_error() -> str:
    return _load().dmu_last_error().decode()


def dmu_probe(variant: int, in0, in1, out, stream=None, check: bool = True) -> int:
    st = _load().dmu_probe(variant, _addr(in0), _addr(in1), _addr(out), _stream(stream))
    if check and st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return st


def dmu_probe_info(variant: int):
    """(m, n, k, in_type, regs_per_lane) of a probe variant."""
    v = [ctypes.c_int() for _ in range(5)]
    st = _load().dmu_probe_info(variant, *[ctypes.byref(x) for x in v])
    if st != DMU_OK:
        raise DmuError(st, dmu_last_error())
    return tuple(x.value for x in v)
