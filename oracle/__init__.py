"""CPU oracle for D = A*B + C (ctypes binding of ``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The GPU library and its
Python binding never import it, and it imports nothing from them.

Every function takes raw element bits (numpy ``uint16`` for fp16/bf16,
``int8``, ``float32``, ``int32``) and returns raw bits of the output type:
``float32`` for fp32, ``uint16`` for fp16/bf16, ``int32`` for int32.  See the
header of ``oracle.c`` for the computation and the passages it follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

TYPES = {"f16": 1, "bf16": 2, "f32": 3, "i8": 4, "i32": 5}
LAYOUTS = {"row": 0, "col": 1}
_NP_IN = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i8": np.int8, "i32": np.int32}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    common = [i64, i64, i64, i64, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, vp, i64, i64]
    lib.oracle_gemm.argtypes = common + [vp, i64, i64, i32]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm_at.argtypes = common + [i64, vp, vp]
    lib.oracle_gemm_at.restype = i32
    lib.oracle_decode_array.argtypes = [i32, vp, vp, i64]
    lib.oracle_decode_array.restype = None
    lib.oracle_encode_array.argtypes = [i32, vp, vp, i64]
    lib.oracle_encode_array.restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def _extent(layout: str, rows: int, cols: int, ld: int) -> int:
    """Elements spanned by a rows x cols matrix with leading dimension ld."""
    if rows == 0 or cols == 0:
        return 0
    if layout == "row":
        return (rows - 1) * ld + cols
    return (cols - 1) * ld + rows


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(x, t, need, name):
    if x is None:
        return None
    x = np.ascontiguousarray(x).reshape(-1)
    if x.dtype.itemsize != np.dtype(_NP_IN[t]).itemsize:
        raise TypeError(f"{name}: element size {x.dtype.itemsize} does not match {t}")
    if x.size < need:
        raise ValueError(f"{name}: buffer holds {x.size} elements, needs {need}")
    return x


def _common(M, N, K, A, lda, B, ldb, in_type, out_type, layout_a, layout_b, batch,
            stride_a, stride_b, C, ldc, stride_c):
    if in_type not in ("f16", "bf16", "f32", "i8"):
        raise ValueError(f"unsupported input type {in_type}")
    acc_t = "i32" if in_type == "i8" else out_type
    span = lambda s, e: 0 if batch == 0 or e == 0 else (batch - 1) * s + e
    A = _prep(A, in_type, span(stride_a, _extent(layout_a, M, K, lda)), "A")
    B = _prep(B, in_type, span(stride_b, _extent(layout_b, K, N, ldb)), "B")
    C = _prep(C, acc_t, span(stride_c, _extent("row", M, N, ldc)), "C")
    args = (M, N, K, batch, TYPES[in_type], TYPES[out_type], LAYOUTS[layout_a], LAYOUTS[layout_b],
            _ptr(A), lda, stride_a, _ptr(B), ldb, stride_b, _ptr(C), ldc, stride_c)
    return args, (A, B, C)


def gemm(M, N, K, A, lda, B, ldb, *, in_type, out_type, layout_a="row", layout_b="row",
         batch=1, stride_a=0, stride_b=0, C=None, ldc=0, stride_c=0, ldd=None, stride_d=None,
         nthreads=None):
    """Full D (flat, batch*stride_d elements; row-major M x N with leading dim ldd)."""
    ldd = N if ldd is None else ldd
    stride_d = M * ldd if stride_d is None else stride_d
    args, keep = _common(M, N, K, A, lda, B, ldb, in_type, out_type, layout_a, layout_b, batch,
                         stride_a, stride_b, C, ldc, stride_c)
    D = np.zeros(max(batch * stride_d, 1), dtype=_NP_IN[out_type])
    st = _load().oracle_gemm(*args, _ptr(D), ldd, stride_d, nthreads or default_threads())
    if st:
        raise ValueError(f"oracle_gemm rejected its arguments (code {st})")
    del keep
    return D[: batch * stride_d]


def gemm_at(M, N, K, A, lda, B, ldb, bij, *, in_type, out_type, layout_a="row",
            layout_b="row", batch=1, stride_a=0, stride_b=0, C=None, ldc=0, stride_c=0):
    """D[b](i,j) for each row (b, i, j) of the integer array ``bij`` (shape [n, 3])."""
    args, keep = _common(M, N, K, A, lda, B, ldb, in_type, out_type, layout_a, layout_b, batch,
                         stride_a, stride_b, C, ldc, stride_c)
    bij = np.ascontiguousarray(bij, dtype=np.int64).reshape(-1, 3)
    out = np.zeros(max(len(bij), 1), dtype=_NP_IN[out_type])
    st = _load().oracle_gemm_at(*args, len(bij), _ptr(bij), _ptr(out))
    if st:
        raise ValueError(f"oracle_gemm_at rejected its arguments (code {st})")
    del keep
    return out[: len(bij)]


def decode(t: str, bits) -> np.ndarray:
    """Exact fp64 values of fp16 or bf16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(bits.size, dtype=np.float64)
    _load().oracle_decode_array(TYPES[t], _ptr(bits), _ptr(out), bits.size)
    return out


def encode(t: str, values) -> np.ndarray:
    """Round fp64 values once (nearest, ties to even) to fp16/bf16 bits or fp32."""
    values = np.ascontiguousarray(values, dtype=np.float64).reshape(-1)
    out = np.empty(values.size, dtype=np.uint32 if t == "f32" else np.uint16)
    _load().oracle_encode_array(TYPES[t], _ptr(values), _ptr(out), values.size)
    return out.view(np.float32) if t == "f32" else out
