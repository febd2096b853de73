"""CPU oracle for D = A*B + C and for attention, O = softmax(scale Q K^T) V
(ctypes binding of ``oracle/oracle.c``).

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

TYPES = {"f16": 1, "bf16": 2, "f32": 3, "i8": 4, "i32": 5, "e4m3": 6}
LAYOUTS = {"row": 0, "col": 1}
ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2}
_NP_IN = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i8": np.int8, "i32": np.int32,
          "e4m3": np.uint8}

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
    ep = [vp, i64, vp, i64, vp, i64, i32]
    lib.oracle_gemm_ex.argtypes = common + ep + [vp, i64, i64, i32]
    lib.oracle_gemm_ex.restype = i32
    lib.oracle_gemm_at_ex.argtypes = common + ep + [i64, vp, vp]
    lib.oracle_gemm_at_ex.restype = i32
    att = [i64, i64, i64, i64, i64, i32, i32, ctypes.c_double, vp, i64, i64, vp, i64, i64, vp, i64, i64]
    lib.oracle_attention.argtypes = att + [vp, i64, i64, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_attention_rows.argtypes = att + [i64, vp, vp, i32]
    lib.oracle_attention_rows.restype = i32
    lib.oracle_decode_array.argtypes = [i32, vp, vp, i64]
    lib.oracle_decode_array.restype = None
    lib.oracle_decode_array8.argtypes = [i32, vp, vp, i64]
    lib.oracle_decode_array8.restype = None
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
    if in_type not in ("f16", "bf16", "f32", "i8", "e4m3"):
        raise ValueError(f"unsupported input type {in_type}")
    acc_t = out_type  # C has the output type
    span = lambda s, e: 0 if batch == 0 or e == 0 else (batch - 1) * s + e
    A = _prep(A, in_type, span(stride_a, _extent(layout_a, M, K, lda)), "A")
    B = _prep(B, in_type, span(stride_b, _extent(layout_b, K, N, ldb)), "B")
    C = _prep(C, acc_t, span(stride_c, _extent("row", M, N, ldc)), "C")
    args = (M, N, K, batch, TYPES[in_type], TYPES[out_type], LAYOUTS[layout_a], LAYOUTS[layout_b],
            _ptr(A), lda, stride_a, _ptr(B), ldb, stride_b, _ptr(C), ldc, stride_c)
    return args, (A, B, C)


def _epilogue(M, N, batch, row_scale, stride_rs, col_scale, stride_cs, bias, stride_bias, act):
    def vec(x, n, stride, name):
        if x is None:
            return None
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        need = 0 if batch == 0 or n == 0 else (batch - 1) * stride + n
        if x.size < need:
            raise ValueError(f"{name}: holds {x.size} values, needs {need}")
        return x
    rs = vec(row_scale, M, stride_rs, "row_scale")
    cs = vec(col_scale, N, stride_cs, "col_scale")
    bs = vec(bias, N, stride_bias, "bias")
    return (_ptr(rs), stride_rs, _ptr(cs), stride_cs, _ptr(bs), stride_bias, ACTS[act]), (rs, cs, bs)


def gemm(M, N, K, A, lda, B, ldb, *, in_type, out_type, layout_a="row", layout_b="row",
         batch=1, stride_a=0, stride_b=0, C=None, ldc=0, stride_c=0, ldd=None, stride_d=None,
         nthreads=None, row_scale=None, stride_rs=0, col_scale=None, stride_cs=0, bias=None,
         stride_bias=0, act="none"):
    """Full D (flat, batch*stride_d elements; row-major M x N with leading dim ldd).

    row_scale (M per batch), col_scale (N per batch), bias (N per batch; all
    float32) and act ("none", "relu", "gelu_tanh") form the optional epilogue.
    """
    ldd = N if ldd is None else ldd
    stride_d = M * ldd if stride_d is None else stride_d
    args, keep = _common(M, N, K, A, lda, B, ldb, in_type, out_type, layout_a, layout_b, batch,
                         stride_a, stride_b, C, ldc, stride_c)
    ep, keep_ep = _epilogue(M, N, batch, row_scale, stride_rs, col_scale, stride_cs, bias,
                            stride_bias, act)
    D = np.zeros(max(batch * stride_d, 1), dtype=_NP_IN[out_type])
    st = _load().oracle_gemm_ex(*args, *ep, _ptr(D), ldd, stride_d, nthreads or default_threads())
    if st:
        raise ValueError(f"oracle_gemm rejected its arguments (code {st})")
    del keep, keep_ep
    return D[: batch * stride_d]


def gemm_at(M, N, K, A, lda, B, ldb, bij, *, in_type, out_type, layout_a="row",
            layout_b="row", batch=1, stride_a=0, stride_b=0, C=None, ldc=0, stride_c=0,
            row_scale=None, stride_rs=0, col_scale=None, stride_cs=0, bias=None, stride_bias=0,
            act="none"):
    """D[b](i,j) for each row (b, i, j) of the integer array ``bij`` (shape [n, 3])."""
    args, keep = _common(M, N, K, A, lda, B, ldb, in_type, out_type, layout_a, layout_b, batch,
                         stride_a, stride_b, C, ldc, stride_c)
    ep, keep_ep = _epilogue(M, N, batch, row_scale, stride_rs, col_scale, stride_cs, bias,
                            stride_bias, act)
    bij = np.ascontiguousarray(bij, dtype=np.int64).reshape(-1, 3)
    out = np.zeros(max(len(bij), 1), dtype=_NP_IN[out_type])
    st = _load().oracle_gemm_at_ex(*args, *ep, len(bij), _ptr(bij), _ptr(out))
    if st:
        raise ValueError(f"oracle_gemm_at rejected its arguments (code {st})")
    del keep, keep_ep
    return out[: len(bij)]


def decode(t: str, bits) -> np.ndarray:
    """Exact fp64 values of fp16, bf16 or e4m3 bit patterns."""
    if t == "e4m3":
        bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
        out = np.empty(bits.size, dtype=np.float64)
        _load().oracle_decode_array8(TYPES[t], _ptr(bits), _ptr(out), bits.size)
        return out
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


def _att_common(batch, sq, sk, d, dv, Q, ldq, stride_q, K, ldk, stride_k, V, ldv, stride_v, in_type, out_type,
                scale):
    span = lambda s_, rows, ld, cols: 0 if batch == 0 or rows == 0 else (batch - 1) * s_ + (rows - 1) * ld + cols
    Q = _prep(Q, in_type, span(stride_q, sq, ldq, d), "Q")
    K = _prep(K, in_type, span(stride_k, sk, ldk, d), "K")
    V = _prep(V, in_type, span(stride_v, sk, ldv, dv), "V")
    # the softmax scale is an fp32 number on the GPU side; the oracle takes that same value
    args = (batch, sq, sk, d, dv, TYPES[in_type], TYPES[out_type], float(np.float32(scale)), _ptr(Q), ldq, stride_q,
            _ptr(K), ldk, stride_k, _ptr(V), ldv, stride_v)
    return args, (Q, K, V)


def attention(batch, sq, sk, d, dv, Q, ldq, stride_q, K, ldk, stride_k, V, ldv, stride_v, *, in_type, out_type,
              scale, ldo=None, stride_o=None, nthreads=None):
    """O = softmax(scale * Q K^T) V for every row (flat, batch*stride_o elements of out_type bits)."""
    ldo = dv if ldo is None else ldo
    stride_o = sq * ldo if stride_o is None else stride_o
    args, keep = _att_common(batch, sq, sk, d, dv, Q, ldq, stride_q, K, ldk, stride_k, V, ldv, stride_v,
                             in_type, out_type, scale)
    O = np.zeros(max(batch * stride_o, 1), dtype=_NP_IN[out_type])
    st = _load().oracle_attention(*args, _ptr(O), ldo, stride_o, nthreads or default_threads())
    if st:
        raise ValueError(f"oracle_attention rejected its arguments (code {st})")
    del keep
    return O[: batch * stride_o]


def attention_rows(batch, sq, sk, d, dv, Q, ldq, stride_q, K, ldk, stride_k, V, ldv, stride_v, rows, *,
                   in_type, out_type, scale, nthreads=None):
    """Rows (b, i) of O (``rows`` shape [n, 2]) as an [n, dv] array of out_type bits."""
    args, keep = _att_common(batch, sq, sk, d, dv, Q, ldq, stride_q, K, ldk, stride_k, V, ldv, stride_v,
                             in_type, out_type, scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    out = np.zeros(max(len(rows) * dv, 1), dtype=_NP_IN[out_type])
    st = _load().oracle_attention_rows(*args, len(rows), _ptr(rows), _ptr(out), nthreads or default_threads())
    if st:
        raise ValueError(f"oracle_attention_rows rejected its arguments (code {st})")
    del keep
    return out[: len(rows) * dv].reshape(len(rows), dv)
