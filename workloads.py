"""Seeded synthetic inputs for D = A*B + C, shared by the GPU path and the oracle.

This module holds no part of the product's arithmetic: it only draws values,
rounds them to the input type with numpy/torch conversions, and lays them out
with the call parameters (sizes, layouts, leading dimensions, strides) that
both sides receive unchanged.  The workloads follow the five problems that
centre the pages' discussion:

  c1   fp16 256^3, A and B row-major, fp32 accumulate and output, C = 0
  c2   bf16 4096^3, A and B row-major, fp32 accumulate, bf16 output
  c3   fp16 5000 x 3000 x 2050, A row-major, B column-major, fp16 output
  c4s  batch 32 of S = Q K^T, Q and K 4096 x 128 (B column-major), fp32 output
  c4o  batch 32 of O = P V, P 4096 x 4096 softmax rows, V 4096 x 128, fp32 output
  c5   int8 8192^3, A row-major, B column-major, int32 output
  c5nn int8 8192^3, A and B row-major (an 8-bit operand that is not K-contiguous), int32 output
  c6   FP8 e4m3 8192^3, A row-major, B column-major, fp32 accumulate, bf16 output
  lk   bf16 1024 x 1024 x 16384 (long K, few output tiles), A and B row-major, bf16 output

Random draws come from ``numpy.random.default_rng([config_id, matrix_id, seed])``
in fp64 and are rounded to the input type.  ``structured`` copies hold small
integers whose products have closed forms; they are exact in every type.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

CONFIG_IDS = {"c1": 1, "c2": 2, "c3": 3, "c4s": 41, "c4o": 42, "c5": 5, "c5nn": 51, "c6": 6, "lk": 7}

# (M, N, K, batch, in_type, out_type, acc_type, layout_a, layout_b)
FULL = {
    "c1": (256, 256, 256, 1, "f16", "f32", "f32", "row", "row"),
    "c2": (4096, 4096, 4096, 1, "bf16", "bf16", "f32", "row", "row"),
    "c3": (5000, 3000, 2050, 1, "f16", "f16", "f16", "row", "col"),
    "c4s": (4096, 4096, 128, 32, "f16", "f32", "f32", "row", "col"),
    "c4o": (4096, 128, 4096, 32, "f16", "f32", "f32", "row", "row"),
    "c5": (8192, 8192, 8192, 1, "i8", "i32", "i32", "row", "col"),
    "c5nn": (8192, 8192, 8192, 1, "i8", "i32", "i32", "row", "row"),
    "c6": (8192, 8192, 8192, 1, "e4m3", "bf16", "f32", "row", "col"),
    "lk": (1024, 1024, 16384, 1, "bf16", "bf16", "f32", "row", "row"),
}

_NP_BITS = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i8": np.int8, "i32": np.int32,
            "e4m3": np.uint8}
ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "i8": 1, "i32": 4}


@dataclass
class Problem:
    """One call's worth of inputs, as raw element bits plus the call parameters."""

    name: str
    M: int
    N: int
    K: int
    batch: int
    in_type: str
    acc_type: str
    out_type: str
    layout_a: str
    layout_b: str
    A: np.ndarray
    lda: int
    stride_a: int
    B: np.ndarray
    ldb: int
    stride_b: int
    C: Optional[np.ndarray] = None
    ldc: int = 0
    stride_c: int = 0
    ldd: int = 0
    stride_d: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def d_elems(self) -> int:
        return self.batch * self.stride_d if self.batch else 0


def to_bits(x: np.ndarray, t: str) -> np.ndarray:
    """Round fp64 draws to the input type (library conversions) and return raw bits."""
    if t == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
    if t == "bf16":
        import torch

        f = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if t == "e4m3":
        import torch

        f = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return f.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if t == "f32":
        return np.asarray(x, dtype=np.float32)
    if t == "i8":
        return np.asarray(x, dtype=np.int8)
    if t == "i32":
        return np.asarray(x, dtype=np.int32)
    raise ValueError(t)


def _rng(cfg: str, matrix_id: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([CONFIG_IDS.get(cfg, 99), matrix_id, seed])


def _layout_params(M, N, K, layout_a, layout_b, pad=0):
    """Leading dimensions for densely stored operands (plus optional padding)."""
    lda = (K if layout_a == "row" else M) + pad
    ldb = (N if layout_b == "row" else K) + pad
    rows_a = M if layout_a == "row" else K
    rows_b = K if layout_b == "row" else N
    return lda, ldb, rows_a * lda, rows_b * ldb


def _storage(logical: np.ndarray, layout: str, ld: int) -> np.ndarray:
    """Store a logical [batch, R, Cc] array row- or column-major with leading dim ld."""
    b, r, c = logical.shape
    if layout == "row":
        out = np.zeros((b, r, ld), dtype=logical.dtype)
        out[:, :, :c] = logical
    else:
        out = np.zeros((b, c, ld), dtype=logical.dtype)
        out[:, :, :r] = np.transpose(logical, (0, 2, 1))
    return out.reshape(-1)


def store(logical: np.ndarray, t: str, layout: str, pad: int = 0) -> tuple[np.ndarray, int]:
    """Raw bits of a logical [batch, R, C] value array in the given layout; returns (bits, ld)."""
    b, r, c = logical.shape
    ld = (c if layout == "row" else r) + pad
    bits = to_bits(np.ascontiguousarray(logical).reshape(-1), t).reshape(b, r, c)
    return _storage(bits, layout, ld), ld


def _slices(cfg, kind, seed, M, N, K, batch):
    """Per-batch generators of the logical fp64 (or integer) A [M, K] and B [K, N]."""
    i = np.arange(M)[:, None]
    j = np.arange(N)[None, :]
    kk_row = np.arange(K)[None, :]
    kk_col = np.arange(K)[:, None]
    if kind == "random":
        ra, rb = _rng(cfg, 0, seed), _rng(cfg, 1, seed)
        if cfg in ("c1", "c4s"):
            return (lambda q: ra.uniform(-1, 1, (M, K))), (lambda q: rb.uniform(-1, 1, (K, N)))
        if cfg in ("c2", "lk"):
            s = 1.0 / np.sqrt(K) if K else 1.0
            return (lambda q: ra.standard_normal((M, K)) * s), (lambda q: rb.standard_normal((K, N)) * s)
        if cfg == "c3":
            return (lambda q: ra.uniform(-0.5, 0.5, (M, K))), (lambda q: rb.uniform(-0.5, 0.5, (K, N)))
        if cfg == "c4o":
            def softmax_rows(q):  # softmax of N(0,1) logits, rows sum to 1
                z = ra.standard_normal((M, K))
                z -= z.max(axis=1, keepdims=True)
                np.exp(z, out=z)
                z /= z.sum(axis=1, keepdims=True)
                return z
            return softmax_rows, (lambda q: rb.uniform(-1, 1, (K, N)))
        if cfg in ("c5", "c5nn"):
            return (lambda q: ra.integers(-128, 128, (M, K))), (lambda q: rb.integers(-128, 128, (K, N)))
        if cfg == "c6":  # N(0, 1) rounded to e4m3 (|x| stays far below its largest value, 448)
            return (lambda q: ra.standard_normal((M, K))), (lambda q: rb.standard_normal((K, N)))
    elif kind == "structured":
        if cfg in ("c1", "c2", "c5", "c5nn", "c6", "lk"):
            return (lambda q: np.broadcast_to(i % 16, (M, K))), (lambda q: np.broadcast_to(j % 8, (K, N)))
        if cfg == "c3":
            return (lambda q: (kk_row % 16 == i % 16).astype(np.float64)), \
                   (lambda q: np.broadcast_to(j % 8, (K, N)))
        if cfg == "c4s":
            return (lambda q: np.broadcast_to((i + q) % 16, (M, K))), \
                   (lambda q: np.broadcast_to(j % 8, (K, N)))
        if cfg == "c4o":
            return (lambda q: (kk_row == (i + q) % K).astype(np.float64)), \
                   (lambda q: ((kk_col + 3 * q + j) % 64) - 32.0)
    raise ValueError((cfg, kind))


def _store_slices(gen, t, layout, batch, rows, cols, ld):
    """Raw bits of all batch slices, stored row- or column-major with leading dim ld."""
    per = (rows if layout == "row" else cols) * ld
    out = np.zeros(batch * per, dtype=_NP_BITS[t])
    for q in range(batch):
        x = np.asarray(gen(q))
        bits = to_bits(np.ascontiguousarray(x).reshape(-1), t).reshape(rows, cols)
        dst = out[q * per: (q + 1) * per]
        if layout == "row":
            dst.reshape(rows, ld)[:, :cols] = bits
        else:
            dst.reshape(cols, ld)[:, :rows] = bits.T
    return out


def make(cfg: str, kind: str = "random", seed: int = 0, *, M=None, N=None, K=None, batch=None,
         pad: int = 0, with_c: bool = False) -> Problem:
    """Build a workload.  Sizes default to the full problem; override to shrink it.

    kind: "random" (the problem's value distribution) or "structured" (closed form).
    pad:  extra elements per leading dimension (exercises ld > rows/cols).
    with_c: add a seeded C operand (the full problems pass C = 0 or none).
    """
    fM, fN, fK, fb, in_t, out_t, acc_t, la, lb = FULL[cfg]
    M = fM if M is None else M
    N = fN if N is None else N
    K = fK if K is None else K
    batch = fb if batch is None else batch
    lda, ldb, sa, sb = _layout_params(M, N, K, la, lb, pad)
    ga, gb = _slices(cfg, kind, seed, M, N, K, batch)
    A = _store_slices(ga, in_t, la, batch, M, K, lda)
    B = _store_slices(gb, in_t, lb, batch, K, N, ldb)
    ldd = N + pad
    meta = {"kind": kind, "seed": seed, "cfg": cfg}
    p = Problem(cfg, M, N, K, batch, in_t, acc_t, out_t, la, lb, A, lda, sa if batch > 1 else 0,
                B, ldb, sb if batch > 1 else 0, ldd=ldd, stride_d=M * ldd, meta=meta)
    if cfg == "c1" and not with_c:
        # c1 states C = 0 explicitly: pass a zero C operand.
        p.C = np.zeros(batch * M * ldd, dtype=_NP_BITS[out_t])
        p.ldc, p.stride_c = ldd, (M * ldd if batch > 1 else 0)
    if with_c:
        rc = _rng(cfg, 2, seed)
        c_t = out_t
        if c_t == "i32":
            cv = rc.integers(-1000, 1000, batch * M * ldd)
        else:
            cv = rc.uniform(-1, 1, batch * M * ldd)
            if kind == "structured":
                cv = np.round(cv * 8)
        p.C = to_bits(cv, c_t)
        p.ldc, p.stride_c = ldd, (M * ldd if batch > 1 else 0)
    return p


def shrink(p: Problem, **kw) -> Problem:
    return replace(p, **kw)


def with_output(p: Problem, out_t: str, seed: int = 0) -> Problem:
    """The same inputs with another output type (int8 -> fp32/fp16/bf16 dequantisation,
    or the other float output of a float problem); a C operand is redrawn in that type."""
    q = replace(p, out_type=out_t, meta=dict(p.meta, out=out_t))
    if p.C is not None:
        rc = _rng(p.meta.get("cfg", p.name), 3, seed)
        n = p.batch * p.M * p.ldc if p.batch > 1 else p.M * p.ldc
        cv = rc.uniform(-1, 1, n)
        if p.meta.get("kind") == "structured":
            cv = np.round(cv * 8)
        q.C = to_bits(cv, out_t) if out_t != "i32" else rc.integers(-1000, 1000, n).astype(np.int32)
    return q


@dataclass
class Epilogue:
    """Operands of the fused epilogue: per-row and per-column scales and a per-column
    bias (float32, one vector per batch slice at the given stride), and an activation."""

    row_scale: Optional[np.ndarray]
    stride_rs: int
    col_scale: Optional[np.ndarray]
    stride_cs: int
    bias: Optional[np.ndarray]
    stride_bias: int
    act: str

    def kwargs(self) -> dict:
        return dict(row_scale=self.row_scale, stride_rs=self.stride_rs, col_scale=self.col_scale,
                    stride_cs=self.stride_cs, bias=self.bias, stride_bias=self.stride_bias,
                    act=self.act)


def make_epilogue(p: Problem, seed: int = 0, act: str = "none", row: bool = True, col: bool = True,
                  bias: bool = True, exact: bool = False) -> Epilogue:
    """Seeded epilogue operands for problem p.

    exact=True draws powers of two for the scales and small integers for the bias, so
    that with integer-valued products every epilogue step is exact in fp32.  Otherwise
    the scales are the per-row / per-column dequantisation factors of an int8 problem
    (about 1/127 of a unit range) or O(1) factors for float problems, and the bias is
    O(1).  Batched problems get a padded stride per vector (M + 3, N + 5).
    """
    rng = np.random.default_rng([77, seed, p.M, p.N, p.batch])
    sr = p.M + 3 if p.batch > 1 else 0
    sc = p.N + 5 if p.batch > 1 else 0
    nr = (p.batch - 1) * sr + p.M if p.batch else 0
    nc = (p.batch - 1) * sc + p.N if p.batch else 0

    def scales(n):
        if exact:
            return (2.0 ** rng.integers(-3, 4, n)).astype(np.float32)
        if p.in_type == "i8":
            return rng.uniform(0.5 / 127, 2.0 / 127, n).astype(np.float32)
        return rng.uniform(0.5, 2.0, n).astype(np.float32)

    rs = scales(nr) if row else None
    cs = scales(nc) if col else None
    if bias:
        bv = rng.integers(-8, 9, nc) if exact else rng.uniform(-1, 1, nc)
        bv = bv.astype(np.float32)
    else:
        bv = None
    return Epilogue(rs, sr, cs, sc, bv, sc, act)
