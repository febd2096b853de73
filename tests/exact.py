"""Exact reference arithmetic for pinning the oracle (test helper, CPU only).

Nothing here shares code with ``oracle/``: values are decoded with the formats'
bit-level definitions through numpy views, and rounding picks the nearest
representable value by exact rational comparison against an enumerated or
neighbour-searched candidate set, ties going to the pattern with an even last
mantissa bit (IEEE 754 roundTiesToEven).
"""
from __future__ import annotations

import bisect
from decimal import Decimal, localcontext
from fractions import Fraction
from functools import lru_cache

import numpy as np


def f16_value(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def bf16_value(bits: int) -> float:
    # bfloat16 is by definition the upper half of an IEEE binary32 pattern.
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@lru_cache(maxsize=None)
def _table(t: str):
    """Sorted non-negative finite values of a 16-bit format with their bit patterns,
    followed by a pseudo-entry 2^(emax+1) standing for +inf (its pattern has an even
    mantissa, so a tie at max + half-ulp goes to infinity as IEEE 754 requires)."""
    bits = np.arange(0x8000, dtype=np.uint16)
    vals = f16_values(bits) if t == "f16" else bf16_values(bits)
    keep = np.isfinite(vals)
    vals, bits = vals[keep], bits[keep]
    order = np.argsort(vals, kind="stable")
    vals, bits = list(vals[order]), [int(b) for b in bits[order]]
    inf_bits = 0x7C00 if t == "f16" else 0x7F80
    top = 2.0 ** 16 if t == "f16" else 2.0 ** 128
    return vals + [top], bits + [inf_bits]


def round16(x: Fraction, t: str) -> int:
    """Bits of the f16/bf16 value nearest to the exact rational x (ties to even)."""
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    vals, bits = _table(t)
    if a >= Fraction(vals[-1]):
        return sign | bits[-1]
    hi = bisect.bisect_left(vals, float(a))
    cands = [c for c in (hi - 2, hi - 1, hi, hi + 1) if 0 <= c < len(vals)]
    best = min(cands, key=lambda c: (abs(Fraction(vals[c]) - a), bits[c] & 1))
    return sign | bits[best]


def round32(x: Fraction) -> np.float32:
    """The binary32 value nearest to the exact rational x (ties to even)."""
    c = np.float32(float(x))
    if not np.isfinite(c):
        return c
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    cands = [v for v in cands if np.isfinite(v)]
    def key(v):
        return (abs(Fraction(float(v)) - x), int(np.array([v], dtype=np.float32).view(np.uint32)[0]) & 1)
    best = min(cands, key=key)
    if best == 0 and x < 0:
        return np.float32(-0.0)
    return best


@lru_cache(maxsize=None)
def _e4m3_table():
    """The 256 e4m3 code values through torch's float8_e4m3fn conversion (a library routine)."""
    import torch

    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_values(bits: np.ndarray) -> np.ndarray:
    return _e4m3_table()[np.asarray(bits, dtype=np.uint8)]


def exact_value(bits, t: str) -> Fraction:
    if t == "e4m3":
        return Fraction(float(_e4m3_table()[int(bits)]))
    if t == "f16":
        return Fraction(f16_value(int(bits)))
    if t == "bf16":
        return Fraction(bf16_value(int(bits)))
    if t == "f32":
        return Fraction(float(bits))
    return Fraction(int(bits))


@lru_cache(maxsize=None)
def _pi60() -> Decimal:
    """pi to 60 digits by Machin's formula, 16 atan(1/5) - 4 atan(1/239)."""
    with localcontext() as ctx:
        ctx.prec = 70
        def atan_inv(n):
            s, term, k, n2 = Decimal(0), Decimal(1) / n, 0, n * n
            while term != 0:
                s += term / (2 * k + 1) if k % 2 == 0 else -term / (2 * k + 1)
                term /= n2
                k += 1
            return s
        return +(16 * atan_inv(5) - 4 * atan_inv(239))


def gelu_tanh(x: Fraction) -> Fraction:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) to 60 significant digits, with
    tanh from exponentials in Python's decimal module (no libm)."""
    with localcontext() as ctx:
        ctx.prec = 60
        d = Decimal(x.numerator) / Decimal(x.denominator)
        u = (2 / _pi60()).sqrt() * (d + Decimal("0.044715") * d * d * d)
        # 0.5 (1 + tanh u) = e^(2u) / (1 + e^(2u)) = 1 / (1 + e^(-2u)); the exponent taken
        # is never positive, so neither form overflows or cancels
        if u < 0:
            e = (2 * u).exp()
            s = e / (1 + e)
        else:
            s = 1 / (1 + (-2 * u).exp())
        g = Fraction(d * s)
    if g == 0 and x < 0:
        # e^(2u) underflowed: the value is negative and below any fp32 subnormal
        return Fraction(-1, 10 ** 400)
    return g


def apply_epilogue(v: Fraction, ep, b: int, i: int, j: int, addend: Fraction) -> Fraction:
    """rs(i) * cs(j) * v + bias(j) + addend, then the activation (exact rationals)."""
    if ep is not None:
        if ep.row_scale is not None:
            v *= Fraction(float(ep.row_scale[b * ep.stride_rs + i]))
        if ep.col_scale is not None:
            v *= Fraction(float(ep.col_scale[b * ep.stride_cs + j]))
        if ep.bias is not None:
            v += Fraction(float(ep.bias[b * ep.stride_bias + j]))
    v += addend
    act = "none" if ep is None else ep.act
    if act == "relu":
        v = v if v > 0 else Fraction(0)
    elif act == "gelu_tanh":
        v = gelu_tanh(v)
    return v


def brute_gemm(p, ep=None):
    """Exact D of a (tiny) workload: rational sums for floats, Python ints for int8,
    followed by the epilogue ``ep`` (a workloads.Epilogue, or None).

    Reads operands element by element from the raw storage with the BLAS-convention
    addressing, independently of the oracle's loops.
    """
    def a_at(b, i, k):
        off = b * p.stride_a + (i * p.lda + k if p.layout_a == "row" else i + k * p.lda)
        return exact_value(p.A[off], p.in_type)

    def b_at(b, k, j):
        off = b * p.stride_b + (k * p.ldb + j if p.layout_b == "row" else k + j * p.ldb)
        return exact_value(p.B[off], p.in_type)

    def wrap32(v):
        v = int(v) & 0xFFFFFFFF
        return v - (1 << 32) if v >= (1 << 31) else v

    c_t = p.out_type
    out = np.zeros(p.batch * p.stride_d, dtype={"f32": np.float32, "f16": np.uint16,
                                                "bf16": np.uint16, "i32": np.int32}[p.out_type])
    for b in range(p.batch):
        for i in range(p.M):
            for j in range(p.N):
                s = sum((a_at(b, i, k) * b_at(b, k, j) for k in range(p.K)), Fraction(0))
                c = exact_value(p.C[b * p.stride_c + i * p.ldc + j], c_t) if p.C is not None else 0
                o = b * p.stride_d + i * p.ldd + j
                if p.out_type == "i32":
                    out[o] = wrap32(s + c)
                    continue
                if p.in_type == "i8":
                    s = Fraction(wrap32(s))  # the int32 accumulator
                v = apply_epilogue(s, ep, b, i, j, Fraction(c))
                if p.out_type == "f32":
                    out[o] = round32(v)
                else:
                    out[o] = round16(v, p.out_type)
    return out
