"""Pins of the oracle's own fp16/bf16/fp32 codecs (CPU only).

Decoding is checked exhaustively against the formats' bit-level definitions
(numpy's binary16 view; bfloat16 = upper half of a binary32).  Encoding is
checked against exact nearest-value search (tests/exact.py) on random values,
every tie between adjacent representable values, subnormals and overflow, and
fp32 encoding against numpy's IEEE double -> single conversion.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact


def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode("f16", bits)
    ref = exact.f16_values(bits)
    assert np.array_equal(got, ref, equal_nan=True)
    # sign of zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode("bf16", bits)
    ref = exact.bf16_values(bits)
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[0x0001] == 2.0 ** -133  # smallest subnormal
    assert got[0x7F7F] == (2 - 2 ** -7) * 2.0 ** 127  # largest finite


@pytest.mark.parametrize("t", ["f16", "bf16"])
def test_encode_ties_and_midpoints(t):
    """Every midpoint between adjacent non-negative values rounds to the even pattern."""
    vals, bits = exact._table(t)
    vals = np.array(vals[:-1])
    bits = np.array(bits[:-1])
    mids = (vals[:-1] + vals[1:]) / 2  # exact in fp64 (needs one more bit than the format)
    got = oracle.encode(t, mids)
    want = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(got, want)
    got_neg = oracle.encode(t, -mids)
    assert np.array_equal(got_neg, want | 0x8000)
    # just above / below a midpoint rounds to the nearer neighbour
    up = oracle.encode(t, np.nextafter(mids, np.inf))
    dn = oracle.encode(t, np.nextafter(mids, -np.inf))
    assert np.array_equal(up, bits[1:])
    assert np.array_equal(dn, bits[:-1])


@pytest.mark.parametrize("t", ["f16", "bf16"])
def test_encode_random_against_exact_search(t):
    rng = np.random.default_rng(7)
    scale = 2.0 ** rng.integers(-30 if t == "f16" else -140, 18 if t == "f16" else 130, 3000)
    x = rng.uniform(-1, 1, 3000) * scale
    got = oracle.encode(t, x)
    want = np.array([exact.round16(Fraction(float(v)), t) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_encode_special_values():
    f = oracle.encode("f16", [np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -25,
                              2.0 ** -25 * 1.0000001, 2.0 ** -26, -0.0, np.nan])
    assert list(f[:10]) == [0x7C00, 0xFC00, 0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0x0000, 0x0001,
                            0x0000, 0x8000]
    assert (f[10] & 0x7C00) == 0x7C00 and (f[10] & 0x3FF) != 0
    b = oracle.encode("bf16", [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -134, 3.0 * 2 ** -135])
    # 1 + 2^-8 ties to 1.0 (even); 1 + 3*2^-8 ties up to 1 + 2^-6 (0x3F82);
    # half the smallest subnormal ties to zero; 1.5 * that rounds up to it.
    assert list(b) == [0x3F80, 0x3F82, 0x0000, 0x0001]


def test_encode_f32_against_numpy():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(20000) * 2.0 ** rng.integers(-160, 130, 20000)
    x = np.concatenate([x, [1 + 2 ** -24, 1 + 3 * 2 ** -24, 2.0 ** -150, 3 * 2.0 ** -151,
                            3.4028235677973366e38, 3.4028235e38 * 1.0000001]])
    with np.errstate(over="ignore"):
        want = x.astype(np.float32)
    got = oracle.encode("f32", x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
