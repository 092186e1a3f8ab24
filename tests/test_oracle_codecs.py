"""Pins for the oracle's IEEE 754 decoders and round-to-nearest-even encoders.

The oracle rounds its fp64 results once into float16, bfloat16 or float32.
These tests pin that rounding to things other than the oracle: numpy's
float16/float32 conversions (correctly rounded from float64), bfloat16 as the
upper half of a float32, and exact rational arithmetic (``fractions``) for
ties and for bfloat16 rounding.
"""
import warnings
from fractions import Fraction

import numpy as np
import pytest

import oracle

warnings.filterwarnings("ignore", message="invalid value encountered in cast")

ALL16 = np.arange(1 << 16, dtype=np.uint32)


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal as values, with NaN matching NaN and signed zeros distinguished."""
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_decode_f16_exhaustive():
    mine = oracle.decode("f16", ALL16)
    ref = ALL16.astype(np.uint16).view(np.float16).astype(np.float64)
    assert _same(mine, ref)


def test_decode_bf16_exhaustive():
    mine = oracle.decode("bf16", ALL16)
    ref = (ALL16 << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    assert _same(mine, ref)


def test_decode_f32_sampled():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, np.array([0, 1, 0x7F7FFFFF, 0x80000001, 0x7F800000, 0xFF800000,
                                           0x00800000, 0x007FFFFF], dtype=np.uint32)])
    mine = oracle.decode("f32", bits)
    ref = bits.view(np.float32).astype(np.float64)
    assert _same(mine, ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_roundtrip_exhaustive(dtype):
    vals = oracle.decode(dtype, ALL16)
    back = oracle.encode(dtype, vals)
    finite_or_inf = ~np.isnan(vals)
    assert np.array_equal(back[finite_or_inf], ALL16[finite_or_inf])
    assert np.all(np.isnan(oracle.decode(dtype, back[~finite_or_inf])))


def _interesting_doubles(rng, dtype):
    """Random doubles plus exact midpoints, near-midpoints, subnormals and the
    overflow boundary of ``dtype``."""
    vals = [rng.standard_normal(20000) * s for s in (1e-8, 1e-5, 1e-3, 1.0, 300.0, 6e4)]
    fin = oracle.decode(dtype, ALL16 if dtype != "f32" else
                        rng.integers(0, 0x7F800000, 20000, dtype=np.uint64).astype(np.uint32))
    fin = fin[np.isfinite(fin)]
    fin = np.sort(np.unique(np.abs(fin)))
    mids = (fin[:-1] + fin[1:]) / 2          # exact midpoints (one more bit is enough)
    vals += [mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), fin, -fin]
    return np.concatenate(vals)


def test_encode_f16_matches_numpy():
    rng = np.random.default_rng(2)
    v = _interesting_doubles(rng, "f16")
    v = np.concatenate([v, [65504.0, 65519.99, 65520.0, 65536.0, 1e6, -65520.0,
                            2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16).astype(np.uint32)
    assert np.array_equal(oracle.encode("f16", v), ref)


def test_encode_f32_matches_numpy():
    rng = np.random.default_rng(3)
    v = _interesting_doubles(rng, "f32")
    big = float(np.finfo(np.float32).max)
    v = np.concatenate([v, [big, big * (1 + 2.0 ** -25), big * (1 + 2.0 ** -24), 1e39,
                            2.0 ** -149, 2.0 ** -150, 2.0 ** -150 * 1.5, 1e-50]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.encode("f32", v), ref)


def _rne_bf16_exact(x: float) -> int:
    """Brute-force RNE into bfloat16 with exact rationals: pick the nearest of
    all finite bfloat16 values; ties go to the even significand; beyond the
    largest finite value by half a unit or more the result is infinity."""
    if x != x:
        return None
    neg = x < 0 or (x == 0 and np.signbit(x))
    a = Fraction(abs(x))
    table = _BF16_POS
    lo, hi = 0, len(table) - 1
    # binary search for neighbours
    if a >= table[-1][0]:
        top, topbits = table[-1]
        half_ulp = (top - table[-2][0]) / 2
        return (0x7F80 if a >= top + half_ulp else topbits) | (0x8000 if neg else 0)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if table[mid][0] <= a:
            lo = mid
        else:
            hi = mid
    (va, ba), (vb, bb) = table[lo], table[hi]
    da, db = a - va, vb - a
    if da < db:
        bits = ba
    elif db < da:
        bits = bb
    else:
        bits = ba if ba % 2 == 0 else bb
    return bits | (0x8000 if neg else 0)


_BF16_POS = [(Fraction(float(v)), int(b)) for b, v in
             zip(range(0, 0x7F80), oracle.decode("bf16", np.arange(0, 0x7F80, dtype=np.uint32)))]


def test_encode_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(4)
    v = _interesting_doubles(rng, "bf16")
    v = v[rng.choice(len(v), size=6000, replace=False)]
    bmax = float(oracle.decode("bf16", np.array([0x7F7F], dtype=np.uint32))[0])
    extra = [bmax, bmax * (1 + 2.0 ** -9), bmax * (1 + 2.0 ** -8), -bmax * (1 + 2.0 ** -8),
             2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 1e-45, 0.0, -0.0,
             1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40]
    v = np.concatenate([v, extra])
    mine = oracle.encode("bf16", v)
    for x, m in zip(v.tolist(), mine.tolist()):
        assert m == _rne_bf16_exact(x), (x, hex(m))


@pytest.mark.parametrize("dtype,one_plus_half_ulp,even,odd_up", [
    ("f16", 1 + 2.0 ** -11, 0x3C00, 0x3C02),
    ("bf16", 1 + 2.0 ** -8, 0x3F80, 0x3F82),
    ("f32", 1 + 2.0 ** -24, 0x3F800000, 0x3F800002),
])
def test_constructed_ties_go_to_even(dtype, one_plus_half_ulp, even, odd_up):
    # 1 + half ulp lies between 1 (even significand) and 1 + ulp (odd): -> 1
    assert oracle.encode(dtype, np.array([one_plus_half_ulp]))[0] == even
    # 1 + 3 half ulps lies between 1 + ulp (odd) and 1 + 2 ulp (even): -> up
    three_half = 1 + 3 * (one_plus_half_ulp - 1)
    assert oracle.encode(dtype, np.array([three_half]))[0] == odd_up
    # negative mirror
    sign = 0x8000 if dtype != "f32" else 0x80000000
    assert oracle.encode(dtype, np.array([-one_plus_half_ulp]))[0] == even | sign


def test_nan_and_infinity():
    for dtype, inf, sign, mant in (("f16", 0x7C00, 0x8000, 0x03FF), ("bf16", 0x7F80, 0x8000, 0x007F),
                                   ("f32", 0x7F800000, 0x80000000, 0x007FFFFF)):
        enc = [int(e) for e in oracle.encode(dtype, np.array([np.inf, -np.inf, np.nan]))]
        assert enc[0] == inf
        assert enc[1] == inf | sign
        assert (enc[2] & inf) == inf and (enc[2] & mant) != 0
