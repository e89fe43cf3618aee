"""Pins for the oracle's scales: exact rational rounding and the absmean beta.

Every expected value here comes from an independent route: Python Fractions,
brute-force search of neighbouring fp32 values, hand-built inputs whose mean
is known in closed form, or a textbook statistic of the half-normal law.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import sbl_oracle as O
from synth import f32_to_bf16_bits


def _brute_f32_round(fr: Fraction) -> np.float32:
    """Nearest fp32 to a non-negative Fraction by searching neighbours."""
    approx = np.float32(float(fr))
    cands = {approx}
    lo = hi = approx
    for _ in range(3):
        lo = np.nextafter(lo, np.float32(0)) if lo > 0 else lo
        hi = np.nextafter(hi, np.float32(np.inf))
        cands |= {lo, hi}
    best = None
    for c in sorted(cands):
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - fr)
        even = (np.array(c, dtype=np.float32).view(np.uint32) & 1) == 0
        key = (d, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_rational_to_f32_matches_neighbour_search():
    rng = np.random.default_rng(123)
    for _ in range(3000):
        scale = int(rng.integers(-160, 90))   # stays below FLT_MAX
        num = int(rng.integers(1, 1 << 40))
        den = int(rng.integers(1, 1 << 30))
        if scale >= 0:
            num <<= scale
        else:
            den <<= -scale
        fr = Fraction(num, den)
        got = O.rational_to_f32(num, den)
        assert got == _brute_f32_round(fr), (num, den)


def test_rational_to_f32_midpoints_go_to_even():
    # 1 + 2^-24 lies halfway between 1 and 1 + 2^-23: even mantissa is 1.0
    assert O.rational_to_f32((1 << 24) + 1, 1 << 24) == np.float32(1.0)
    # 1 + 3*2^-24 lies halfway between 1+2^-23 (odd) and 1+2^-22 (even)
    assert O.rational_to_f32((1 << 24) + 3, 1 << 24) == np.float32(1.0 + 2.0 ** -22)
    # smallest subnormal halfway case: 2^-150 -> 0 (even), 3*2^-150 -> 2*2^-149
    assert O.rational_to_f32(1, 1 << 150) == np.float32(0.0)
    assert O.rational_to_f32(3, 1 << 150) == np.float32(2.0 ** -148)
    # exact fp32 values round to themselves
    for v in [1.0, 0.1, 3.0e-39, 1.2e-38, 65504.0, 3.4e38]:
        f = Fraction(float(np.float32(v)))
        assert O.rational_to_f32(f.numerator, f.denominator) == np.float32(v)


def _bf16_values(rng, n):
    """BF16 bit patterns spanning zeros, subnormals, normal and large values."""
    kind = rng.integers(0, 5, n)
    mag = np.where(kind == 0, 0,
          np.where(kind == 1, rng.integers(1, 0x80, n),            # subnormal
          np.where(kind == 2, rng.integers(0x3000, 0x4000, n),     # [2^-31, 2)
          np.where(kind == 3, rng.integers(0x0080, 0x3000, n),     # tiny normal
                   rng.integers(0x4000, 0x7F80, n)))))              # large
    sign = rng.integers(0, 2, n) << 15
    return (mag | sign).astype(np.uint16)


def test_absmean_equals_fraction_sum():
    rng = np.random.default_rng(7)
    for n in [1, 2, 3, 8, 17, 64, 333]:
        bits = _bf16_values(rng, n)
        vals = O.bf16_to_f32(bits)
        exact = sum((Fraction(float(abs(v))) for v in vals), Fraction(0)) / n
        assert O.absmean_exact(bits) == exact
        assert O.absmean_beta(bits) == _brute_f32_round(exact)


def test_beta_constant_magnitude():
    # every |w| = a  ->  beta = a exactly, whatever the signs
    rng = np.random.default_rng(3)
    for a in [0.015625, 0.0200195, 1.5, 3.0e-5]:
        ab = f32_to_bf16_bits(np.array([a], np.float32))[0]
        signs = rng.integers(0, 2, 1000).astype(np.uint16) << 15
        bits = (ab | signs).astype(np.uint16)
        assert O.absmean_beta(bits) == O.bf16_to_f32(np.array([ab]))[0]


def test_beta_midpoint_inputs():
    n = 1 << 17
    one = 0x3F80                      # 1.0
    one_p = 0x3F81                    # 1 + 2^-7
    one_p3 = 0x3F83                   # 1 + 3*2^-7
    bits = np.full(n, one, np.uint16)
    bits[5] = one_p                   # mean = 1 + 2^-24: a tie -> 1.0
    assert O.absmean_beta(bits) == np.float32(1.0)
    bits[5] = one_p3                  # mean = 1 + 3*2^-24: a tie -> 1 + 2^-22
    assert O.absmean_beta(bits) == np.float32(1.0 + 2.0 ** -22)
    bits[5] = one_p
    bits[9] = one_p | 0x8000          # mean = 1 + 2^-23 exactly
    assert O.absmean_beta(bits) == np.float32(1.0 + 2.0 ** -23)


def test_beta_gaussian_half_normal_mean():
    # E|w| = sigma * sqrt(2/pi) for w ~ N(0, sigma^2)
    rng = np.random.default_rng(11)
    sigma = 0.02
    w = rng.standard_normal(1 << 21).astype(np.float32) * np.float32(sigma)
    beta = float(O.absmean_beta(f32_to_bf16_bits(w)))
    assert abs(beta / (sigma * math.sqrt(2 / math.pi)) - 1) < 3e-3


def test_beta_rejects_nonfinite():
    with pytest.raises(ValueError):
        O.absmean_beta(np.array([0x3F80, 0x7F80], np.uint16))
