"""Pins for the oracle's ablation orders (the pages' training-design analysis):
mask-then-quant (beta over the kept masters only) and masks from the ternary
codes instead of the masters.

Independent routes: a hand-derived 24-weight example whose three orders
differ in known places, exact-Fraction means and RoundClip on tiny random
matrices, enumeration of every C(m, n) subset on |codes|, and invariants.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import sbl_oracle as O
from synth import f32_to_bf16_bits


def _row(mags_256):
    """One row of masters, magnitude mags/256, sign + at even and - at odd k."""
    mags = np.asarray(mags_256, np.float64) / 256.0
    sign = np.where(np.arange(mags.size) % 2 == 0, 1.0, -1.0)
    return f32_to_bf16_bits((sign * mags).astype(np.float32))[None, :]


# groups of 8: [8 x6, 1, 1], [5 x5, 3, 1, 1], [7, 6, 5, 4, 3, 9, 9, 9]  (units of 1/256)
HAND = [8, 8, 8, 8, 8, 8, 1, 1, 5, 5, 5, 5, 5, 3, 1, 1, 7, 6, 5, 4, 3, 9, 9, 9]
SIGN = np.where(np.arange(24) % 2 == 0, 1, -1).astype(np.int8)


def test_hand_example_three_orders():
    bits = _row(HAND)
    # quant-then-mask: beta = 132/24/256 = 11/512; beta/2 = 2.75/256, so 3 and above are nonzero
    keep_master = np.zeros(24, bool)
    keep_master[[0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 16, 17, 18, 21, 22, 23]] = True
    beta, keep, codes = O.quant_weights(bits, 6, 8, O.QUANT_THEN_MASK)
    assert beta == np.float32(11 / 512)
    assert np.array_equal(keep[0], keep_master)
    assert np.array_equal(codes[0], SIGN * keep_master)
    # mask-then-quant: beta = (48 + 28 + 45)/18/256 = 121/4608; beta/2 = 3.361/256,
    # so the kept 3 (k = 13) becomes 0
    beta, keep, codes = O.quant_weights(bits, 6, 8, O.MASK_THEN_QUANT)
    assert beta == np.float32(121 / 4608)
    assert np.array_equal(keep[0], keep_master)
    want = SIGN * keep_master
    want[13] = 0
    assert np.array_equal(codes[0], want)
    # masks from codes: beta as quant-then-mask; group 3 has 8 nonzero codes, all
    # tied at |c| = 1, so the 6 lowest indices win (the two 9s at k = 22, 23 drop)
    beta, keep, codes = O.quant_weights(bits, 6, 8, O.MASK_FROM_CODES)
    assert beta == np.float32(11 / 512)
    keep_codes = np.zeros(24, bool)
    keep_codes[[0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 16, 17, 18, 19, 20, 21]] = True
    assert np.array_equal(keep[0], keep_codes)
    assert np.array_equal(codes[0], SIGN * keep_codes)


def _brute_top_n(vals, n):
    """Lexicographically first subset of n positions with the largest sum."""
    best = None
    for sub in itertools.combinations(range(len(vals)), n):
        key = (-sum(vals[i] for i in sub), sub)
        if best is None or key < best:
            best = key
    keep = np.zeros(len(vals), bool)
    keep[list(best[1])] = True
    return keep


def _roundclip(w, beta):
    r = Fraction(w) / Fraction(float(max(np.float32(beta), np.float32(1e-5))))
    return max(-1, min(1, round(r)))       # half to even


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (5, 8), (3, 8), (1, 4)])
def test_mask_then_quant_brute_force(n, m):
    rng = np.random.default_rng([200, n, m])
    pool = f32_to_bf16_bits(np.array([0.0, -0.0, 0.003, -0.004, 0.01, -0.02, 0.025, 0.05, -0.05],
                                     np.float32))
    bits = rng.choice(pool, size=(4, 4 * m)).astype(np.uint16)
    beta, keep, codes = O.quant_weights(bits, n, m, O.MASK_THEN_QUANT)
    w = O.bf16_to_f32(bits).astype(np.float64)
    kept = [Fraction(abs(float(w[r, c]))) for r in range(4) for c in range(4 * m) if keep[r, c]]
    assert len(kept) == 4 * 4 * n
    mean = sum(kept) / len(kept)
    assert Fraction(float(beta)) == Fraction(float(np.float32(float(mean)))) or \
        abs(Fraction(float(beta)) - mean) <= mean * Fraction(1, 1 << 24)
    for r in range(4):
        for c in range(4 * m):
            want = _roundclip(w[r, c], beta) if keep[r, c] else 0
            assert codes[r, c] == want, (r, c)
    # the mask itself is the masters' mask (as quant-then-mask)
    assert np.array_equal(keep, O.nm_keep(bits, n, m))


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (5, 8), (7, 8), (3, 4)])
def test_mask_from_codes_brute_force(n, m):
    rng = np.random.default_rng([201, n, m])
    pool = f32_to_bf16_bits(np.array([0.0, 0.001, -0.002, 0.01, -0.02, 0.03, -0.05], np.float32))
    bits = rng.choice(pool, size=(5, 4 * m)).astype(np.uint16)
    beta, keep, codes = O.quant_weights(bits, n, m, O.MASK_FROM_CODES)
    assert beta == O.absmean_beta(bits)
    w = O.bf16_to_f32(bits).astype(np.float64)
    c_all = np.array([[_roundclip(v, beta) for v in row] for row in w], np.int8)
    for r in range(5):
        for g in range(4):
            sl = slice(g * m, (g + 1) * m)
            want = _brute_top_n([abs(int(v)) for v in c_all[r, sl]], n)
            assert np.array_equal(keep[r, sl], want), (r, g)
            assert np.array_equal(codes[r, sl], c_all[r, sl] * want)
            # as many nonzero codes as the group allows
            assert np.count_nonzero(codes[r, sl]) == min(n, np.count_nonzero(c_all[r, sl]))


def test_orders_agree_without_ties_or_drops():
    """With n == m nothing is dropped: all three orders give the method's result."""
    rng = np.random.default_rng(202)
    bits = f32_to_bf16_bits((rng.standard_normal((8, 64)) * 0.02).astype(np.float32))
    ref = O.quant_weights(bits, 8, 8)
    for order in (O.MASK_THEN_QUANT, O.MASK_FROM_CODES):
        beta, keep, codes = O.quant_weights(bits, 8, 8, order)
        assert beta == ref[0] and np.array_equal(keep, ref[1]) and np.array_equal(codes, ref[2])


def test_unknown_order_rejected():
    with pytest.raises(ValueError):
        O.quant_weights(_row(HAND), 6, 8, "mask_then_mask")
