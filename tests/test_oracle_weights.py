"""Pins for the oracle's ternary codes, N:M masks and byte formats.

Independent routes: exact-Fraction RoundClip, enumeration of every C(m, n)
subset, invariants that the pages fix (ternary codes, at most n nonzeros per
group, exactly n kept, mask chosen from the master weights), closed-form zero
fractions for Gaussian masters, and the hand-derived 16-weight example.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import sbl_oracle as O
from synth import f32_to_bf16_bits


def _roundclip_fraction(w: float, beta: float) -> int:
    r = Fraction(w) / Fraction(float(max(np.float32(beta), np.float32(1e-5))))
    return max(-1, min(1, round(r)))       # Fraction.__round__ is half-to-even


def test_ternarize_matches_fraction_roundclip():
    rng = np.random.default_rng(5)
    w = rng.standard_normal(4000).astype(np.float32) * np.float32(0.02)
    bits = f32_to_bf16_bits(w)
    vals = O.bf16_to_f32(bits)
    for beta in [np.float32(0.016), O.absmean_beta(bits), np.float32(2.0e-6), np.float32(0.04)]:
        got = O.ternarize(bits, beta)
        want = np.array([_roundclip_fraction(float(v), beta) for v in vals], np.int8)
        assert np.array_equal(got, want)


def test_ternarize_tie_at_half_beta_goes_to_zero():
    # magnitudes {a, 3a} in equal numbers: beta = 2a, so |w| = a is exactly
    # beta/2 (RoundClip(1/2) = 0) and 3a maps to sign(w)
    a = np.float32(0.0078125)
    vals = np.array([a, -a, 3 * a, -3 * a] * 4, np.float32)
    bits = f32_to_bf16_bits(vals)
    beta = O.absmean_beta(bits)
    assert beta == np.float32(2 * a)
    assert O.ternarize(bits, beta).tolist() == [0, 0, 1, -1] * 4


def test_ternarize_beta_below_the_floor():
    # beta below 1e-5 is replaced by 1e-5: |w| ~ 4e-6 lies above beta/2 = 1e-6
    # but below 1e-5/2, so it quantizes to 0; |w| ~ 6e-6 goes to sign(w)
    bits = f32_to_bf16_bits(np.array([4e-6, -4e-6, 6e-6, -6e-6], np.float32))
    beta = np.float32(2e-6)
    got = O.ternarize(bits, beta)
    assert got.tolist() == [0, 0, 1, -1]
    assert got.tolist() == [_roundclip_fraction(float(v), beta) for v in O.bf16_to_f32(bits)]


def test_ternarize_is_monotone_and_ternary():
    rng = np.random.default_rng(9)
    bits = f32_to_bf16_bits(rng.standard_normal(10000).astype(np.float32))
    beta = O.absmean_beta(bits)
    c = O.ternarize(bits, beta)
    assert set(np.unique(c)) <= {-1, 0, 1}
    mag = np.abs(O.bf16_to_f32(bits))
    order = np.argsort(mag, kind="stable")
    assert np.all(np.diff(np.abs(c[order]).astype(int)) >= 0)
    assert np.all((np.sign(O.bf16_to_f32(bits)) * c) >= 0)


def test_ternarize_zero_fraction_gaussian():
    # P(c = 0) = P(|w| <= beta/2) with beta -> sigma*sqrt(2/pi): erf(1/(2*sqrt(pi)))
    rng = np.random.default_rng(21)
    bits = f32_to_bf16_bits(rng.standard_normal(1 << 20).astype(np.float32) * np.float32(0.02))
    c = O.ternarize(bits, O.absmean_beta(bits))
    want = math.erf(1 / (2 * math.sqrt(math.pi)))
    assert abs((c == 0).mean() - want) < 3e-3
    assert abs(want - 0.3101) < 1e-4


def _brute_mask_group(mags, n):
    """Lexicographically first subset (sorted index tuple) of maximum total magnitude."""
    best = None
    for sub in itertools.combinations(range(len(mags)), n):
        s = sum(Fraction(float(mags[i])) for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    keep = np.zeros(len(mags), bool)
    keep[list(best[1])] = True
    return keep


@pytest.mark.parametrize("m", [4, 8])
def test_mask_matches_subset_enumeration(m):
    rng = np.random.default_rng(100 + m)
    for n in range(1, m + 1):
        # few distinct magnitudes -> many ties; signed zeros included
        pool = f32_to_bf16_bits(np.array([0.0, -0.0, 0.01, -0.01, 0.02, 0.5, -0.5], np.float32))
        bits = rng.choice(pool, size=(6, 4 * m)).astype(np.uint16)
        keep = O.nm_keep(bits, n, m)
        mags = np.abs(O.bf16_to_f32(bits))
        for r in range(bits.shape[0]):
            for g in range(4):
                sl = slice(g * m, (g + 1) * m)
                assert np.array_equal(keep[r, sl], _brute_mask_group(mags[r, sl], n)), (n, r, g)


def test_mask_invariants_on_gaussian():
    rng = np.random.default_rng(33)
    bits = f32_to_bf16_bits(rng.standard_normal((64, 512)).astype(np.float32) * np.float32(0.02))
    for n, m in [(6, 8), (2, 4), (3, 8), (8, 8)]:
        keep = O.nm_keep(bits, n, m).reshape(64, -1, m)
        mag = np.abs(O.bf16_to_f32(bits)).reshape(64, -1, m)
        assert np.all(keep.sum(-1) == n)
        if n < m:
            kept_min = np.where(keep, mag, np.inf).min(-1)
            pruned_max = np.where(~keep, mag, -np.inf).max(-1)
            assert np.all(kept_min >= pruned_max)


def test_mask_ties_prefer_lower_index():
    v = f32_to_bf16_bits(np.array([0.5] * 8, np.float32)).reshape(1, 8)
    assert O.nm_keep(v, 6, 8).tolist() == [[True] * 6 + [False] * 2]
    v = f32_to_bf16_bits(np.array([0.1, 0.3, 0.3, 0.2, -0.3, 0.3, 0.0, -0.0], np.float32)).reshape(1, 8)
    # 0.3 (x4, at 1,2,4,5) then 0.2, 0.1: keep 6 = {1,2,4,5,3,0}
    assert O.nm_keep(v, 6, 8)[0].tolist() == [True, True, True, True, True, True, False, False]
    # 2 of 4 in the first half: two 0.3s tie -> positions 1 and 2
    assert O.nm_keep(v, 2, 4)[0].tolist() == [False, True, True, False, True, True, False, False]


def test_mask_is_from_master_not_codes():
    # all four weights quantize to the same code (+1), but the master order decides
    w = np.array([[0.020, 0.030, 0.025, 0.021]], np.float32)
    bits = f32_to_bf16_bits(w)
    beta, keep, codes = O.quant_weights(bits, 2, 4)
    assert keep[0].tolist() == [False, True, True, False]
    assert codes[0].tolist() == [0, 1, 1, 0]


def test_quant_then_mask_invariants():
    rng = np.random.default_rng(44)
    bits = f32_to_bf16_bits(rng.standard_normal((32, 256)).astype(np.float32) * np.float32(0.02))
    for n, m in [(6, 8), (2, 4), (4, 8)]:
        beta, keep, codes = O.quant_weights(bits, n, m)
        full = O.ternarize(bits, beta)
        assert beta == O.absmean_beta(bits)          # beta over all masters, pruned included
        assert np.array_equal(codes[keep], full[keep])
        assert np.all(codes[~keep] == 0)
        nz = (codes != 0).reshape(32, -1, m).sum(-1)
        nz_full = (full != 0).reshape(32, -1, m).sum(-1)
        assert np.all(nz <= n)
        assert np.array_equal(nz, np.minimum(n, nz_full))


def _binomial_zero_fraction(n, m, p):
    e_min = sum(min(n, b) * math.comb(m, b) * p ** b * (1 - p) ** (m - b) for b in range(m + 1))
    return 1 - e_min / m


def test_masked_zero_fraction_closed_forms():
    rng = np.random.default_rng(55)
    bits = f32_to_bf16_bits(rng.standard_normal((512, 2048)).astype(np.float32) * np.float32(0.02))
    p = 1 - math.erf(1 / (2 * math.sqrt(math.pi)))
    for n, m, closed in [(6, 8, 0.3460), (2, 4, 0.5252)]:
        _, _, codes = O.quant_weights(bits, n, m)
        want = _binomial_zero_fraction(n, m, p)
        assert abs(want - closed) < 1e-3
        assert abs((codes == 0).mean() - want) < 3e-3


def test_pack_round_trips():
    rng = np.random.default_rng(66)
    bits = f32_to_bf16_bits(rng.standard_normal((8, 128)).astype(np.float32))
    for n, m in [(6, 8), (2, 4), (8, 8), (5, 8), (4, 4)]:
        beta, keep, codes = O.quant_weights(bits, n, m)
        d2 = O.pack_dense2(codes)
        assert d2.shape == (8, 32)
        assert np.array_equal(O.unpack_dense2(d2, 128), codes)
        bm = O.pack_bitmap(keep)
        assert np.array_equal(O.unpack_bitmap(bm, 128), keep)
        if (128 * n // m) % 4 == 0:
            nm = O.pack_nm(codes, keep, n, m)
            assert nm.shape == (8, 128 * n // m // 4)
            assert np.array_equal(O.unpack_nm(nm, bm, n, m, 128), codes)
        assert not np.any(((d2[..., None] >> np.array([0, 2, 4, 6], np.uint8)) & 3) == 3)


def test_dense2_layout_per_element_and_word_decode():
    # per-element statement of the layout, and the property it is chosen for:
    # (word >> 2s) & 0x03030303 gives u of weights 16b+4s .. 16b+4s+3 in byte order
    rng = np.random.default_rng(67)
    codes = rng.integers(-1, 2, (3, 64)).astype(np.int8)
    p = O.pack_dense2(codes)
    for r in range(3):
        for kk in range(64):
            byte = p[r, 4 * (kk // 16) + kk % 4]
            assert ((int(byte) >> (2 * ((kk // 4) % 4))) & 3) - 1 == codes[r, kk]
        words = p[r].view("<u4")
        for b in range(4):
            for s in range(4):
                d = (int(words[b]) >> (2 * s)) & 0x03030303
                got = [((d >> (8 * j)) & 3) - 1 for j in range(4)]
                assert got == codes[r, 16 * b + 4 * s: 16 * b + 4 * s + 4].tolist()


def test_panel_order_hand_example():
    # 2 rows x 5 blocks of 16 bytes (k = 320, DENSE2): panel 0 = blocks 0..3 of
    # row 0 then of row 1 (64 bytes each), panel 1 = block 4 of row 0, then row 1
    rows = np.arange(160, dtype=np.uint8).reshape(2, 80)
    want = list(range(0, 64)) + list(range(80, 144)) + list(range(64, 80)) + list(range(144, 160))
    assert O.to_panels(rows, 16).tolist() == want


def test_panel_order_per_byte_and_inverse():
    # per-byte statement: byte j of row r (block kb = j // b) sits at
    # n_out * (4b * (kb // 4)) + r * (blocks in that panel) * b + (j - 4b * (kb // 4))
    rng = np.random.default_rng(68)
    for n_out, nkb, b in [(3, 7, 16), (5, 4, 12), (2, 9, 8), (1, 6, 10), (4, 1, 16)]:
        rows = rng.integers(0, 256, (n_out, nkb * b)).astype(np.uint8)
        flat = O.to_panels(rows, b)
        assert flat.size == rows.size
        for r in range(n_out):
            for j in range(nkb * b):
                p = (j // b) // 4
                nb = min(4, nkb - 4 * p)
                assert flat[n_out * 4 * b * p + r * nb * b + (j - 4 * b * p)] == rows[r, j]
        assert np.array_equal(O.from_panels(flat, n_out, nkb * b, b), rows)
        pick = rng.choice(n_out, min(2, n_out), replace=False)
        assert np.array_equal(O.from_panels(flat, n_out, nkb * b, b, rows=pick), rows[pick])
    one = rng.integers(0, 256, (1, 5 * 16)).astype(np.uint8)
    assert np.array_equal(O.to_panels(one, 16), one[0])        # one row: storage = row order
