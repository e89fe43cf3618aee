"""Pins for the oracle's group scales: one exact absmean beta per block of
consecutive output rows ([BN-cpp] "Cuantizacion y normalizacion de grupos").

Independent routes: one group is the per-matrix method; every group equals
the per-matrix method on its own rows (the per-matrix oracle is pinned
elsewhere); closed-form betas on constant-magnitude rows; locality (changing
one group's masters changes only that group); the grouped rescale against
an exact-Fraction evaluation of its two roundings."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import sbl_oracle as O


def test_one_group_is_the_method():
    rng = np.random.default_rng(400)
    bits = synth.gaussian_masters(rng, 40, 128)
    betas, keep, codes = O.quant_weights_grouped(bits, 6, 8, 40)
    beta, keep1, codes1 = O.quant_weights(bits, 6, 8)
    assert betas.tolist() == [beta] and np.array_equal(keep, keep1) and np.array_equal(codes, codes1)
    betas, _, _ = O.quant_weights_grouped(bits, 6, 8, 1000)      # a group larger than the matrix
    assert betas.tolist() == [beta]


@pytest.mark.parametrize("rpg", [1, 3, 16, 25])
def test_each_group_is_the_method_on_its_rows(rpg):
    rng = np.random.default_rng([401, rpg])
    bits = synth.gaussian_masters(rng, 50, 64, outlier_frac=0.02)
    betas, keep, codes = O.quant_weights_grouped(bits, 2, 4, rpg)
    assert len(betas) == -(-50 // rpg)
    for g, r0 in enumerate(range(0, 50, rpg)):
        sl = slice(r0, min(50, r0 + rpg))
        b, k1, c1 = O.quant_weights(bits[sl], 2, 4)
        assert betas[g] == b and np.array_equal(keep[sl], k1) and np.array_equal(codes[sl], c1)


def test_closed_form_constant_rows():
    """Rows of group g all hold magnitude a_g (signs alternate): beta_g = a_g, and
    every kept code is +-1 (|w| = beta > beta/2)."""
    mags = [0.015625, 0.25, 0.0078125]
    rows = []
    for a in mags:
        for _ in range(4):
            rows.append(np.where(np.arange(64) % 2 == 0, a, -a))
    bits = synth.f32_to_bf16_bits(np.array(rows, np.float32))
    betas, keep, codes = O.quant_weights_grouped(bits, 6, 8, 4)
    assert betas.tolist() == mags
    assert np.all(np.abs(codes[keep]) == 1) and np.all(codes[~keep] == 0)


def test_groups_are_local():
    rng = np.random.default_rng(402)
    bits = synth.gaussian_masters(rng, 24, 128)
    b0, _, c0 = O.quant_weights_grouped(bits, 6, 8, 8)
    bits2 = bits.copy()
    bits2[8:16] = synth.gaussian_masters(rng, 8, 128, sigma=0.5)
    b1, _, c1 = O.quant_weights_grouped(bits2, 6, 8, 8)
    assert b0[0] == b1[0] and b0[2] == b1[2] and b0[1] != b1[1]
    assert np.array_equal(c0[:8], c1[:8]) and np.array_equal(c0[16:], c1[16:])


def test_rescale_grouped_two_roundings():
    rng = np.random.default_rng(403)
    acc = rng.integers(-40000, 40000, (3, 10)).astype(np.int32)
    betas = np.array([0.0113, 0.0207, 0.0042, 3e-6], np.float32)   # the last one below the floor
    gamma = np.array([1.7, 0.0, 250.0], np.float32)
    y = O.rescale_grouped(acc, betas, 3, gamma)

    def rn32(fr):
        return Fraction(float(np.float32(float(fr))))   # exact for the values that arise here

    for t in range(3):
        g = Fraction(float(max(np.float32(gamma[t]), np.float32(1e-5))))
        for r in range(10):
            b = Fraction(float(max(np.float32(betas[r // 3]), np.float32(1e-5))))
            s = rn32(rn32(b * g) / 128)
            want = np.float32(float(Fraction(int(acc[t, r])) * s))
            assert y[t, r] == want
    # one group: the per-matrix rescale
    assert np.array_equal(O.rescale_grouped(acc, betas[:1], 10, gamma), O.rescale(acc, betas[0], gamma))


def test_kgroups_one_group_is_the_method():
    rng = np.random.default_rng(404)
    bits = synth.gaussian_masters(rng, 24, 192)
    x = synth.gaussian_acts(rng, 3, 192, hot_channels=2)
    beta, keep, codes = O.quant_weights(bits, 6, 8)
    q1, g1 = O.quant_acts(x)
    q, g = O.quant_acts_kgrouped(x, 192)
    assert np.array_equal(q, q1) and np.array_equal(g[:, 0], g1)
    acc, y = O.linear_kgrouped(codes, q, np.array([beta]), 24, g, 192)
    a1, y1 = O.linear(codes, q1, beta, g1)
    assert np.array_equal(acc[:, :, 0], a1) and np.array_equal(y, y1)


def test_kgroups_blocks_are_independent_quantizations():
    """Each feature block is the per-token quantizer on that block alone; a hot
    channel only coarsens its own block; the block products add up to the
    whole-row product when gamma is the same everywhere."""
    rng = np.random.default_rng(405)
    x = synth.gaussian_acts(rng, 4, 256)
    x[:, 70] = 100.0                                     # a hot channel in block 1 of 4 (kg = 64)
    q, g = O.quant_acts_kgrouped(x, 64)
    for j in range(4):
        qj, gj = O.quant_acts(x[:, 64 * j:64 * (j + 1)])
        assert np.array_equal(q[:, 64 * j:64 * (j + 1)], qj) and np.array_equal(g[:, j], gj)
    assert np.all(g[:, 1] > 10 * g[:, 0])
    bits = synth.gaussian_masters(rng, 16, 256)
    beta, keep, codes = O.quant_weights(bits, 6, 8)
    acc, _ = O.linear_kgrouped(codes, q, np.array([beta]), 16, g, 64)
    assert np.array_equal(acc.sum(axis=2), O.contract(codes, q))


def test_kgroups_sum_in_block_order():
    """y is the fp32 sum of the blocks' rescaled products in ascending order,
    checked by a direct loop with Fraction-exact per-block terms."""
    from fractions import Fraction
    rng = np.random.default_rng(406)
    bits = synth.gaussian_masters(rng, 8, 192)
    x = synth.gaussian_acts(rng, 2, 192)
    betas, keep, codes = O.quant_weights_grouped(bits, 2, 4, 3)
    q, g = O.quant_acts_kgrouped(x, 64)
    acc, y = O.linear_kgrouped(codes, q, betas, 3, g, 64)
    for t in range(2):
        for r in range(8):
            tot = np.float32(0)
            b = Fraction(float(max(np.float32(betas[r // 3]), np.float32(1e-5))))
            for j in range(3):
                gj = Fraction(float(max(np.float32(g[t, j]), np.float32(1e-5))))
                s = Fraction(float(np.float32(float(b * gj)))) / 128
                term = np.float32(float(Fraction(int(acc[t, r, j])) * s))
                tot = np.float32(tot + term)
            assert y[t, r] == tot


# ---- block scales: one beta per block of rows x features ----

def test_blocks_spanning_k_are_the_row_groups():
    rng = np.random.default_rng(407)
    bits = synth.gaussian_masters(rng, 30, 256, outlier_frac=0.02)
    for rpg in (1, 7, 30):
        b2, keep2, c2 = O.quant_weights_blocked(bits, 6, 8, rpg, 256)
        b1, keep1, c1 = O.quant_weights_grouped(bits, 6, 8, rpg)
        assert b2.shape == (len(b1), 1) and np.array_equal(b2[:, 0], b1)
        assert np.array_equal(keep2, keep1) and np.array_equal(c2, c1)


@pytest.mark.parametrize("rpg,cpg,n,m", [(1, 64, 6, 8), (5, 128, 2, 4), (16, 192, 6, 8), (40, 64, 5, 8)])
def test_each_block_is_the_method_on_its_submatrix(rpg, cpg, n, m):
    """Every block's beta, mask and codes equal the per-matrix method run on the
    block's masters alone (m divides cpg, so the mask's groups never straddle a
    block edge)."""
    rng = np.random.default_rng([408, rpg, cpg, n, m])
    bits = synth.gaussian_masters(rng, 37, 384, outlier_frac=0.02)
    betas, keep, codes = O.quant_weights_blocked(bits, n, m, rpg, cpg)
    assert betas.shape == (-(-37 // rpg), 384 // cpg)
    for gi, r0 in enumerate(range(0, 37, rpg)):
        for gj, c0 in enumerate(range(0, 384, cpg)):
            blk = (slice(r0, min(37, r0 + rpg)), slice(c0, c0 + cpg))
            b, k1, c1 = O.quant_weights(bits[blk], n, m)
            assert betas[gi, gj] == b
            assert np.array_equal(keep[blk], k1) and np.array_equal(codes[blk], c1)


def test_blocks_closed_form_and_locality():
    """Constant-magnitude blocks have beta = that magnitude; changing one
    block's masters changes only that block's beta and codes."""
    mags = np.array([[0.015625, 0.25], [0.0078125, 2.0]], np.float32)
    w = np.zeros((4, 128), np.float32)
    for gi in range(2):
        for gj in range(2):
            w[2 * gi:2 * gi + 2, 64 * gj:64 * gj + 64] = mags[gi, gj]
    w[:, ::2] *= -1
    betas, keep, codes = O.quant_weights_blocked(synth.f32_to_bf16_bits(w), 6, 8, 2, 64)
    assert np.array_equal(betas, mags)
    assert np.all(np.abs(codes[keep]) == 1) and np.all(codes[~keep] == 0)
    rng = np.random.default_rng(409)
    bits = synth.gaussian_masters(rng, 8, 256)
    b0, _, c0 = O.quant_weights_blocked(bits, 6, 8, 4, 128)
    bits2 = bits.copy()
    bits2[4:8, 128:] = synth.gaussian_masters(rng, 4, 128, sigma=0.5)
    b1, _, c1 = O.quant_weights_blocked(bits2, 6, 8, 4, 128)
    changed = b0 != b1
    assert changed[1, 1] and changed.sum() == 1
    assert np.array_equal(c0[:4], c1[:4]) and np.array_equal(c0[4:, :128], c1[4:, :128])


def test_block_scales_in_the_product():
    """With one beta per (row group, feature block): a beta table constant along
    the feature blocks gives the row-group product; otherwise every block's
    term uses its own beta (Fraction-exact terms, fp32 sum in block order)."""
    rng = np.random.default_rng(410)
    bits = synth.gaussian_masters(rng, 9, 192)
    x = synth.gaussian_acts(rng, 2, 192, hot_channels=1)
    q, g = O.quant_acts_kgrouped(x, 64)
    rb, keep, codes = O.quant_weights_grouped(bits, 6, 8, 4)
    acc1, y1 = O.linear_kgrouped(codes, q, rb, 4, g, 64)
    acc2, y2 = O.linear_kgrouped(codes, q, np.repeat(rb[:, None], 3, axis=1), 4, g, 64)
    assert np.array_equal(acc1, acc2) and np.array_equal(y1, y2)
    betas, keep, codes = O.quant_weights_blocked(bits, 6, 8, 4, 64)
    acc, y = O.linear_kgrouped(codes, q, betas, 4, g, 64)
    assert np.array_equal(acc.sum(axis=2), O.contract(codes, q))
    for t in range(2):
        for r in range(9):
            tot = np.float32(0)
            for j in range(3):
                b = Fraction(float(max(np.float32(betas[r // 4, j]), np.float32(1e-5))))
                gj = Fraction(float(max(np.float32(g[t, j]), np.float32(1e-5))))
                s = Fraction(float(np.float32(float(b * gj)))) / 128
                tot = np.float32(tot + np.float32(float(Fraction(int(acc[t, r, j])) * s)))
            assert y[t, r] == tot
    with pytest.raises(ValueError):
        O.linear_kgrouped(codes, q, betas[:, :2], 4, g, 64)
