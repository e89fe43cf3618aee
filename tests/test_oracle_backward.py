"""Pins for the oracle's backward (dual straight-through estimator: identity
through the quantizers inside the clipping range, dense gradient to every
master through the mask).

Independent routes: exact-Fraction loops over the definition on tiny shapes,
the adjoint identities that tie the two gradients to the forward product
(<dY, Y> = <beta C, dW> = <x_hat, dX> without the clip), crafted clip cases
decided in exact arithmetic, and the dense-gradient property at pruned
positions."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import sbl_oracle as O


def _setup(seed, t, n_out, k, n=6, m=8):
    rng = np.random.default_rng(seed)
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, t, k)
    beta, keep, codes = O.quant_weights(bits, n, m)
    q, gamma = O.quant_acts(x)
    dy = synth.f32_to_bf16_bits(rng.standard_normal((t, n_out)).astype(np.float32))
    return bits, x, beta, keep, codes, q, gamma, dy


def test_brute_force_fractions():
    bits, x, beta, keep, codes, q, gamma, dy = _setup(300, 3, 5, 64)
    r = O.backward(codes, beta, x, q, gamma, dy)
    b = Fraction(float(max(np.float32(beta), np.float32(1e-5))))
    dyf = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f32(dy)]
    xh = [[Fraction(float(np.float32(max(np.float32(g), np.float32(1e-5)) * np.float32(v)))) / 128 for v in row]
          for g, row in zip(gamma, q)]
    for t in range(3):
        for kk in range(64):
            s = sum(dyf[t][nn] * int(codes[nn, kk]) for nn in range(5))
            want = b * s * int(r["clip"][t, kk])
            assert Fraction(r["dx"][t, kk]) == want or abs(Fraction(r["dx"][t, kk]) - want) <= abs(want) * Fraction(1, 1 << 50)
    for nn in range(5):
        for kk in range(64):
            want = sum(dyf[t][nn] * xh[t][kk] for t in range(3))
            assert abs(Fraction(r["dw"][nn, kk]) - want) <= abs(want) * Fraction(1, 1 << 50) + Fraction(1, 1 << 80)


def test_adjoint_identities():
    """The STE gradients are the adjoints of the forward product in real terms:
    Y[t, n] = sum_k beta C[n, k] x_hat[t, k]."""
    bits, x, beta, keep, codes, q, gamma, dy = _setup(301, 7, 48, 256)
    r = O.backward(codes, beta, x, q, gamma, dy, clip=False)
    b = float(O.beta_eff(beta))
    xh = O.dequant_acts(q, gamma).astype(np.float64)
    dyf = O.bf16_to_f32(dy).astype(np.float64)
    y = np.einsum("nk,tk->tn", b * codes.astype(np.float64), xh)
    lhs = float(np.sum(dyf * y))
    assert np.isclose(lhs, float(np.sum(b * codes * r["dw"])), rtol=1e-12, atol=1e-12)
    assert np.isclose(lhs, float(np.sum(xh * r["dx"])), rtol=1e-12, atol=1e-12)


def test_dequant_is_the_scaled_code():
    _, x, _, _, _, q, gamma, _ = _setup(302, 4, 8, 128)
    xh = O.dequant_acts(q, gamma)
    for t in range(4):
        g = Fraction(float(max(np.float32(gamma[t]), np.float32(1e-5))))
        for kk in range(0, 128, 7):
            exact = g * int(q[t, kk]) / 128
            assert abs(Fraction(float(xh[t, kk])) - exact) <= abs(exact) * Fraction(1, 1 << 24)
    # and it approximates x within half a quantization step (unclamped entries)
    step = np.maximum(gamma, 1e-5)[:, None] / 128
    ok = O.clip_pass(x, gamma) > 0
    assert np.all(np.abs(xh - x)[ok] <= 0.5 * np.broadcast_to(step, x.shape)[ok] * (1 + 1e-6))


def test_clip_pass_crafted():
    """128 |x| / gamma = 126, 127, 127.4 pass; 127.6 and 128 (the row's max)
    are clamped; decided in exact arithmetic, far from any fp32 rounding."""
    gamma = np.float32(2.0)
    vals = np.array([126, 127, 127.4, 127.6, 128, -127.4, -127.6, 0.0, 3.0], np.float64) * 2.0 / 128
    x = vals.astype(np.float32)[None, :]
    got = O.clip_pass(x, np.array([gamma]))[0]
    assert got.tolist() == [1, 1, 1, 0, 0, 1, 0, 1, 1]
    # the quantizer agrees: a passing entry is not at the clamp bound unless it is exactly 127
    q, g = O.quant_acts(x)
    assert g[0] == gamma
    assert q[0].tolist()[:5] == [126, 127, 127, 127, 127]


def test_mask_ste_reaches_pruned_masters():
    bits, x, beta, keep, codes, q, gamma, dy = _setup(303, 5, 16, 128)
    r = O.backward(codes, beta, x, q, gamma, dy)
    pruned = ~keep
    assert pruned.any()
    assert np.count_nonzero(r["dw"][pruned]) == pruned.sum()    # Gaussian data: no exact zeros
    # dW does not depend on the mask or on the codes at all
    r2 = O.backward(np.zeros_like(codes), beta, x, q, gamma, dy)
    assert np.array_equal(r["dw"], r2["dw"])
    # while dX sees only the masked codes: pruned positions contribute nothing
    c_full = O.ternarize(bits, beta)
    r3 = O.backward(c_full, beta, x, q, gamma, dy)
    assert not np.allclose(r["dx"], r3["dx"])


def test_single_token_single_output():
    """t = n_out = 1: dX = beta dy c (clip-masked) and dW = dy x_hat."""
    rng = np.random.default_rng(304)
    codes = rng.integers(-1, 2, (1, 64)).astype(np.int8)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    q, gamma = O.quant_acts(x)
    dy = synth.f32_to_bf16_bits(np.array([[0.375]], np.float32))
    beta = np.float32(0.0125)
    r = O.backward(codes, beta, x, q, gamma, dy)
    mask = O.clip_pass(x, gamma)[0]
    assert mask.sum() == 63                                  # the max entry is clamped
    assert np.array_equal(r["dx"][0], float(beta) * 0.375 * codes[0] * mask)
    assert np.array_equal(r["dw"][0], 0.375 * O.dequant_acts(q, gamma)[0].astype(np.float64))


def test_bounds_cover_the_fp32_sum():
    """An fp32 sum in the worst (sequential) order stays inside the bound."""
    bits, x, beta, keep, codes, q, gamma, dy = _setup(305, 4, 200, 64)
    r = O.backward(codes, beta, x, q, gamma, dy, clip=False)
    dyf = O.bf16_to_f32(dy)
    b = np.float32(O.beta_eff(beta))
    for t in range(4):
        for kk in range(0, 64, 9):
            acc = np.float32(0)
            for nn in range(200):
                acc = np.float32(acc + np.float32(dyf[t, nn] * np.float32(codes[nn, kk])))
            got = float(np.float32(b * acc))
            assert abs(got - r["dx"][t, kk]) <= r["dx_bound"][t, kk]


def test_rejects_bad_input():
    bits, x, beta, keep, codes, q, gamma, dy = _setup(306, 2, 8, 64)
    with pytest.raises(ValueError):
        O.backward(codes, beta, x, q, gamma, dy[:, :4])
    bad = dy.copy()
    bad[0, 0] = 0x7F80                                        # +inf
    with pytest.raises(ValueError):
        O.backward(codes, beta, x, q, gamma, bad)
