"""Pins for the oracle's activation quantizer, contraction, rescale, and the
hand-derived worked example (tests/golden/worked_example_k16.txt)."""

import os
from fractions import Fraction

import numpy as np

from oracle import sbl_oracle as O
from synth import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_k16.txt")


def _load_golden():
    d = {}
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            d[key.strip()] = val.split()
    return d


def test_worked_example_end_to_end():
    g = _load_golden()
    w = np.array([float(v) / 256 for v in g["w_times_256"]], np.float32).reshape(1, 16)
    bits = f32_to_bf16_bits(w)
    assert np.array_equal(O.bf16_to_f32(bits), w)          # exact in BF16
    beta, keep, codes = O.quant_weights(bits, 6, 8)
    assert Fraction(float(beta)) == Fraction(g["beta"][0])
    assert O.ternarize(bits, beta)[0].tolist() == [int(v) for v in g["codes_unmasked"]]
    assert O.pack_bitmap(keep)[0].tolist() == [int(h, 16) for h in g["keep_bitmap_hex"]]
    assert codes[0].tolist() == [int(v) for v in g["codes_masked"]]
    assert O.pack_dense2(codes)[0].tolist() == [int(h, 16) for h in g["dense2_hex"]]
    assert O.pack_nm(codes, keep, 6, 8)[0].tolist() == [int(h, 16) for h in g["nm68_codes_hex"]]
    x = np.array([float(v) for v in g["x"]], np.float32).reshape(1, 16)
    q, gamma = O.quant_acts(x)
    assert gamma[0] == np.float32(g["gamma"][0])
    assert q[0].tolist() == [int(v) for v in g["q"]]
    acc, y = O.linear(codes, q, beta, gamma)
    assert acc[0, 0] == int(g["acc"][0])
    assert O.contract(O.ternarize(bits, beta), q)[0, 0] == int(g["acc_unmasked"][0])
    assert Fraction(float(y[0, 0])) == Fraction(g["y"][0])


def test_quant_acts_against_exact_rationals():
    rng = np.random.default_rng(77)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    x[1, 7] *= 30.0
    x[3] = 0.0
    q, gamma = O.quant_acts(x)
    for t in range(5):
        g = float(np.abs(x[t]).max())
        assert gamma[t] == np.float32(g)
        geff = max(g, float(np.float32(1e-5)))
        for kk in range(96):
            exact = Fraction(128) * Fraction(float(x[t, kk])) / Fraction(geff)
            if abs(exact) >= Fraction(255, 2):
                assert abs(int(q[t, kk])) == 127 and np.sign(q[t, kk]) == np.sign(exact)
            else:
                assert abs(Fraction(int(q[t, kk])) - exact) <= Fraction(1, 2) + abs(exact) * Fraction(1, 1 << 22)
    assert np.all(q[3] == 0) and gamma[3] == 0


def test_quant_acts_ties_and_clamp():
    # gamma = 2 -> q = rint(64 x): 64x = 2.5 -> 2, -1.5 -> -2, 0.5 -> 0, 127.5 -> 127 (clamp 128 -> 127)
    x = np.array([[2.0, 2.5 / 64, -1.5 / 64, 0.5 / 64, 127.5 / 64, -2.0, 1.0 / 64, 3.5 / 64]], np.float32)
    q, gamma = O.quant_acts(x)
    assert gamma[0] == 2.0
    assert q[0].tolist() == [127, 2, -2, 0, 127, -127, 1, 4]


def _brute_contract(codes, q):
    return np.array([[sum(int(a) * int(b) for a, b in zip(codes[r], q[t]))
                      for r in range(codes.shape[0])] for t in range(q.shape[0])], np.int64)


def test_contract_matches_python_ints_non_square():
    rng = np.random.default_rng(88)
    codes = rng.integers(-1, 2, (7, 40)).astype(np.int8)
    q = rng.integers(-127, 128, (3, 40)).astype(np.int8)
    acc = O.contract(codes, q)
    assert acc.shape == (3, 7)
    assert np.array_equal(acc, _brute_contract(codes, q))
    # the extreme magnitude 127*k is exact
    k = 8192
    acc = O.contract(np.ones((1, k), np.int8), np.full((1, k), -127, np.int8))
    assert acc[0, 0] == -127 * k


def test_rescale_against_float64_and_zero():
    rng = np.random.default_rng(99)
    acc = rng.integers(-3_000_000, 3_000_000, (4, 50)).astype(np.int32)
    acc[0, :5] = 0
    beta = np.float32(0.0159)
    gamma = (rng.random(4) * 40).astype(np.float32)
    gamma[2] = 0.0
    y = O.rescale(acc, beta, gamma)
    geff = np.maximum(gamma.astype(np.float64), float(np.float32(1e-5)))
    ref = acc.astype(np.float64) * float(beta) * geff[:, None] / 128.0
    nz = acc != 0
    assert np.all(np.abs(y[nz] / ref[nz] - 1) < 2.0 ** -22)
    assert np.all(y[~nz] == 0)


def test_forward_equals_dequantized_float_matmul():
    # integer result == brute-force dequantized float matmul on tiny inputs
    rng = np.random.default_rng(111)
    bits = f32_to_bf16_bits(rng.standard_normal((6, 64)).astype(np.float32) * np.float32(0.02))
    x = rng.standard_normal((3, 64)).astype(np.float32)
    out = O.forward(bits, x, 6, 8)
    w_deq = out["codes"].astype(np.float64) * float(O.beta_eff(out["beta"]))
    x_deq = out["q"].astype(np.float64) * (np.maximum(out["gamma"], 1e-5)[:, None].astype(np.float64) / 128.0)
    ref = x_deq @ w_deq.T
    # exact integer zeros come out as tiny float64 cancellation residues in ref
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-12)
    assert np.all(out["y"][out["acc"] == 0] == 0)
