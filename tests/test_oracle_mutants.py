"""The oracle's pins catch plausible mistakes.

Each case swaps one oracle function for a deliberately wrong variant (a
dropped term, a wrong sign, index or rounding rule, a transposed operand, a
changed byte layout), runs the pins that cover that step, and requires at
least one of them to fail.  The mistakes are planted in the oracle, on the
CPU; nothing here touches the HIP library.
"""

from fractions import Fraction

import numpy as np
import pytest

import test_oracle_ablations as AB
import test_oracle_acts_linear as A
import test_oracle_backward as B
import test_oracle_grouped as G
import test_oracle_scales as S
import test_oracle_weights as W
from oracle import sbl_oracle as O


def _ties_to_higher_index(orig):
    def top_n_keep(mag, n, m):
        mag = np.asarray(mag)
        n_out, k = mag.shape
        a = mag.reshape(n_out, k // m, m)
        idx = np.arange(m)
        higher = idx[None, :] > idx[:, None]              # the mistake: i > j wins ties
        rank = (a[..., None, :] > a[..., :, None]).sum(-1) + \
            ((a[..., None, :] == a[..., :, None]) & higher).sum(-1)
        return (rank < n).reshape(n_out, k)
    return top_n_keep


def _mask_from_codes(orig):
    return lambda bits, n, m, order=O.QUANT_THEN_MASK: orig(bits, n, m, O.MASK_FROM_CODES)


def _absmean_doubled(orig):
    return lambda bits, keep=None: orig(bits, keep) * 2


def _mean_of_signed_w(orig):
    def absmean_exact(bits, keep=None):
        w = O.bf16_to_f32(np.asarray(bits, np.uint16).ravel()).astype(np.float64)
        if keep is not None:
            w = w[np.asarray(keep, bool).ravel()]
        return Fraction(float(w.mean()))                   # the mistake: no |.|
    return absmean_exact


def _round_half_away(orig):
    def ternarize(bits, beta):
        w = O.bf16_to_f32(bits).astype(np.float64)
        r = w / np.float64(O.beta_eff(beta))
        return np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -1, 1).astype(np.int8)
    return ternarize


def _no_beta_floor(orig):
    def ternarize(bits, beta):
        w = O.bf16_to_f32(bits).astype(np.float64)
        return np.clip(np.rint(w / np.float64(beta)), -1, 1).astype(np.int8)
    return ternarize


def _quant_acts_variant(signed_max=False, qb=128, lo=-127):
    def make(orig):
        def quant_acts(x):
            x = np.asarray(x, np.float32)
            gamma = (x.max(axis=1) if signed_max else np.abs(x).max(axis=1)).astype(np.float32)
            s = (np.maximum(gamma, np.float32(1e-5)) / np.float32(qb)).astype(np.float32)
            t = (x / s[:, None]).astype(np.float32)
            return np.clip(np.rint(t), lo, 127).astype(np.int8), gamma
        return quant_acts
    return make


def _contract_drops_last_k(orig):
    return lambda codes, q: orig(np.asarray(codes)[:, :-1], np.asarray(q)[:, :-1])


def _contract_transposed(orig):
    return lambda codes, q: orig(codes, q).T


def _rescale_without_2_pow_minus_7(orig):
    return lambda acc, beta, gamma: (orig(acc, beta, gamma) * np.float32(128)).astype(np.float32)


def _rescale_without_gamma_floor(orig):
    def rescale(acc, beta, gamma):
        s = ((O.beta_eff(beta) * np.asarray(gamma, np.float32)).astype(np.float32) / np.float32(128))
        return (np.asarray(acc).astype(np.float32) * s.astype(np.float32)[:, None]).astype(np.float32)
    return rescale


def _bitmap_msb_first(orig):
    def pack_bitmap(keep):
        kp = np.asarray(keep, bool)
        n_out, k = kp.shape
        return np.packbits(kp.reshape(n_out, k // 8, 8), axis=-1, bitorder="big").reshape(n_out, k // 8)
    return pack_bitmap


def _dense2_twos_complement(orig):
    def pack_dense2(codes):
        c = np.asarray(codes, np.int8)
        n_out, k = c.shape
        u = (c.astype(np.int16) & 3).astype(np.uint8)       # the mistake: u = c mod 4, not c + 1
        out = np.zeros((n_out, k // 4), np.uint8)
        for kk in range(16):
            out[:, 4 * np.arange(k // 16) + kk % 4] |= (u[:, kk::16] << (2 * (kk // 4))).astype(np.uint8)
        return out
    return pack_dense2


def _rational_toward_zero(orig):
    def rational_to_f32(num, den):
        v = orig(num, den)
        if np.isfinite(v) and Fraction(float(v)) > Fraction(num, den):
            v = np.nextafter(v, np.float32(0))              # the mistake: truncation
        return np.float32(v)
    return rational_to_f32


def _nm_fields_reversed(orig):
    def pack_nm(codes, keep, n, m):
        b = orig(codes, keep, n, m)
        out = np.zeros_like(b)
        for s in range(4):                                  # kept codes in descending order
            out |= (((b >> (2 * s)) & 3) << (2 * (3 - s))).astype(np.uint8)
        return out
    return pack_nm


def _clip_pass_off_by_one(orig):
    def clip_pass(x, gamma):
        x = np.asarray(x, np.float32)
        s = (np.maximum(np.asarray(gamma, np.float32), np.float32(1e-5)) / np.float32(128)).astype(np.float32)
        t = np.rint((x / s[:, None]).astype(np.float32))
        return (np.abs(t) <= 128).astype(np.float64)
    return clip_pass


def _backward_without_clip(orig):
    return lambda codes, beta, x, q, gamma, dy_bits, clip=True: orig(codes, beta, x, q, gamma, dy_bits, clip=False)


def _dw_only_through_nonzero_codes(orig):
    def backward(codes, beta, x, q, gamma, dy_bits, clip=True):
        r = orig(codes, beta, x, q, gamma, dy_bits, clip)
        r["dw"] = r["dw"] * (np.asarray(codes) != 0)
        return r
    return backward


def _dequant_without_2_pow_minus_7(orig):
    return lambda q, gamma: (orig(q, gamma) * np.float32(128)).astype(np.float32)


def _row_groups_one_too_large(orig):
    return lambda bits, n, m, rows_per_group: orig(bits, n, m, rows_per_group + 1)


def _row_group_scales_reversed(orig):
    return lambda acc, betas, rows_per_group, gamma: orig(acc, np.asarray(betas)[::-1], rows_per_group, gamma)


def _one_gamma_per_token(orig):
    def quant_acts_kgrouped(x, kg):
        q, g = O.quant_acts(x)
        return q, np.repeat(g[:, None], np.asarray(x).shape[1] // kg, axis=1)
    return quant_acts_kgrouped


def _blocks_added_descending(orig):
    def linear_kgrouped(codes, q, betas, rows_per_group, gamma, kg):
        def rev(a):                                          # feature blocks in reverse order
            a = np.asarray(a)
            return a.reshape(a.shape[0], -1, kg)[:, ::-1].reshape(a.shape)
        b = np.asarray(betas)
        acc, y = orig(rev(codes), rev(q), b if b.ndim == 1 else b[:, ::-1], rows_per_group,
                      np.asarray(gamma)[:, ::-1], kg)
        return acc[:, :, ::-1], y
    return linear_kgrouped


def _mask_then_quant_beta_over_all(orig):
    def quant_weights(bits, n, m, order=O.QUANT_THEN_MASK):
        if order == O.MASK_THEN_QUANT:                     # the mistake: beta over every master
            beta, keep, _ = orig(bits, n, m, O.QUANT_THEN_MASK)
            return beta, keep, (O.ternarize(bits, beta) * keep).astype(np.int8)
        return orig(bits, n, m, order)
    return quant_weights


def _block_beta_over_whole_rows(orig):
    def quant_weights_blocked(bits, n, m, rows_per_group, cols_per_group):
        betas, keep, _ = orig(bits, n, m, rows_per_group, cols_per_group)
        rows, _, _ = O.quant_weights_grouped(bits, n, m, rows_per_group)   # the mistake: beta over the row block
        betas = np.repeat(np.asarray(rows, np.float32)[:, None], betas.shape[1], axis=1)
        codes = np.zeros(np.shape(bits), np.int8)
        for gi in range(betas.shape[0]):
            sl = slice(gi * rows_per_group, (gi + 1) * rows_per_group)
            codes[sl] = O.ternarize(np.asarray(bits)[sl], betas[gi, 0])
        return betas, keep, (codes * keep).astype(np.int8)
    return quant_weights_blocked


MUTANTS = [
    ("mask ties to the higher index", "top_n_keep", _ties_to_higher_index,
     [W.test_mask_ties_prefer_lower_index, lambda: W.test_mask_matches_subset_enumeration(8)]),
    ("mask chosen from the codes, not the masters", "quant_weights", _mask_from_codes,
     [W.test_mask_is_from_master_not_codes, A.test_worked_example_end_to_end]),
    ("absmean off by a factor 2 (exponent offset)", "absmean_exact", _absmean_doubled,
     [S.test_absmean_equals_fraction_sum, W.test_ternarize_tie_at_half_beta_goes_to_zero]),
    ("mean of w instead of |w|", "absmean_exact", _mean_of_signed_w,
     [S.test_beta_gaussian_half_normal_mean, A.test_worked_example_end_to_end]),
    ("RoundClip rounds half away from zero", "ternarize", _round_half_away,
     [W.test_ternarize_tie_at_half_beta_goes_to_zero]),
    ("RoundClip divides by beta without the 1e-5 floor", "ternarize", _no_beta_floor,
     [W.test_ternarize_matches_fraction_roundclip, W.test_ternarize_beta_below_the_floor]),
    ("gamma = max x instead of max |x|", "quant_acts", _quant_acts_variant(signed_max=True),
     [A.test_quant_acts_against_exact_rationals, A.test_worked_example_end_to_end]),
    ("activation scale Qb = 127", "quant_acts", _quant_acts_variant(qb=127),
     [A.test_quant_acts_ties_and_clamp, A.test_quant_acts_against_exact_rationals]),
    ("activations clipped to -128", "quant_acts", _quant_acts_variant(lo=-128),
     [A.test_quant_acts_ties_and_clamp]),
    ("contraction drops the last k", "contract", _contract_drops_last_k,
     [A.test_contract_matches_python_ints_non_square]),
    ("contraction result transposed", "contract", _contract_transposed,
     [A.test_contract_matches_python_ints_non_square, A.test_worked_example_end_to_end]),
    ("rescale without the 2^-7", "rescale", _rescale_without_2_pow_minus_7,
     [A.test_rescale_against_float64_and_zero, A.test_forward_equals_dequantized_float_matmul]),
    ("rescale without the gamma floor", "rescale", _rescale_without_gamma_floor,
     [A.test_rescale_against_float64_and_zero]),
    ("bitmap bits most significant first", "pack_bitmap", _bitmap_msb_first,
     [W.test_pack_round_trips, A.test_worked_example_end_to_end]),
    ("DENSE2 stores c mod 4 instead of c + 1", "pack_dense2", _dense2_twos_complement,
     [W.test_pack_round_trips, A.test_worked_example_end_to_end]),
    ("fp32 rounding of beta toward zero", "rational_to_f32", _rational_toward_zero,
     [S.test_rational_to_f32_matches_neighbour_search, S.test_rational_to_f32_midpoints_go_to_even]),
    ("N:M codes stored in descending k", "pack_nm", _nm_fields_reversed,
     [W.test_pack_round_trips, A.test_worked_example_end_to_end]),
    ("activation clip test off by one", "clip_pass", _clip_pass_off_by_one,
     [B.test_clip_pass_crafted]),
    ("dX without the quantizer's clip mask", "backward", _backward_without_clip,
     [B.test_brute_force_fractions, B.test_single_token_single_output]),
    ("dW only through nonzero codes", "backward", _dw_only_through_nonzero_codes,
     [B.test_mask_ste_reaches_pruned_masters, B.test_brute_force_fractions]),
    ("x_hat without the 2^-7", "dequant_acts", _dequant_without_2_pow_minus_7,
     [B.test_dequant_is_the_scaled_code]),
    ("row groups one row too large", "quant_weights_grouped", _row_groups_one_too_large,
     [lambda: G.test_each_group_is_the_method_on_its_rows(3), G.test_closed_form_constant_rows]),
    ("row-group scales applied in reverse", "rescale_grouped", _row_group_scales_reversed,
     [G.test_rescale_grouped_two_roundings]),
    ("one gamma per token instead of per feature block", "quant_acts_kgrouped", _one_gamma_per_token,
     [G.test_kgroups_blocks_are_independent_quantizations]),
    ("feature blocks added in descending order", "linear_kgrouped", _blocks_added_descending,
     [G.test_kgroups_sum_in_block_order]),
    ("panels two blocks wide instead of four", "PANEL_BLOCKS", lambda orig: 2,
     [W.test_panel_order_hand_example, W.test_panel_order_per_byte_and_inverse]),
    ("mask-then-quant ablation with beta over every master", "quant_weights", _mask_then_quant_beta_over_all,
     [AB.test_hand_example_three_orders, lambda: AB.test_mask_then_quant_brute_force(6, 8)]),
    ("block scales taken over whole row blocks", "quant_weights_blocked", _block_beta_over_whole_rows,
     [lambda: G.test_each_block_is_the_method_on_its_submatrix(16, 192, 6, 8), G.test_blocks_closed_form_and_locality]),
]


@pytest.mark.parametrize("name,attr,make,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, attr, make, pins):
    for pin in pins:                                   # the pins hold for the oracle as it is
        pin()
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    failed = []
    for pin in pins:
        try:
            pin()
        except Exception:                              # an assertion, or a shape or value error
            failed.append(getattr(pin, "__name__", "pin"))
    assert failed, f"no pin caught: {name}"
