"""The two weight-preparation variants of the pages' training-design analysis
(Sparse-BitNet summary, section 3, the ablated orders) on the GPU, through
sbl_quant_weights_batch_ex, against the oracle bit for bit:

  * SBL_QW_BETA_KEPT (mask-then-quant): beta averages the masters the n:m
    mask keeps; the mask is the masters' mask.
  * SBL_QW_MASK_FROM_CODES: beta as the method's; each group keeps its n
    largest |code| (ties to the lower index).

Every output (beta, mask bitmap, codes, packed stream, meta) is compared; each
case runs twice on the same workspaces (filled with 0xFF bytes first)."""

import math

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, meta_rows, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

QW_BETA_KEPT, QW_MASK_FROM_CODES = 1, 2
ORDER = {QW_BETA_KEPT: O.MASK_THEN_QUANT, QW_MASK_FROM_CODES: O.MASK_FROM_CODES}
PATTERNS = [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_DENSE2, 5, 8), (FMT_NM, 3, 8),
            (FMT_NM, 7, 8), (FMT_DENSE2, 1, 4), (FMT_NM, 8, 8), (FMT_NM, 3, 4)]


def _item(bits, fmt, n, m, outs=("mask_bits", "codes", "packed")):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = bits.shape
    it = dict(w=to_dev(bits), beta=torch.full((1,), -1.0, device="cuda"), mask_bits=None, codes=None,
              packed=None, meta=None,
              workspace=torch.full((sbl.sbl_workspace_bytes(n_out, k),), 0xFF, dtype=torch.uint8, device="cuda"))
    if "mask_bits" in outs:
        it["mask_bits"] = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    if "codes" in outs:
        it["codes"] = torch.empty((n_out, k), dtype=torch.int8, device="cuda")
    if "packed" in outs:
        it["packed"] = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
        if fmt == FMT_NM:
            it["meta"] = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    return it


def _check(bits, g, fmt, n, m, flag):
    n_out, k = bits.shape
    beta, keep, codes = O.quant_weights(bits, n, m, ORDER[flag])
    assert g["beta"][0] == beta, (bits.shape, g["beta"][0], beta)
    if "mask_bits" in g:
        assert np.array_equal(g["mask_bits"], O.pack_bitmap(keep))
    if "codes" in g:
        assert np.array_equal(g["codes"], codes)
    if "packed" in g:
        if fmt == FMT_DENSE2:
            assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m), O.pack_dense2(codes))
        else:
            if (k * n // m) % 4 == 0:
                assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m),
                                      O.pack_nm(codes, keep, n, m))
            assert np.array_equal(meta_rows(g["meta"], n_out, k), O.pack_bitmap(keep))


def _run(mats, fmt, n, m, flag, label, outs=None):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    outs = outs or [("mask_bits", "codes", "packed")] * len(mats)
    items = [_item(bits, fmt, n, m, o) for bits, o in zip(mats, outs)]
    for rep in range(2):
        say(f"ablation flag={flag} {label} fmt={fmt} {n}:{m} call {rep}")
        sbl.sbl_quant_weights_batch(items, n, m, fmt, flags=flag)
        torch.cuda.synchronize()
        for bits, it in zip(mats, items):
            g = {key: to_np(v) for key, v in it.items() if key not in ("w", "workspace") and v is not None}
            _check(bits, g, fmt, n, m, flag)


@pytest.mark.parametrize("flag", [QW_BETA_KEPT, QW_MASK_FROM_CODES])
@pytest.mark.parametrize("fmt,n,m", PATTERNS)
def test_variant_matches_oracle(fmt, n, m, flag):
    rng = np.random.default_rng([61, fmt, n, m, flag])
    mats = [synth.gaussian_masters(rng, 300, 1024),
            synth.rare_mixture(rng, 256, 1024),              # out-of-window sums in many workgroups
            synth.plant_ties(synth.gaussian_masters(rng, 130, 1536), rng),
            synth.gaussian_masters(rng, 1, 64)]               # one group row, one workgroup
    _run(mats, fmt, n, m, flag, "mixed matrices")


@pytest.mark.parametrize("flag", [QW_BETA_KEPT, QW_MASK_FROM_CODES])
def test_variant_output_subsets(flag):
    """beta alone (its own finalizing kernel), packed alone, mask alone."""
    rng = np.random.default_rng([62, flag])
    mats = [synth.gaussian_masters(rng, 200, 512), synth.rare_mixture(rng, 96, 1024),
            synth.gaussian_masters(rng, 64, 256)]
    _run(mats, FMT_NM, 6, 8, flag, "subsets", outs=[(), ("packed",), ("mask_bits",)])
    _run(mats, FMT_DENSE2, 2, 4, flag, "beta only", outs=[(), (), ()])


@pytest.mark.parametrize("flag", [QW_BETA_KEPT, QW_MASK_FROM_CODES])
def test_variant_many_partial_sums(flag):
    """A 3072 x 4096 matrix has more partial sums than one wave finalizes, so
    beta gets its own kernel before the mask/pack pass; a few out-of-range
    values make some partial sums carry exact records."""
    rng = np.random.default_rng([63, flag])
    bits = synth.gaussian_masters(rng, 3072, 4096)
    flat = bits.reshape(-1)
    idx = rng.choice(flat.size, 5, replace=False)
    flat[idx] = np.array([0x0001, 0x8123, 0x2F00, 0x4100, 0xC3A5], np.uint16)
    _run([bits], FMT_NM, 6, 8, flag, "3072x4096")


def test_flags_rejected():
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(64)
    it = _item(synth.gaussian_masters(rng, 16, 64), FMT_NM, 6, 8)
    for flags in (3, 16, -1):
        with pytest.raises(RuntimeError):
            sbl.sbl_quant_weights_batch([it], 6, 8, FMT_NM, flags=flags)
    torch.cuda.synchronize()
    assert to_np(it["beta"])[0] == -1.0                   # nothing ran


def _binomial_zero_fraction(n, m, p):
    """Zero-code fraction after an n:m mask when each code of a group is
    nonzero independently with probability p: the mask keeps min(n, B) of the
    B nonzero codes (they are the largest magnitudes, or the largest |code|)."""
    e_kept = sum(min(n, b) * math.comb(m, b) * p ** b * (1 - p) ** (m - b) for b in range(m + 1))
    return 1 - e_kept / m


@pytest.mark.parametrize("flag", [0, QW_BETA_KEPT, QW_MASK_FROM_CODES])
def test_sparsity_sweep(flag):
    """The pages' sparsity sweep 8:8 ... 2:8 (and 2:4) on one Gaussian matrix:
    every output bit-exact with the oracle, and the zero-code fraction of the
    GPU codes at the binomial closed form where it applies (the method's order
    and masks from codes; mask-then-quant has a different scale)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([65, flag])
    bits = synth.gaussian_masters(rng, 512, 2048)
    p = 1 - math.erf(1 / (2 * math.sqrt(math.pi)))     # P(code != 0) for Gaussian masters
    order = ORDER.get(flag, O.QUANT_THEN_MASK)
    fracs = []
    for n, m in [(8, 8), (7, 8), (6, 8), (5, 8), (4, 8), (3, 8), (2, 8), (2, 4)]:
        it = _item(bits, FMT_NM, n, m)
        say(f"sweep flag={flag} {n}:{m}")
        sbl.sbl_quant_weights_batch([it], n, m, FMT_NM, flags=flag)
        torch.cuda.synchronize()
        beta, keep, codes = O.quant_weights(bits, n, m, order)
        g_codes = to_np(it["codes"])
        assert to_np(it["beta"])[0] == beta
        assert np.array_equal(g_codes, codes)
        assert np.array_equal(to_np(it["mask_bits"]), O.pack_bitmap(keep))
        zf = float((g_codes == 0).mean())
        say(f"  zero fraction {zf:.4f}")
        if flag != QW_BETA_KEPT:
            assert abs(zf - _binomial_zero_fraction(n, m, p)) < 3e-3
        if m == 8:
            fracs.append(zf)
    assert all(a < b for a, b in zip(fracs, fracs[1:]))  # sparser patterns zero more codes
