"""Weight preparation with every subset of outputs, in one launch (the
masters held on the chip) and in two (SBL_QW_TWO_PASS).

In the two-launch path beta is finalized at the start of the mask/pack
pass, or by its own kernel when beta is the only output, from the partial
sums the absmean pass wrote into the workspace (exact out-of-range sums for
the workgroups that met such values).  Workspaces start out filled with 0xFF bytes (they need no
initialization); each case runs twice on the same workspaces and is compared
with the oracle bit for bit."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, meta_rows, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

SUBSETS = {
    "packed": ("packed",),
    "mask": ("mask_bits",),
    "codes": ("codes",),
    "mask+packed": ("mask_bits", "packed"),
    "codes+packed": ("codes", "packed"),
    "beta": (),
}
PATTERNS = [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_DENSE2, 3, 4), (FMT_NM, 7, 8),
            (FMT_NM, 5, 8)]


def _item(bits, outs, fmt, n, m):
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


def _check(bits, g, fmt, n, m):
    n_out, k = bits.shape
    beta, keep, codes = O.quant_weights(bits, n, m)
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
                assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m), O.pack_nm(codes, keep, n, m))
            assert np.array_equal(meta_rows(g["meta"], n_out, k), O.pack_bitmap(keep))


def _run(mats, subsets, fmt, n, m, label, flags=0):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    items = [_item(bits, SUBSETS[s], fmt, n, m) for bits, s in zip(mats, subsets)]
    for rep in range(2):
        say(f"weight outputs {label} fmt={fmt} {n}:{m} flags={flags} call {rep}")
        sbl.sbl_quant_weights_batch(items, n, m, fmt, flags=flags)
        torch.cuda.synchronize()
        for bits, it in zip(mats, items):
            g = {key: to_np(v) for key, v in it.items() if key not in ("w", "workspace") and v is not None}
            _check(bits, g, fmt, n, m)


# 0: one launch where the batch fits on the chip (all of these); 4: SBL_QW_TWO_PASS
@pytest.mark.parametrize("flags", [0, 4])
@pytest.mark.parametrize("subset", list(SUBSETS))
@pytest.mark.parametrize("fmt,n,m", PATTERNS)
def test_output_subsets(fmt, n, m, subset, flags):
    rng = np.random.default_rng([57, fmt, n, m, len(subset)])
    mats = [synth.gaussian_masters(rng, 300, 1024),
            synth.rare_mixture(rng, 256, 1024),                # several workgroups of both passes flagged
            synth.plant_ties(synth.gaussian_masters(rng, 130, 1536), rng)]
    _run(mats, [subset] * 3, fmt, n, m, subset, flags)


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 2, 4)])
def test_mixed_output_batches(fmt, n, m):
    """Items of one batch with different output sets (a beta-only item gets
    its beta from the mask/pack launch of the others)."""
    rng = np.random.default_rng([58, fmt, n, m])
    mats = [synth.gaussian_masters(rng, 200, 512), synth.rare_mixture(rng, 96, 1024),
            synth.gaussian_masters(rng, 64, 256), synth.gaussian_masters(rng, 33, 320)]
    for flags in (0, 4):
        _run(mats, ["packed", "beta", "mask", "codes"], fmt, n, m, "mixed, one beta-only", flags)
        _run(mats, ["packed", "mask+packed", "mask", "packed"], fmt, n, m, "mixed", flags)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 2, 4)])
def test_few_out_of_range_values(fmt, n, m):
    """Gaussian masters with a handful of tiny, subnormal and large values
    scattered over a matrix of many workgroups: only a few partial sums carry
    an exact out-of-range record."""
    rng = np.random.default_rng([59, fmt, n, m])
    bits = synth.gaussian_masters(rng, 2048, 4096)
    flat = bits.reshape(-1)
    idx = rng.choice(flat.size, 5, replace=False)
    flat[idx] = np.array([0x0001, 0x8123, 0x2F00, 0x4100, 0xC3A5], np.uint16)   # 2^-133 .. 330
    for flags in (0, 4):
        _run([bits, synth.gaussian_masters(rng, 64, 4096)], ["packed", "mask+packed"], fmt, n, m, "few flagged",
             flags)
