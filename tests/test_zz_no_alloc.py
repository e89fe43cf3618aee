"""The allocation-free weight preparation (sbl_quant_weights_batch_noalloc,
the library's fixed per-GPU scratch instead of caller workspaces) gives the
same bits as sbl_quant_weights_batch with workspaces: beta, mask, packed
codes and metadata.  Two calls in a row share the scratch, the second with a
smaller batch, and they cover both launch plans (two passes over a large
batch, one launch over a batch that fits the chip)."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _items(shapes, seed, n, m, fmt, workspaces):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(seed)
    out = []
    for no, k in shapes:
        bits = synth.plant_ties(synth.gaussian_masters(rng, no, k), rng, m=m, n=n if n < m else m - 1)
        it = dict(w=to_dev(bits), beta=torch.full((1,), -1.0, device="cuda"),
                  mask_bits=torch.zeros((no, k // 8), dtype=torch.uint8, device="cuda"),
                  packed=torch.zeros(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device="cuda"),
                  meta=torch.zeros((no, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None)
        if workspaces:
            it["workspace"] = sbl.new_workspace(no, k)
        out.append(it)
    return out


def _same(a, b):
    for x, y in zip(a, b):
        assert to_np(x["beta"])[0] == to_np(y["beta"])[0]
        assert np.array_equal(to_np(x["mask_bits"]), to_np(y["mask_bits"]))
        assert np.array_equal(to_np(x["packed"]), to_np(y["packed"]))
        if x["meta"] is not None:
            assert np.array_equal(to_np(x["meta"]), to_np(y["meta"]))


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 2, 4)])
def test_noalloc_matches_workspace_call(fmt, n, m):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    sbl.load()
    calls = [("large batch (two passes)", [(4096, 4096), (4096, 4096), (4096, 4096), (1536, 1536)], 1),
             ("smaller batch (one launch)", [(1536, 1536), (1536, 4096), (64, 128)], 2)]
    for what, shapes, seed in calls:
        say(f"noalloc {what} fmt={fmt} {n}:{m} shapes={shapes}")
        ref = _items(shapes, seed, n, m, fmt, workspaces=True)
        got = _items(shapes, seed, n, m, fmt, workspaces=False)
        sbl.sbl_quant_weights_batch(ref, n, m, fmt)
        sbl.sbl_quant_weights_batch_noalloc(got, n, m, fmt)
        torch.cuda.synchronize()
        _same(got, ref)
