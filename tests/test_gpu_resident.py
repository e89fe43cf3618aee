"""The one-launch weight preparation (masters held in registers while the
exact beta is completed) against the oracle, and against the two-launch path.

Every workgroup publishes its exact partial sum under a per-call tag and waits
for its matrix's other slots; the wait is bounded, after which it computes the
missing sums itself (forced here with SBL_QW_NO_WAIT).  These tests check that
the results are the oracle's bit for bit in every mode, and that no call ever
takes a partial sum left by an earlier call: masters change between calls on
one workspace, between graph replays of one captured call, and workspaces
start out filled with random bytes or hold another shape's layout."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, meta_rows, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

TWO_PASS, NO_WAIT = 4, 8
MODES = {"one-launch": 0, "no-wait": NO_WAIT, "two-pass": TWO_PASS}


def _item(w, fmt, n, m, ws=None, fill=0xFF):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = w.shape
    if ws is None:
        ws = torch.full((sbl.sbl_workspace_bytes(n_out, k),), fill, dtype=torch.uint8, device="cuda")
    return dict(w=w, beta=torch.full((1,), -1.0, device="cuda"),
                mask_bits=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda"),
                codes=torch.empty((n_out, k), dtype=torch.int8, device="cuda"),
                packed=torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda"),
                meta=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None,
                workspace=ws)


def _check(bits, it, fmt, n, m, label):
    n_out, k = bits.shape
    beta, keep, codes = O.quant_weights(bits, n, m)
    assert to_np(it["beta"])[0] == beta, label
    assert np.array_equal(to_np(it["mask_bits"]), O.pack_bitmap(keep)), label
    assert np.array_equal(to_np(it["codes"]), codes), label
    got = packed_rows(to_np(it["packed"]), n_out, k, fmt, n, m)
    if fmt == FMT_DENSE2:
        assert np.array_equal(got, O.pack_dense2(codes)), label
    else:
        if (k * n // m) % 4 == 0:
            assert np.array_equal(got, O.pack_nm(codes, keep, n, m)), label
        assert np.array_equal(meta_rows(to_np(it["meta"]), n_out, k), O.pack_bitmap(keep)), label


def _call(items, n, m, fmt, flags):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    sbl.sbl_quant_weights_batch(items, n, m, fmt, flags=flags)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 7, 8),
                                     (FMT_DENSE2, 8, 8), (FMT_NM, 3, 4)])
def test_modes_match_oracle(fmt, n, m, mode):
    rng = np.random.default_rng([71, fmt, n, m])
    mats = [synth.gaussian_masters(rng, 300, 1024),          # 5 slots, the last one partial
            synth.rare_mixture(rng, 256, 1024),              # every slot carries an exact record
            synth.plant_ties(synth.gaussian_masters(rng, 130, 1536), rng),
            synth.gaussian_masters(rng, 1, 64)]              # one chunk
    items = [_item(to_dev(b), fmt, n, m) for b in mats]
    for rep in range(2):
        say(f"resident {mode} fmt={fmt} {n}:{m} call {rep}")
        _call(items, n, m, fmt, MODES[mode])
        for i, (b, it) in enumerate(zip(mats, items)):
            _check(b, it, fmt, n, m, (mode, rep, i))


def test_successive_calls_take_no_stale_sums():
    """New masters before every call on the same workspaces, the modes mixed:
    a partial sum of an earlier call must never be taken for the current one."""
    rng = np.random.default_rng(72)
    fmt, n, m = FMT_NM, 6, 8
    shapes = [(512, 2048), (64, 4096), (48, 320)]           # 16, 4 and 1 slots
    mats = [synth.gaussian_masters(rng, *s) for s in shapes]
    ws = [to_dev(b) for b in mats]
    items = [_item(w, fmt, n, m) for w in ws]
    seq = [0, NO_WAIT, 0, TWO_PASS, 0, NO_WAIT, NO_WAIT, 0, 0]
    for step, flags in enumerate(seq):
        if step % 3 == 2:                                   # a matrix with out-of-range values now and then
            mats = [synth.rare_mixture(rng, *s) for s in shapes]
        else:
            mats = [synth.gaussian_masters(rng, *s, sigma=0.01 * (1 + step)) for s in shapes]
        for w, b in zip(ws, mats):
            w.copy_(to_dev(b))
        say(f"successive call {step} flags={flags}")
        _call(items, n, m, fmt, flags)
        for i, (b, it) in enumerate(zip(mats, items)):
            _check(b, it, fmt, n, m, (step, flags, i))


def test_graph_replays_with_new_masters():
    """One captured call replayed with the masters changed in place between
    replays: every replay is a new call (the workspace generation moves on)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(73)
    fmt, n, m = FMT_NM, 6, 8
    shapes = [(256, 1536), (96, 1024)]
    mats = [synth.gaussian_masters(rng, *s) for s in shapes]
    ws = [to_dev(b) for b in mats]
    items = [_item(w, fmt, n, m) for w in ws]
    _call(items, n, m, fmt, 0)                                # warm-up outside the capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sbl.sbl_quant_weights_batch(items, n, m, fmt)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(5):
        mats = [synth.gaussian_masters(rng, *sh, sigma=0.005 * (rep + 1)) for sh in shapes]
        if rep == 3:
            mats[1] = synth.rare_mixture(rng, *shapes[1])
        for w, b in zip(ws, mats):
            w.copy_(to_dev(b))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i, (b, it) in enumerate(zip(mats, items)):
            _check(b, it, fmt, n, m, ("replay", rep, i))


def test_random_workspace_contents():
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(74)
    fmt, n, m = FMT_DENSE2, 2, 4
    mats = [synth.gaussian_masters(rng, 640, 1024), synth.rare_mixture(rng, 70, 2048)]
    items = []
    for b in mats:
        nbytes = sbl.sbl_workspace_bytes(*b.shape)
        junk = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
        items.append(_item(to_dev(b), fmt, n, m, ws=junk))
    for flags in (0, NO_WAIT, 0):
        say(f"random workspace flags={flags}")
        _call(items, n, m, fmt, flags)
        for i, (b, it) in enumerate(zip(mats, items)):
            _check(b, it, fmt, n, m, (flags, i))


def test_workspace_shared_by_shapes():
    """One workspace, sized for the larger matrix, serves matrices of
    different slot counts in turn (each layout lands on the other's words)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(75)
    fmt, n, m = FMT_NM, 6, 8
    ws = torch.full((sbl.sbl_workspace_bytes(1024, 4096),), 0xFF, dtype=torch.uint8, device="cuda")
    for step, shape in enumerate([(1024, 4096), (100, 640), (1024, 4096), (512, 4096), (1024, 4096)]):
        b = synth.gaussian_masters(rng, *shape) if step != 2 else synth.rare_mixture(rng, *shape)
        it = _item(to_dev(b), fmt, n, m, ws=ws)
        for flags in (0, TWO_PASS, 0):
            say(f"shared workspace step {step} {shape} flags={flags}")
            _call([it], n, m, fmt, flags)
            _check(b, it, fmt, n, m, (step, flags))


def test_batch_of_eight_near_capacity():
    """Eight matrices of 4M weights each (512 one-launch workgroups, two per
    CU on 256 CUs): one launch when the chip holds them all, else two; the
    results are the same either way."""
    rng = np.random.default_rng(76)
    fmt, n, m = FMT_NM, 6, 8
    mats = [synth.gaussian_masters(rng, 1024, 4096) for _ in range(8)]
    mats[5] = synth.rare_mixture(rng, 1024, 4096)
    items = [_item(to_dev(b), fmt, n, m) for b in mats]
    for flags in (0, 0):
        say(f"eight matrices flags={flags}")
        _call(items, n, m, fmt, flags)
        for i, (b, it) in enumerate(zip(mats, items)):
            _check(b, it, fmt, n, m, (flags, i))
