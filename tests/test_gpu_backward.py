"""Backward of the layer (dual straight-through estimator) on the GPU against
the oracle: dX and dW within the oracle's elementwise fp32 bounds (exact
products, fp32 sums of L terms in any order: (L + 1) 2^-24 sum|terms|), and
dX exactly 0 wherever the activation clamp acted.

The forward quantities (beta, packed weights, xq, gamma) come from the GPU
path for the GPU backward and from the oracle for the oracle's; the forward
parity tests show they are the same bits."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu


def _gpu_forward_parts(bits, x, n, m, fmt):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    w = sbl.quant_weights(to_dev(bits), n, m, fmt)
    xq, gamma = sbl.quant_acts(to_dev(x.astype(np.float32)))
    torch.cuda.synchronize()
    return w, xq, gamma


def _check(got, ref, bound, name):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound
    assert not bad.any(), (name, int(bad.sum()), float(err[bad].max()), float(bound[bad].min()))


def _dirty_workspace(t, n_out, k):
    """A backward workspace full of 0xFF bytes (NaN as BF16): every element the
    call reads must have been written by the call itself."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    return torch.full((sbl.sbl_backward_workspace_bytes(t, n_out, k),), 255, dtype=torch.uint8, device="cuda")


def _run(t, n_out, k, n, m, fmt, seed, rows=None, hot=0, ws=False):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng(seed)
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, t, k, hot_channels=hot)
    dy = synth.f32_to_bf16_bits((rng.standard_normal((t, n_out)) * 0.05).astype(np.float32))
    say(f"backward t={t} n_out={n_out} k={k} {n}:{m} fmt={fmt} workspace={ws}")
    w, xq, gamma = _gpu_forward_parts(bits, x, n, m, fmt)
    dx = torch.full((t, k), np.nan, dtype=torch.float32, device="cuda")
    dw = torch.full((n_out, k), np.nan, dtype=torch.float32, device="cuda")
    sbl.sbl_linear_backward(to_dev(dy), w["packed"], w["meta"], fmt, n, m, w["beta"], to_dev(x.astype(np.float32)),
                            xq, gamma, dx=dx, dw=dw, workspace=_dirty_workspace(t, n_out, k) if ws else None)
    torch.cuda.synchronize()
    dx, dw = to_np(dx), to_np(dw)
    beta, keep, codes = O.quant_weights(bits, n, m)
    q, g = O.quant_acts(x)
    assert np.array_equal(to_np(xq), q) and np.array_equal(to_np(gamma), g)
    tr = np.arange(t) if rows is None else rows[0]
    nr = np.arange(n_out) if rows is None else rows[1]
    r = O.backward(codes, beta, x[tr], q[tr], g[tr], dy[tr])           # dX rows tr
    clip = r["clip"] == 0
    assert np.all(dx[tr][clip] == 0.0)
    _check(dx[tr], r["dx"], r["dx_bound"], "dx")
    r = O.backward(codes[nr], beta, x, q, g, dy[:, nr])                  # dW rows nr
    _check(dw[nr], r["dw"], r["dw_bound"], "dw")
    return dx, dw


@pytest.mark.parametrize("ws", [False, True], ids=["tiles", "workspace"])
@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8),
                                     (FMT_NM, 8, 8), (FMT_NM, 3, 4)])
@pytest.mark.parametrize("t,n_out,k", [(1, 8, 64), (5, 72, 192), (130, 264, 320)])
def test_backward_matches_oracle(t, n_out, k, n, m, fmt, ws):
    _run(t, n_out, k, n, m, fmt, seed=[90, t, n_out, k, n, m, fmt], hot=2 if k >= 192 else 0, ws=ws)


@pytest.mark.parametrize("ws", [False, True], ids=["tiles", "workspace"])
def test_backward_larger_tiles(ws):
    """Several full 128 x 128 tiles in both kernels, ragged edges on every axis."""
    _run(300, 520, 448, 6, 8, FMT_NM, seed=91, hot=8, ws=ws)


def test_backward_workspace_reused_at_a_smaller_shape():
    """One workspace for a large call and then a smaller one (other padding,
    stale contents from the first call): both within the oracle's bounds."""
    _run(200, 392, 512, 6, 8, FMT_DENSE2, seed=95, hot=4, ws=True)
    _run(70, 136, 192, 6, 8, FMT_NM, seed=96, hot=2, ws=True)


def test_backward_outputs_one_at_a_time():
    """dx alone, dw alone (the other pointer NULL): each equals the joint call's."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    t, n_out, k, n, m, fmt = 40, 96, 256, 6, 8, FMT_NM
    rng = np.random.default_rng(92)
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, t, k)
    dy = to_dev(synth.f32_to_bf16_bits((rng.standard_normal((t, n_out)) * 0.05).astype(np.float32)))
    w, xq, gamma = _gpu_forward_parts(bits, x, n, m, fmt)
    xd = to_dev(x.astype(np.float32))
    both = [torch.empty((t, k), device="cuda"), torch.empty((n_out, k), device="cuda")]
    sbl.sbl_linear_backward(dy, w["packed"], w["meta"], fmt, n, m, w["beta"], xd, xq, gamma, dx=both[0], dw=both[1])
    dx1 = torch.empty((t, k), device="cuda")
    dw1 = torch.empty((n_out, k), device="cuda")
    sbl.sbl_linear_backward(dy, w["packed"], w["meta"], fmt, n, m, w["beta"], xd, None, gamma, dx=dx1)
    sbl.sbl_linear_backward(dy, None, None, fmt, n, m, None, None, xq, gamma, dw=dw1)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(dx1), to_np(both[0])) and np.array_equal(to_np(dw1), to_np(both[1]))


@pytest.mark.parametrize("ws", [False, True], ids=["tiles", "workspace"])
def test_backward_3b_block_matrix_sampled(ws):
    """A 3B-class gate matrix (8640 x 3200) with 2048 tokens, as the benchmark
    times it: sampled token rows of dX (including both sides of the 128-token
    wave halves and of the 256-token workgroup tiles) and output rows of dW."""
    rng = np.random.default_rng(93)
    rows = (np.unique(np.concatenate([[0, 127, 128, 255, 256, 2047], rng.integers(0, 2048, 12)])),
            np.unique(np.concatenate([[0, 8639], rng.integers(0, 8640, 14)])))
    _run(2048, 8640, 3200, 6, 8, FMT_NM, seed=94, rows=rows, hot=8, ws=ws)


def test_backward_workspace_outputs_one_at_a_time():
    """Through the workspace: dx alone and dw alone equal the joint call's bits."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    t, n_out, k, n, m, fmt = 90, 200, 320, 6, 8, FMT_DENSE2
    rng = np.random.default_rng(97)
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, t, k)
    dy = to_dev(synth.f32_to_bf16_bits((rng.standard_normal((t, n_out)) * 0.05).astype(np.float32)))
    w, xq, gamma = _gpu_forward_parts(bits, x, n, m, fmt)
    xd = to_dev(x.astype(np.float32))
    ws = _dirty_workspace(t, n_out, k)
    both = [torch.empty((t, k), device="cuda"), torch.empty((n_out, k), device="cuda")]
    sbl.sbl_linear_backward(dy, w["packed"], w["meta"], fmt, n, m, w["beta"], xd, xq, gamma, dx=both[0], dw=both[1],
                            workspace=ws)
    dx1 = torch.empty((t, k), device="cuda")
    dw1 = torch.empty((n_out, k), device="cuda")
    sbl.sbl_linear_backward(dy, w["packed"], w["meta"], fmt, n, m, w["beta"], xd, None, gamma, dx=dx1, workspace=ws)
    sbl.sbl_linear_backward(dy, None, None, fmt, n, m, None, None, xq, gamma, dw=dw1, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(dx1), to_np(both[0])) and np.array_equal(to_np(dw1), to_np(both[1]))
