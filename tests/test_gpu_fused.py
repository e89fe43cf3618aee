"""Activation quantization fused into the product (sbl_linear_acts_batch):
the fused launch and the fallback (sbl_quant_acts, then sbl_linear_batch) must
give bit-identical xq, gamma, acc and y, and both must match the oracle
(int8 activations, gamma and int32 acc bit for bit; y within 1e-6 relative)."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, check_y, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

# (label, [(n_out, k)], m_tok, fmt, n, m); every item of a case shares k
CASES = [
    ("qkv 0.7B M=1", [(1536, 1536)] * 3, 1, FMT_NM, 6, 8),
    ("gate/up 0.7B M=4", [(4096, 1536)] * 2, 4, FMT_DENSE2, 6, 8),
    ("down 0.7B M=1", [(1536, 4096)], 1, FMT_NM, 2, 4),
    ("o 3B M=2", [(3200, 3200)], 2, FMT_NM, 6, 8),
    ("down 3B M=1", [(3200, 8640)], 1, FMT_NM, 6, 8),
    ("down 70B M=1 (28672 inputs, fused)", [(64, 28672)], 1, FMT_NM, 6, 8),
    ("down 70B M=2 (not fused)", [(48, 28672)], 2, FMT_DENSE2, 6, 8),
    ("ragged rows, partial panel, M=3", [(33, 320), (17, 320)], 3, FMT_DENSE2, 6, 8),
    ("one tile, M=16", [(16, 64)], 16, FMT_NM, 6, 8),
    ("wide input, M=16 (not fused)", [(64, 4096)], 16, FMT_NM, 6, 8),
    ("nine items (not fused)", [(48, 256)] * 9, 2, FMT_NM, 2, 4),
    ("empty item among others", [(40, 512), (0, 512), (24, 512)], 1, FMT_DENSE2, 6, 8),
]


def _prepare(rng, shapes, n, m, fmt):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    items, host = [], []
    for no, k in shapes:
        if no == 0:
            items.append(dict(packed=torch.empty(16, dtype=torch.uint8, device="cuda"),
                              meta=torch.empty(16, dtype=torch.uint8, device="cuda"),
                              beta=torch.ones(1, device="cuda"), n_out=0,
                              y=torch.empty(16, device="cuda")))
            host.append(None)
            continue
        bits = synth.gaussian_masters(rng, no, k)
        o = sbl.quant_weights(to_dev(bits), n, m, fmt=fmt)
        items.append(dict(packed=o["packed"], meta=o["meta"], beta=o["beta"], n_out=no))
        host.append(bits)
    return items, host


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_matches_separate_and_oracle(case):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    label, shapes, m_tok, fmt, n, m = case
    k = shapes[0][1]
    rng = np.random.default_rng([71, len(label), m_tok, fmt, n])
    say(f"fused acts: {label}")
    items, host = _prepare(rng, shapes, n, m, fmt)
    x = synth.gaussian_acts(rng, m_tok, k, hot_channels=4)
    x[0, 5] = 0.0
    if m_tok > 1:
        x[1, :] = 0.0                                # all-zero token: gamma = 0, scale floor 1e-5
    xd = to_dev(x.astype(np.float32))

    def run(fused):
        xq = torch.full((m_tok, k), 77, dtype=torch.int8, device="cuda")
        gamma = torch.full((m_tok,), -1.0, device="cuda")
        outs = [dict(it, y=torch.full((m_tok, max(it["n_out"], 1)), 3.0, device="cuda"),
                     acc=torch.full((m_tok, max(it["n_out"], 1)), 7, dtype=torch.int32, device="cuda"))
                for it in items]
        if fused:
            sbl.sbl_linear_acts_batch(xd, xq, gamma, outs, fmt, n, m)
        else:
            sbl.sbl_quant_acts(xd, xq, gamma)
            sbl.sbl_linear_batch([dict(o, xq=xq, gamma=gamma) for o in outs], fmt, n, m)
        torch.cuda.synchronize()
        return to_np(xq), to_np(gamma), [(to_np(o["y"]), to_np(o["acc"])) for o in outs]

    fq, fg, fres = run(True)
    sq, sg, sres = run(False)
    assert np.array_equal(fq, sq)
    assert np.array_equal(fg.view(np.uint32), sg.view(np.uint32))
    q_ref, g_ref = O.quant_acts(x)
    assert np.array_equal(fq, q_ref)
    assert np.array_equal(fg, g_ref)
    for (fy, fa), (sy, sa), bits, (no, _) in zip(fres, sres, host, shapes):
        assert np.array_equal(fa, sa)
        assert np.array_equal(fy.view(np.uint32), sy.view(np.uint32))
        if bits is None:
            assert np.all(fa == 7) and np.all(fy == 3.0)   # an empty product writes nothing
            continue
        beta, keep, codes = O.quant_weights(bits, n, m)
        acc_ref, y_ref = O.linear(codes, q_ref, beta, g_ref)
        assert np.array_equal(fa, acc_ref)
        check_y(fy, y_ref, acc_ref)


def _near_half_rows(rng, n_rows, k):
    """Rows whose values sit at and next to the rounding boundaries of the
    quantizer: x = (j + 1/2) * s moved by up to 3 fp32 ulps, with s = gamma/128
    for a gamma planted at position 0 (a power-of-two multiple or a random
    value).  The rest of each row is filled with such values for random j."""
    x = np.zeros((n_rows, k), np.float32)
    for t in range(n_rows):
        gamma = np.float32(3.0) if t % 2 == 0 else np.float32(rng.uniform(0.3, 40.0))
        s = np.float32(gamma) * np.float32(1.0 / 128)
        j = rng.integers(-128, 128, k - 1)
        base = ((j + 0.5) * np.float64(s)).astype(np.float32)
        steps = rng.integers(-3, 4, k - 1)
        v = base.copy()
        for d in (1, -1):
            for _ in range(3):
                mv = steps * d > 0
                v[mv] = np.nextafter(v[mv], np.float32(d * np.inf))
                steps = np.where(mv, steps - d, steps)
        v = np.clip(v, -gamma, gamma)
        x[t, 0] = gamma
        x[t, 1:] = v
    return x


@pytest.mark.parametrize("m_tok,k", [(3, 4096), (130, 1024), (1, 28672)])
def test_quant_acts_near_half_integers(m_tok, k):
    """Values within a few ulps of the half-integers of x/s: the quantizer's
    multiply-and-check evaluation must give the IEEE quotient's rounding
    everywhere (the standalone quantizer in both workgroup shapes, and the
    quantization fused into the GEMV)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([73, m_tok, k])
    x = _near_half_rows(rng, m_tok, k)
    say(f"near-half activations m_tok={m_tok} k={k}")
    q_ref, g_ref = O.quant_acts(x)
    xq, gamma = sbl.quant_acts(to_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(xq), q_ref)
    assert np.array_equal(to_np(gamma), g_ref)
    if m_tok <= 16:
        bits = synth.gaussian_masters(rng, 32, k)
        o = sbl.quant_weights(to_dev(bits), 6, 8, fmt=FMT_NM)
        xq2 = torch.empty((m_tok, k), dtype=torch.int8, device="cuda")
        g2 = torch.empty(m_tok, device="cuda")
        y = torch.empty((m_tok, 32), device="cuda")
        sbl.sbl_linear_acts_batch(to_dev(x), xq2, g2, [dict(o, n_out=32, y=y)], FMT_NM, 6, 8)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(xq2), q_ref)
        assert np.array_equal(to_np(g2), g_ref)
