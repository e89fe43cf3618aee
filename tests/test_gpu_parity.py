"""GPU parity of every step of the path against the CPU oracle, element by
element, through the C ABI.  Codes, masks, packed bytes, int8 activations,
gamma, beta and int32 accumulators must be bit-exact; y within 1e-6 relative
(and exactly 0 where acc == 0)."""

import numpy as np
import pytest

import synth
from oracle import sbl_oracle as O
from gpu_util import (FMT_DENSE2, FMT_NM, check_y, compare_all, gpu_forward, gpu_quant_weights,
                      meta_rows, oracle_forward, packed_rows, say, to_dev, to_np)

pytestmark = pytest.mark.gpu

FORMATS = [(FMT_DENSE2, "dense2"), (FMT_NM, "nm")]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_linear_layers_absmean_amd import sbl
    sbl.load()


@pytest.mark.parametrize("fmt,fname", FORMATS)
@pytest.mark.parametrize("m_tok", [1, 16])
def test_unit_layer_256(fmt, fname, m_tok):
    """256 x 256 layer, 6:8 along k, masters N(0, 0.02) seed 0, activations N(0,1) seed 1."""
    bits = synth.workload_masters("unit256", 0, 256, 256)
    x = synth.workload_acts("unit256", 0, m_tok, 256)
    say(f"unit256 fmt={fname} m_tok={m_tok}")
    g = gpu_forward(bits, x, 6, 8, fmt)
    r = oracle_forward(bits, x, 6, 8)
    compare_all(g, r, fmt, 256)


RAGGED_PATTERNS = [(6, 8), (2, 4), (8, 8), (4, 4), (5, 8), (3, 8), (1, 4), (7, 8), (3, 4), (1, 8), (4, 8)]


@pytest.mark.parametrize("n,m", RAGGED_PATTERNS)
@pytest.mark.parametrize("fmt,fname", FORMATS)
def test_ragged_shapes_all_patterns(n, m, fmt, fname):
    rng = np.random.default_rng([7, n, m, fmt])
    n_out, k = 200, 320                      # not multiples of the 64-row / 256-k tiles
    bits = synth.gaussian_masters(rng, n_out, k)
    for m_tok in (1, 5, 17, 40):
        x = synth.gaussian_acts(rng, m_tok, k)
        say(f"ragged {n}:{m} fmt={fname} m_tok={m_tok}")
        g = gpu_forward(bits, x, n, m, fmt)
        r = oracle_forward(bits, x, n, m)
        compare_all(g, r, fmt, n_out)


def _beta_only(bits):
    g = gpu_quant_weights(bits, 6, 8, FMT_DENSE2)
    r = O.quant_weights(bits, 6, 8)
    assert to_np(g["beta"])[0] == r[0], (to_np(g["beta"])[0], r[0])
    assert np.array_equal(to_np(g["codes"]), r[2])
    assert np.array_equal(to_np(g["mask"]), O.pack_bitmap(r[1]))
    return r[0]


def test_beta_midpoint_rounding():
    """Means that sit exactly on fp32 midpoints round to even."""
    n_out, k = 8, 1 << 14                    # 2^17 values
    bits = np.full((n_out, k), 0x3F80, np.uint16)           # 1.0
    bits[0, 5] = 0x3F81                                     # mean 1 + 2^-24 -> 1.0
    say("beta midpoint 1+2^-24")
    assert _beta_only(bits) == np.float32(1.0)
    bits[0, 5] = 0x3F83                                     # mean 1 + 3*2^-24 -> 1 + 2^-22
    say("beta midpoint 1+3*2^-24")
    assert _beta_only(bits) == np.float32(1 + 2.0 ** -22)


def test_beta_rare_path_values():
    """Subnormal, tiny, large and zero masters (outside the fast [2^-31, 2) window)."""
    rng = np.random.default_rng(99)
    n_out, k = 64, 512
    kind = rng.integers(0, 5, (n_out, k))
    mag = np.select([kind == 0, kind == 1, kind == 2, kind == 3],
                    [0, rng.integers(1, 0x80, (n_out, k)), rng.integers(0x0080, 0x3000, (n_out, k)),
                     rng.integers(0x3000, 0x4000, (n_out, k))],
                    rng.integers(0x4000, 0x7F00, (n_out, k)))
    bits = (mag | (rng.integers(0, 2, (n_out, k)) << 15)).astype(np.uint16)
    say("beta rare path mixture")
    _beta_only(bits)


def test_beta_subnormal_mean_and_zero_matrix():
    n_out, k = 4, 256
    bits = np.zeros((n_out, k), np.uint16)
    bits[1, 3] = 0x0001                                      # one 2^-133 value
    say("beta subnormal mean")
    b = _beta_only(bits)
    assert b == O.absmean_beta(bits)
    bits[:] = 0x8000                                         # all -0
    say("beta all zeros")
    assert _beta_only(bits) == 0.0


def test_ties_planted():
    base = synth.gaussian_masters(np.random.default_rng(5), 128, 512)
    x = synth.gaussian_acts(np.random.default_rng(8), 3, 512)
    for n, m in [(6, 8), (2, 4)]:
        bits = synth.plant_ties(base, np.random.default_rng(6), m=m, n=n)
        for fmt, fname in FORMATS:
            say(f"ties {n}:{m} {fname}")
            compare_all(gpu_forward(bits, x, n, m, fmt), oracle_forward(bits, x, n, m), fmt, 128)


def test_quant_acts_edge_rows():
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    k = 128
    x = np.random.default_rng(3).standard_normal((6, k)).astype(np.float32)
    x[0, :8] = [2.0, 2.5 / 64, -1.5 / 64, 0.5 / 64, 127.5 / 64, -2.0, 1.0 / 64, 3.5 / 64]
    x[0, 8:] = 0.0
    x[1] = 0.0                                              # gamma = 0 -> q = 0
    x[2] *= 1e30                                            # huge values
    x[3] *= 1e-30                                           # gamma below 1e-5: gamma_eff = 1e-5
    x[4, 17] = -3.0e38                                      # near FLT_MAX
    x[5] = 1e-5
    say("quant_acts edge rows")
    xq, gamma = sbl.quant_acts(to_dev(x))
    torch.cuda.synchronize()
    q_ref, g_ref = O.quant_acts(x)
    assert np.array_equal(to_np(gamma), g_ref)
    assert np.array_equal(to_np(xq), q_ref)
    assert to_np(xq)[0, :8].tolist() == [127, 2, -2, 0, 127, -127, 1, 4]


@pytest.mark.parametrize("k", [64, 3200, 4096, 4160, 8192, 8256, 16384, 16448, 28672])
def test_quant_acts_many_tokens(k):
    """At 128 tokens and more the quantizer sizes its per-thread register slots
    by the row (rows up to 4096, 8192 and 16384 values, longer rows in two
    sweeps): every variant and both sides of each boundary, bit for bit."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    m_tok = 130
    x = synth.gaussian_acts(np.random.default_rng([14, k]), m_tok, k, hot_channels=4)
    x[1] = 0.0
    x[2, k - 1] = 50.0                                      # gamma from the row's last value
    say(f"quant_acts {m_tok} x {k}")
    xq, gamma = sbl.quant_acts(to_dev(x))
    torch.cuda.synchronize()
    q_ref, g_ref = O.quant_acts(x)
    assert np.array_equal(to_np(gamma), g_ref)
    assert np.array_equal(to_np(xq), q_ref)


@pytest.mark.parametrize("k", [16384, 16448, 28672, 32704, 32768])
def test_quant_acts_split_rows(k):
    """Decode-sized tokens of 16384-32768 values are split over 8 workgroups,
    each quantizing its part of the row from registers: both ends of that
    range, parts that do not start on a 1024-piece boundary, the row maximum
    in the last part."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    m_tok = 3
    x = synth.gaussian_acts(np.random.default_rng([15, k]), m_tok, k, hot_channels=4)
    x[1] = 0.0
    x[2, k - 1] = -50.0
    say(f"quant_acts split {m_tok} x {k}")
    xq, gamma = sbl.quant_acts(to_dev(x))
    torch.cuda.synchronize()
    q_ref, g_ref = O.quant_acts(x)
    assert np.array_equal(to_np(gamma), g_ref)
    assert np.array_equal(to_np(xq), q_ref)


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (5, 8), (8, 8)])
def test_pack_standalone(n, m):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([11, n, m])
    n_out, k = 33, 192
    bits = synth.gaussian_masters(rng, n_out, k)
    beta, keep, codes = O.quant_weights(bits, n, m)
    bitmap = O.pack_bitmap(keep)
    for fmt, fname in FORMATS:
        say(f"pack {n}:{m} {fname}")
        packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
        meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
        sbl.sbl_pack(to_dev(codes), to_dev(bitmap), n, m, fmt, packed, meta)
        torch.cuda.synchronize()
        want = O.pack_dense2(codes) if fmt == FMT_DENSE2 else O.pack_nm(codes, keep, n, m)
        assert np.array_equal(packed_rows(to_np(packed), n_out, k, fmt, n, m), want)
        if meta is not None:
            assert np.array_equal(meta_rows(to_np(meta), n_out, k), bitmap)


def test_deterministic_repeat():
    bits = synth.gaussian_masters(np.random.default_rng(12), 300, 1024)
    x = synth.gaussian_acts(np.random.default_rng(13), 20, 1024)
    say("determinism")
    a = gpu_forward(bits, x, 6, 8, FMT_NM)
    b = gpu_forward(bits, x, 6, 8, FMT_NM)
    for key in ("beta", "mask", "codes", "packed", "meta", "xq", "gamma", "acc"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))


def test_empty_batches_are_noops():
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    say("empty batches")
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    xq, gamma = sbl.quant_acts(x)
    assert xq.shape == (0, 64)
    bits = synth.gaussian_masters(np.random.default_rng(1), 16, 64)
    w = gpu_quant_weights(bits, 6, 8, FMT_DENSE2)
    y, acc = sbl.linear(w["packed"], None, FMT_DENSE2, 6, 8, w["beta"], xq, gamma, 16, want_acc=True)
    torch.cuda.synchronize()
    assert y.shape == (0, 16)


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
def test_linear_batch_matches_single_calls(fmt, n, m):
    """Grouped launches (decode items share one GEMV launch) give the oracle's results."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([21, fmt, n, m])
    shapes = [(96, 128, 1), (200, 320, 3), (33, 64, 16), (130, 512, 2), (64, 192, 40), (17, 256, 1),
              (300, 640, 5), (48, 128, 8), (80, 384, 1), (16, 64, 1),
              # several items above the decode range: one grouped GEMM launch (2:4: sparse MFMA)
              (300, 640, 33), (130, 512, 200), (520, 1216, 150),
              # an odd row count: token rows of y are not 16-byte aligned
              (67, 192, 70)]
    items, refs = [], []
    for n_out, k, m_tok in shapes:
        bits = synth.gaussian_masters(rng, n_out, k)
        x = synth.gaussian_acts(rng, m_tok, k)
        w = gpu_quant_weights(bits, n, m, fmt)
        xq, gamma = sbl.quant_acts(to_dev(x))
        y = torch.empty((m_tok, n_out), dtype=torch.float32, device="cuda")
        acc = torch.empty((m_tok, n_out), dtype=torch.int32, device="cuda")
        items.append(dict(packed=w["packed"], meta=w["meta"], beta=w["beta"], xq=xq, gamma=gamma,
                          n_out=n_out, y=y, acc=acc))
        refs.append(oracle_forward(bits, x, n, m))
    say(f"linear_batch fmt={fmt} {n}:{m} items={len(items)}")
    sbl.sbl_linear_batch(items, fmt, n, m)
    torch.cuda.synchronize()
    for it, r in zip(items, refs):
        assert np.array_equal(to_np(it["acc"]), r["acc"])
        check_y(to_np(it["y"]), r["y"], r["acc"])


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4)])
def test_gemm_multi_tile_ragged(fmt, n, m):
    """Token counts above the decode range: several 256-row x 128-token tiles,
    ragged in rows, tokens and k (a half 128-k step at the end)."""
    rng = np.random.default_rng([31, fmt, n, m])
    n_out, k, m_tok = 600, 704, 300
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, m_tok, k, t_row_frac=0.25)
    say(f"gemm multi-tile fmt={fmt} {n}:{m}")
    compare_all(gpu_forward(bits, x, n, m, fmt), oracle_forward(bits, x, n, m), fmt, n_out)


@pytest.mark.parametrize("n_out,k,m_tok", [(1, 64, 17), (33, 128, 40), (257, 576, 129), (520, 1216, 260),
                                           (64, 512, 128)])
def test_gemm24_edge_shapes(n_out, k, m_tok):
    """The 2:4 sparse-MFMA GEMM at its boundaries: one row, a lone half 128-k
    step (K = 64), K covering the unrolled loop plus a tail, 17 tokens (just
    above the decode range), ragged and exact tiles (64 rows x 128 tokens)."""
    rng = np.random.default_rng([37, n_out, k, m_tok])
    bits = synth.plant_ties(synth.gaussian_masters(rng, n_out, k), rng, m=4, n=2)
    x = synth.gaussian_acts(rng, m_tok, k, t_row_frac=0.25)
    say(f"gemm 2:4 sparse MFMA n_out={n_out} k={k} m_tok={m_tok}")
    compare_all(gpu_forward(bits, x, 2, 4, FMT_NM), oracle_forward(bits, x, 2, 4), FMT_NM, n_out)


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
def test_quant_weights_batch_matches_oracle(fmt, n, m):
    """Grouped weight preparation (10 matrices: two launch groups) gives the
    oracle's beta, mask, codes and packed bytes; a second call on the same
    workspaces gives the same bits."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([31, fmt, n, m])
    mats = [synth.gaussian_masters(rng, 96, 128), synth.rare_mixture(rng, 64, 512),
            synth.gaussian_masters(rng, 200, 320), synth.gaussian_masters(rng, 1, 64),
            synth.plant_ties(synth.gaussian_masters(rng, 130, 512), rng),
            synth.gaussian_masters(rng, 1536, 512, outlier_frac=0.01),
            synth.rare_mixture(rng, 3, 1024), synth.gaussian_masters(rng, 17, 256),
            synth.gaussian_masters(rng, 640, 3200), synth.gaussian_masters(rng, 48, 128)]
    items = []
    for bits in mats:
        n_out, k = bits.shape
        items.append(dict(
            w=to_dev(bits), beta=torch.empty(1, dtype=torch.float32, device="cuda"),
            mask_bits=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda"),
            codes=torch.empty((n_out, k), dtype=torch.int8, device="cuda"),
            packed=torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8,
                               device="cuda"),
            meta=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None,
            workspace=sbl.new_workspace(n_out, k)))
    outs = []
    for rep in range(2):
        say(f"quant_weights_batch fmt={fmt} {n}:{m} items={len(items)} call {rep}")
        sbl.sbl_quant_weights_batch(items, n, m, fmt)
        torch.cuda.synchronize()
        outs.append([{key: to_np(v) for key, v in it.items() if key not in ("w", "workspace") and v is not None}
                     for it in items])
    for bits, g, g2 in zip(mats, outs[0], outs[1]):
        n_out, k = bits.shape
        beta, keep, codes = O.quant_weights(bits, n, m)
        assert g["beta"][0] == beta, (bits.shape, g["beta"][0], beta)
        assert np.array_equal(g["mask_bits"], O.pack_bitmap(keep))
        assert np.array_equal(g["codes"], codes)
        if fmt == FMT_DENSE2:
            assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m), O.pack_dense2(codes))
        else:
            if (k * n // m) % 4 == 0:
                assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m), O.pack_nm(codes, keep, n, m))
            assert np.array_equal(meta_rows(g["meta"], n_out, k), O.pack_bitmap(keep))
        for key in g:
            assert np.array_equal(g[key], g2[key]), key
