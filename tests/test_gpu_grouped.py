"""Group scales on the GPU (one exact absmean beta per block of output rows):
sbl_quant_weights_grouped and sbl_linear_grouped against the oracle, bit for
bit for beta, mask, codes, packed bytes, metadata and acc; y within the usual
1e-6 relative."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, check_y, meta_rows, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu


def _run(bits, x, n, m, fmt, rpg, label):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = bits.shape
    groups = -(-n_out // rpg)
    say(f"grouped {label} {n_out}x{k} rows_per_group={rpg} {n}:{m} fmt={fmt}")
    beta = torch.full((groups,), -1.0, device="cuda")
    mask = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    codes = torch.empty((n_out, k), dtype=torch.int8, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
    ws = torch.full((sbl.sbl_workspace_bytes_grouped(n_out, k, rpg),), 0xFF, dtype=torch.uint8, device="cuda")
    w = to_dev(bits)
    for rep in range(2):                                     # the same workspace twice
        sbl.sbl_quant_weights_grouped(w, n, m, rpg, beta, ws, mask_bits=mask, codes=codes, fmt=fmt, packed=packed,
                                      meta=meta)
    xq, gamma = sbl.quant_acts(to_dev(x.astype(np.float32)))
    y = torch.empty((x.shape[0], n_out), dtype=torch.float32, device="cuda")
    acc = torch.empty((x.shape[0], n_out), dtype=torch.int32, device="cuda")
    sbl.sbl_linear_grouped(packed, meta, fmt, n, m, beta, rpg, xq, gamma, n_out, y, acc)
    torch.cuda.synchronize()
    betas, keep, c = O.quant_weights_grouped(bits, n, m, rpg)
    assert np.array_equal(to_np(beta), betas)
    assert np.array_equal(to_np(mask), O.pack_bitmap(keep))
    assert np.array_equal(to_np(codes), c)
    if fmt == FMT_DENSE2:
        assert np.array_equal(packed_rows(to_np(packed), n_out, k, fmt, n, m), O.pack_dense2(c))
    else:
        if (k * n // m) % 4 == 0:
            assert np.array_equal(packed_rows(to_np(packed), n_out, k, fmt, n, m), O.pack_nm(c, keep, n, m))
        assert np.array_equal(meta_rows(to_np(meta), n_out, k), O.pack_bitmap(keep))
    q, g = O.quant_acts(x)
    acc_ref = O.contract(c, q)
    assert np.array_equal(to_np(acc), acc_ref)
    check_y(to_np(y), O.rescale_grouped(acc_ref, betas, rpg, g), acc_ref)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
@pytest.mark.parametrize("n_out,k,rpg", [(64, 128, 1), (300, 1024, 16), (130, 1536, 64), (100, 640, 1000)])
def test_grouped_matches_oracle(n_out, k, rpg, fmt, n, m):
    rng = np.random.default_rng([95, n_out, k, rpg, fmt, n, m])
    bits = synth.gaussian_masters(rng, n_out, k, outlier_frac=0.01)
    x = synth.gaussian_acts(rng, 3, k, hot_channels=2)
    _run(bits, x, n, m, fmt, rpg, "gaussian")


@pytest.mark.parametrize("rpg", [1, 7, 256])
def test_grouped_rare_values(rpg):
    """Zeros, subnormals, tiny and large magnitudes: exact out-of-window sums per group."""
    rng = np.random.default_rng([96, rpg])
    bits = synth.rare_mixture(rng, 260, 512)
    x = synth.gaussian_acts(rng, 2, 512)
    _run(bits, x, 6, 8, FMT_NM, rpg, "rare mixture")


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
@pytest.mark.parametrize("n_out,k,rpg,t", [(300, 640, 1, 40), (520, 1216, 24, 300), (136, 320, 100, 5),
                                           (1100, 512, 257, 17)])
@pytest.mark.parametrize("with_acc", [True, False])
def test_grouped_products_every_path(n_out, k, rpg, t, fmt, n, m, with_acc):
    """beta per row group read by each product kernel's epilogue: the GEMV
    (<= 16 tokens), the int8 MFMA GEMM (DENSE2, 6:8), the 2:4 sparse-MFMA GEMM
    and the generic kernel (5:8), over ragged row and token tiles, with and
    without the int32 output."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([99, n_out, k, rpg, t, fmt, n, m])
    bits = synth.gaussian_masters(rng, n_out, k, outlier_frac=0.01)
    x = synth.gaussian_acts(rng, t, k, hot_channels=2)
    say(f"grouped products {n_out}x{k} rows_per_group={rpg} t={t} {n}:{m} fmt={fmt} acc={with_acc}")
    groups = -(-n_out // rpg)
    beta = torch.empty(groups, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
    ws = torch.empty(sbl.sbl_workspace_bytes_grouped(n_out, k, rpg), dtype=torch.uint8, device="cuda")
    sbl.sbl_quant_weights_grouped(to_dev(bits), n, m, rpg, beta, ws, fmt=fmt, packed=packed, meta=meta)
    xq, gamma = sbl.quant_acts(to_dev(x.astype(np.float32)))
    y = torch.full((t, n_out), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.empty((t, n_out), dtype=torch.int32, device="cuda") if with_acc else None
    sbl.sbl_linear_grouped(packed, meta, fmt, n, m, beta, rpg, xq, gamma, n_out, y, acc)
    torch.cuda.synchronize()
    betas, keep, c = O.quant_weights_grouped(bits, n, m, rpg)
    assert np.array_equal(to_np(beta), betas)
    q, g = O.quant_acts(x)
    acc_ref = O.contract(c, q)
    if with_acc:
        assert np.array_equal(to_np(acc), acc_ref)
    check_y(to_np(y), O.rescale_grouped(acc_ref, betas, rpg, g), acc_ref)


def test_grouped_large_groups_decode_and_prefill():
    """Groups spanning many absmean workgroups; GEMV (4 tokens) and GEMM (40 tokens) products."""
    rng = np.random.default_rng(97)
    bits = synth.gaussian_masters(rng, 2048, 4096)
    for t in (4, 40):
        _run(bits, synth.gaussian_acts(rng, t, 4096), 6, 8, FMT_NM, 512, f"{t} tokens")


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
@pytest.mark.parametrize("n_out,k,kg,t,rpg", [(64, 256, 64, 3, 64), (130, 1536, 512, 5, 16), (100, 640, 128, 1, 1000),
                                               (72, 4096, 4096, 2, 8), (40, 8192, 64, 2, 8)])
def test_activation_groups_match_oracle(n_out, k, kg, t, rpg, fmt, n, m):
    """gamma per token and block of kg features, beta per row group: xq and gamma
    bit for bit, and y bit for bit (the same fp32 operations in the same order)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([98, n_out, k, kg, t, fmt, n, m])
    bits = synth.gaussian_masters(rng, n_out, k)
    x = synth.gaussian_acts(rng, t, k, hot_channels=3)
    say(f"activation groups {n_out}x{k} kg={kg} t={t} rows_per_group={rpg} {n}:{m} fmt={fmt}")
    groups = -(-n_out // rpg)
    beta = torch.empty(groups, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
    ws = torch.empty(sbl.sbl_workspace_bytes_grouped(n_out, k, rpg), dtype=torch.uint8, device="cuda")
    sbl.sbl_quant_weights_grouped(to_dev(bits), n, m, rpg, beta, ws, fmt=fmt, packed=packed, meta=meta)
    xq = torch.empty((t, k), dtype=torch.int8, device="cuda")
    gamma = torch.empty((t, k // kg), dtype=torch.float32, device="cuda")
    sbl.sbl_quant_acts_kgrouped(to_dev(x.astype(np.float32)), kg, xq, gamma)
    y = torch.empty((t, n_out), dtype=torch.float32, device="cuda")
    sbl.sbl_linear_kgrouped(packed, meta, fmt, n, m, beta, rpg, xq, gamma, kg, n_out, y)
    torch.cuda.synchronize()
    q, g = O.quant_acts_kgrouped(x, kg)
    assert np.array_equal(to_np(xq), q) and np.array_equal(to_np(gamma), g)
    betas, keep, codes = O.quant_weights_grouped(bits, n, m, rpg)
    assert np.array_equal(to_np(beta), betas)
    _, y_ref = O.linear_kgrouped(codes, q, betas, rpg, g, kg)
    assert np.array_equal(to_np(y), y_ref)


@pytest.mark.parametrize("rpg", [1, 128])
@pytest.mark.parametrize("idx", [4, 6])
def test_group_scales_at_benchmark_shapes(idx, rpg):
    """The group-scale benchmark's configuration: a 3B-class gate (8640 x 3200)
    or down (3200 x 8640) matrix of the decode workload, 6:8 N:M, M = 1.
    Weights and the beta-per-row-group product against the oracle in full,
    then the activation-group product (gamma per 320 features) bit for bit."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    name, n_out, k = synth.block_shapes(3200, 8640)[idx]
    bits = synth.workload_masters("b3", idx, n_out, k)
    x = synth.workload_acts("b3", idx, 1, k)
    _run(bits, x, 6, 8, FMT_NM, rpg, f"3B {name}")
    kg = 320
    say(f"activation groups 3B {name} kg={kg} rows_per_group={rpg}")
    groups = -(-n_out // rpg)
    beta = torch.empty(groups, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, 6, 8, FMT_NM), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    ws = torch.empty(sbl.sbl_workspace_bytes_grouped(n_out, k, rpg), dtype=torch.uint8, device="cuda")
    sbl.sbl_quant_weights_grouped(to_dev(bits), 6, 8, rpg, beta, ws, fmt=FMT_NM, packed=packed, meta=meta)
    xq = torch.empty((1, k), dtype=torch.int8, device="cuda")
    gamma = torch.empty((1, k // kg), dtype=torch.float32, device="cuda")
    sbl.sbl_quant_acts_kgrouped(to_dev(x.astype(np.float32)), kg, xq, gamma)
    y = torch.empty((1, n_out), dtype=torch.float32, device="cuda")
    sbl.sbl_linear_kgrouped(packed, meta, FMT_NM, 6, 8, beta, rpg, xq, gamma, kg, n_out, y)
    torch.cuda.synchronize()
    q, g = O.quant_acts_kgrouped(x, kg)
    assert np.array_equal(to_np(xq), q) and np.array_equal(to_np(gamma), g)
    betas, keep, codes = O.quant_weights_grouped(bits, 6, 8, rpg)
    _, y_ref = O.linear_kgrouped(codes, q, betas, rpg, g, kg)
    assert np.array_equal(to_np(y), y_ref)


# ---- block scales: one beta per block of rows x features ----

def _run_blocked(bits, x, n, m, fmt, rpg, cpg, label):
    """sbl_quant_weights_blocked (twice, one workspace) and sbl_linear_blocked
    against the oracle: beta, mask, codes, packed bytes and metadata bit for
    bit; y bit for bit (the same fp32 operations in the same order)."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = bits.shape
    gr, gk = -(-n_out // rpg), k // cpg
    say(f"block scales {label} {n_out}x{k} rows_per_group={rpg} cols_per_group={cpg} {n}:{m} fmt={fmt}")
    beta = torch.full((gr, gk), -1.0, device="cuda")
    mask = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    codes = torch.empty((n_out, k), dtype=torch.int8, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
    ws = torch.full((sbl.sbl_workspace_bytes_blocked(n_out, k, rpg, cpg),), 0xFF, dtype=torch.uint8, device="cuda")
    w = to_dev(bits)
    for _ in range(2):
        sbl.sbl_quant_weights_blocked(w, n, m, rpg, cpg, beta, ws, mask_bits=mask, codes=codes, fmt=fmt,
                                      packed=packed, meta=meta)
    t = x.shape[0]
    xq = torch.empty((t, k), dtype=torch.int8, device="cuda")
    gamma = torch.empty((t, gk), dtype=torch.float32, device="cuda")
    sbl.sbl_quant_acts_kgrouped(to_dev(x.astype(np.float32)), cpg, xq, gamma)
    y = torch.full((t, n_out), float("nan"), dtype=torch.float32, device="cuda")
    sbl.sbl_linear_blocked(packed, meta, fmt, n, m, beta, rpg, xq, gamma, cpg, n_out, y)
    torch.cuda.synchronize()
    betas, keep, c = O.quant_weights_blocked(bits, n, m, rpg, cpg)
    assert np.array_equal(to_np(beta), betas)
    assert np.array_equal(to_np(mask), O.pack_bitmap(keep))
    assert np.array_equal(to_np(codes), c)
    if fmt == FMT_DENSE2:
        assert np.array_equal(packed_rows(to_np(packed), n_out, k, fmt, n, m), O.pack_dense2(c))
    else:
        if (k * n // m) % 4 == 0:
            assert np.array_equal(packed_rows(to_np(packed), n_out, k, fmt, n, m), O.pack_nm(c, keep, n, m))
        assert np.array_equal(meta_rows(to_np(meta), n_out, k), O.pack_bitmap(keep))
    q, g = O.quant_acts_kgrouped(x, cpg)
    assert np.array_equal(to_np(xq), q) and np.array_equal(to_np(gamma), g)
    _, y_ref = O.linear_kgrouped(c, q, betas, rpg, g, cpg)
    assert np.array_equal(to_np(y), y_ref)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4), (FMT_NM, 5, 8)])
@pytest.mark.parametrize("n_out,k,rpg,cpg,t", [(64, 256, 1, 64, 2), (130, 1536, 16, 512, 3), (100, 640, 1000, 128, 1),
                                               (300, 2048, 128, 256, 5), (37, 4096, 37, 4096, 2)])
def test_block_scales_match_oracle(n_out, k, rpg, cpg, t, fmt, n, m):
    """Blocks held by one absmean workgroup and blocks split over several (300 x
    2048 with 128 x 256 blocks: 32768 values each), a ragged last row block, and
    blocks spanning k (the row-group case)."""
    rng = np.random.default_rng([99, n_out, k, rpg, cpg, fmt, n, m])
    bits = synth.gaussian_masters(rng, n_out, k, outlier_frac=0.01)
    x = synth.gaussian_acts(rng, t, k, hot_channels=2)
    _run_blocked(bits, x, n, m, fmt, rpg, cpg, "gaussian")


@pytest.mark.parametrize("rpg,cpg", [(1, 64), (7, 128), (260, 256)])
def test_block_scales_rare_values(rpg, cpg):
    """Zeros, subnormals, tiny and large magnitudes: exact out-of-window sums per block."""
    rng = np.random.default_rng([100, rpg, cpg])
    bits = synth.rare_mixture(rng, 260, 512)
    x = synth.gaussian_acts(rng, 2, 512)
    _run_blocked(bits, x, 6, 8, FMT_NM, rpg, cpg, "rare mixture")


@pytest.mark.parametrize("idx", [4, 6])
def test_block_scales_at_benchmark_shapes(idx):
    """A 3B-class gate (8640 x 3200) or down (3200 x 8640) matrix of the decode
    workload, 6:8 N:M, M = 1, beta per 128 rows x 320 features."""
    name, n_out, k = synth.block_shapes(3200, 8640)[idx]
    bits = synth.workload_masters("b3", idx, n_out, k)
    x = synth.workload_acts("b3", idx, 1, k)
    _run_blocked(bits, x, 6, 8, FMT_NM, 128, 320, f"3B {name}")
