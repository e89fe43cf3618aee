"""Parity at the full sizes of the benchmark configurations, in the launch
configuration bench.py times: one grouped weight-preparation call over the
block's matrices, one activation quantization per input and one grouped
product per input group.

At these sizes the oracle checks:
  * beta exactly, over every master weight of every matrix;
  * mask bits and packed bytes (codes + metadata) on sampled rows;
  * int8 activations and gamma for every token;
  * int32 acc bit for bit and fp32 y within the 1e-6 relative bound, on the
    sampled rows times every token (decode) or sampled tokens (prefill).
"""

import functools

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, check_y, meta_rows, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

GROUPS = [[0, 1, 2], [3], [4, 5], [6]]        # q/k/v, o, gate/up, down share an input


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from sparse_linear_layers_absmean_amd import sbl
    sbl.load()


@functools.lru_cache(maxsize=8)
def masters(wname, i, n_out, k):
    return synth.workload_masters(wname, i, n_out, k)


@functools.lru_cache(maxsize=4)
def acts(wname, i, m_tok, k):
    return synth.workload_acts(wname, i, m_tok, k)


def run_block(wname, h, f, m_tok, fmt, n, m, which=None, n_rows=40, n_toks=48):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    mats = synth.block_shapes(h, f)
    which = list(range(len(mats))) if which is None else which
    rng = np.random.default_rng([99, h, m_tok, fmt, n, m])
    say(f"full-size {wname} m_tok={m_tok} fmt={fmt} {n}:{m} matrices={which}")
    items, host = [], {}
    for i in which:
        _, no, k = mats[i]
        bits = masters(wname, i, no, k)
        host[i] = bits
        items.append(dict(
            w=to_dev(bits), beta=torch.empty(1, dtype=torch.float32, device="cuda"),
            mask_bits=torch.empty((no, k // 8), dtype=torch.uint8, device="cuda"),
            packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device="cuda"),
            meta=torch.empty((no, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None,
            workspace=sbl.new_workspace(no, k)))
    sbl.sbl_quant_weights_batch(items, n, m, fmt)
    by = dict(zip(which, items))
    # one input per group, as in a transformer block
    results = {}
    for grp in GROUPS:
        members = [i for i in grp if i in by]
        if not members:
            continue
        k = mats[members[0]][2]
        x = acts(wname, grp[0], m_tok, k)
        xq, gamma = sbl.quant_acts(to_dev(x))
        lin = []
        for i in members:
            no = mats[i][1]
            it = by[i]
            lin.append(dict(packed=it["packed"], meta=it["meta"], beta=it["beta"], xq=xq, gamma=gamma,
                            n_out=no, y=torch.empty((m_tok, no), dtype=torch.float32, device="cuda"),
                            acc=torch.empty((m_tok, no), dtype=torch.int32, device="cuda")))
        sbl.sbl_linear_batch(lin, fmt, n, m)
        torch.cuda.synchronize()
        q_ref, g_ref = O.quant_acts(x)
        assert np.array_equal(to_np(xq), q_ref)
        assert np.array_equal(to_np(gamma), g_ref)
        toks = np.arange(m_tok) if m_tok <= n_toks else np.unique(
            np.concatenate([[0, m_tok - 1], rng.choice(m_tok, n_toks - 2, replace=False)]))
        for i, it in zip(members, lin):
            results[i] = (it, q_ref[toks], g_ref[toks], toks)
    torch.cuda.synchronize()
    for i in which:
        _, no, k = mats[i]
        bits = host[i]
        it = by[i]
        beta = O.absmean_beta(bits)
        assert to_np(it["beta"])[0] == beta, (i, to_np(it["beta"])[0], beta)
        rows = np.unique(np.concatenate([[0, no - 1], rng.choice(no, n_rows - 2, replace=False)]))
        keep = O.nm_keep(bits[rows], n, m)
        codes = O.ternarize(bits[rows], beta) * keep.astype(np.int8)
        bitmap = O.pack_bitmap(keep)
        rows_t = torch.from_numpy(rows).cuda()
        assert np.array_equal(to_np(it["mask_bits"][rows_t]), bitmap), i
        packed = packed_rows(to_np(it["packed"]), no, k, fmt, n, m, rows=rows)
        if fmt == FMT_DENSE2:
            assert np.array_equal(packed, O.pack_dense2(codes)), i
        else:
            assert np.array_equal(packed, O.pack_nm(codes, keep, n, m)), i
            assert np.array_equal(meta_rows(to_np(it["meta"]), no, k, rows=rows), bitmap), i
        lin, q_s, g_s, toks = results[i]
        toks_t = torch.from_numpy(toks).cuda()
        acc = to_np(lin["acc"][toks_t][:, rows_t])
        y = to_np(lin["y"][toks_t][:, rows_t])
        acc_ref, y_ref = O.linear(codes, q_s, beta, g_s)
        assert np.array_equal(acc, acc_ref), i
        check_y(y, y_ref, acc_ref)


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4)])
def test_decode_0p7b_block(fmt, n, m):
    run_block("b0p7", 1536, 4096, 1, fmt, n, m)


@pytest.mark.parametrize("m_tok", [1, 4, 8])
@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_DENSE2, 6, 8)])
def test_decode_3b_block(fmt, n, m, m_tok):
    run_block("b3", 3200, 8640, m_tok, fmt, n, m)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8)])
def test_prefill_3b_block(fmt, n, m):
    run_block("b3_prefill", 3200, 8640, 2048, fmt, n, m)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8)])
def test_train_13b_block_with_ties(fmt, n, m):
    """Per-step weight preparation with many planted ties, then the forward
    product at M = 4096 tokens (q, o and the gate/down shapes)."""
    run_block("b13", 5120, 13824, 4096, fmt, n, m, which=[0, 3, 4, 6])


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8)])
def test_decode_70b_block(fmt, n, m):
    """One matrix of each shape of a 70B-class block (q 8192x8192, gate
    28672x8192, down 8192x28672); the others repeat these shapes."""
    run_block("b70", 8192, 28672, 1, fmt, n, m, which=[0, 4, 6])
