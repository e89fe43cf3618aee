"""Parity at the full sizes of the benchmark configurations, in the launch
configuration bench.py times: one grouped weight-preparation call over the
block's matrices, one activation quantization per input and one grouped
product per input group.

Everything is compared element by element with the oracle:
  * beta exactly, over every master weight of every matrix;
  * every row of the mask bits, the packed bytes (codes + metadata, in their
    panel-major storage) and, through them, the ternary codes;
  * int8 activations and gamma for every token;
  * int32 acc bit for bit and fp32 y within the 1e-6 relative bound, for
    every row and every token.
The 13B-class block runs all 7 matrices; the 70B-class block runs one matrix
of each of its three shapes (q/k/v/o, gate/up, down), all rows.

The oracle runs row blocks of a matrix on a thread pool (NumPy releases the
interpreter lock in these array operations); each block is an unchanged
oracle call, and rows are independent in the mask, the codes and the packing.
"""

import numpy as np
import pytest

import synth
from gpu_util import (FMT_DENSE2, FMT_NM, check_y, oracle_packed_panels, oracle_weight_rows, par_map,
                      say, to_dev, to_np)
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu

GROUPS = [[0, 1, 2], [3], [4, 5], [6]]        # q/k/v, o, gate/up, down share an input

_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from sparse_linear_layers_absmean_amd import sbl
    sbl.load()


def _cached(key, make):
    """Keep the inputs and oracle results of one block (several tests reuse
    them); drop another block's when a new one comes."""
    block = key[0]
    if _CACHE.get("_block") != block:
        _CACHE.clear()
        _CACHE["_block"] = block
    if key not in _CACHE:
        _CACHE[key] = make()
    return _CACHE[key]


def masters_all(wname, mats, which):
    def make():
        got = par_map(lambda i: synth.workload_masters(wname, i, mats[i][1], mats[i][2]), which)
        return dict(zip(which, got))
    return _cached((wname, "masters", tuple(which)), make)


def oracle_weights(wname, i, bits, n, m):
    """(beta, keep, codes) of matrix i: the method's quant-then-mask."""
    def make():
        beta = O.absmean_beta(bits)
        keep, codes = oracle_weight_rows(bits, beta, n, m)
        return beta, keep, codes
    return _cached((wname, "weights", i, n, m), make)


def acts(wname, i, m_tok, k):
    return _cached((wname, "acts", i, m_tok, k), lambda: synth.workload_acts(wname, i, m_tok, k))


def run_block(wname, h, f, m_tok, fmt, n, m, which=None):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    mats = synth.block_shapes(h, f)
    which = list(range(len(mats))) if which is None else which
    say(f"full-size {wname} m_tok={m_tok} fmt={fmt} {n}:{m} matrices={which}")
    host = masters_all(wname, mats, which)
    items = []
    for i in which:
        _, no, k = mats[i]
        items.append(dict(
            w=to_dev(host[i]), beta=torch.empty(1, dtype=torch.float32, device="cuda"),
            mask_bits=torch.empty((no, k // 8), dtype=torch.uint8, device="cuda"),
            packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device="cuda"),
            meta=torch.empty((no, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None,
            workspace=sbl.new_workspace(no, k)))
    sbl.sbl_quant_weights_batch(items, n, m, fmt)
    by = dict(zip(which, items))
    inputs = {}
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
        for i, it in zip(members, lin):
            inputs[i] = (it, x, xq, gamma)
    torch.cuda.synchronize()
    say("  GPU done; comparing with the oracle")
    for i in which:
        _, no, k = mats[i]
        it = by[i]
        beta, keep, codes = oracle_weights(wname, i, host[i], n, m)
        assert to_np(it["beta"])[0] == beta, (i, to_np(it["beta"])[0], beta)
        assert np.array_equal(to_np(it["mask_bits"]), O.pack_bitmap(keep)), i
        packed_ref, meta_ref = oracle_packed_panels(codes, keep, fmt, n, m)
        assert np.array_equal(to_np(it["packed"]), packed_ref), i
        if fmt == FMT_NM:
            assert np.array_equal(to_np(it["meta"]).reshape(-1), meta_ref), i
        lin, x, xq, gamma = inputs[i]
        q_ref, g_ref = O.quant_acts(x)
        assert np.array_equal(to_np(xq), q_ref), i
        assert np.array_equal(to_np(gamma), g_ref), i
        acc_ref, y_ref = O.linear(codes, q_ref, beta, g_ref)
        assert np.array_equal(to_np(lin["acc"]), acc_ref), i
        check_y(to_np(lin["y"]), y_ref, acc_ref)
        say(f"  matrix {i} ({no}x{k}): every element equal")


@pytest.mark.parametrize("fmt,n,m", [(FMT_DENSE2, 6, 8), (FMT_NM, 6, 8), (FMT_NM, 2, 4)])
def test_decode_0p7b_block(fmt, n, m):
    run_block("b0p7", 1536, 4096, 1, fmt, n, m)


@pytest.mark.parametrize("m_tok", [1, 4, 8])
@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_NM, 2, 4), (FMT_DENSE2, 6, 8)])
def test_decode_3b_block(fmt, n, m, m_tok):
    run_block("b3", 3200, 8640, m_tok, fmt, n, m)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8), (FMT_NM, 2, 4)])
def test_prefill_3b_block(fmt, n, m):
    """2048 tokens: the dense int8 MFMA GEMM (6:8, DENSE2) and the 2:4 GEMM on
    the sparse MFMA, at the shapes and grouping the benchmark times."""
    run_block("b3_prefill", 3200, 8640, 2048, fmt, n, m)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8)])
def test_train_13b_block_with_ties(fmt, n, m):
    """Per-step weight preparation over all 7 matrices, with ties planted on
    the 6:8 keep boundary, then the forward product at M = 4096 tokens."""
    run_block("b13", 5120, 13824, 4096, fmt, n, m)


@pytest.mark.parametrize("fmt,n,m", [(FMT_NM, 6, 8), (FMT_DENSE2, 6, 8)])
def test_decode_70b_block(fmt, n, m):
    """One matrix of each shape of a 70B-class block (q 8192x8192, gate
    28672x8192, down 8192x28672), every row; the others repeat these shapes."""
    run_block("b70", 8192, 28672, 1, fmt, n, m, which=[0, 4, 6])
