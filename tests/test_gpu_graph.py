"""HIP-graph replay of a whole step (weight preparation, activation quantization,
grouped products), as the benchmark times it: every replay, with eager work
and synchronizations between replays, must reproduce the eager results bit
for bit, and the eager results must match the CPU oracle."""

import numpy as np
import pytest

import synth
from gpu_util import FMT_DENSE2, FMT_NM, check_y, oracle_forward, packed_rows, say, to_dev, to_np
from oracle import sbl_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from sparse_linear_layers_absmean_amd import sbl
    sbl.load()


@pytest.mark.parametrize("fmt,n,m,m_tok", [(FMT_NM, 6, 8, 1), (FMT_DENSE2, 6, 8, 4), (FMT_NM, 2, 4, 40)])
def test_step_graph_replays_match_eager(fmt, n, m, m_tok):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([41, fmt, n, m, m_tok])
    shapes = [(192, 256), (320, 256), (256, 640)]          # two share an input, one has its own
    bits = [synth.gaussian_masters(rng, no, k) for no, k in shapes]
    xs_np = [synth.gaussian_acts(rng, m_tok, 256), synth.gaussian_acts(rng, m_tok, 640)]
    groups = [[0, 1], [2]]
    w = [to_dev(b) for b in bits]
    xs = [to_dev(x) for x in xs_np]
    outs = []
    for no, k in shapes:
        outs.append(dict(
            beta=torch.empty(1, dtype=torch.float32, device="cuda"),
            packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device="cuda"),
            meta=torch.empty((no, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None,
            ws=sbl.new_workspace(no, k),
            y=torch.empty((m_tok, no), dtype=torch.float32, device="cuda"),
            acc=torch.empty((m_tok, no), dtype=torch.int32, device="cuda"), n_out=no))
    acts = [dict(xq=torch.empty((m_tok, x.shape[1]), dtype=torch.int8, device="cuda"),
                 gamma=torch.empty(m_tok, dtype=torch.float32, device="cuda")) for x in xs]

    def step():
        sbl.sbl_quant_weights_batch(
            [dict(w=w[i], beta=o["beta"], packed=o["packed"], meta=o["meta"], workspace=o["ws"])
             for i, o in enumerate(outs)], n, m, fmt)
        for gi, grp in enumerate(groups):
            sbl.sbl_quant_acts(xs[gi], acts[gi]["xq"], acts[gi]["gamma"])
            sbl.sbl_linear_batch([dict(packed=outs[i]["packed"], meta=outs[i]["meta"],
                                       beta=outs[i]["beta"], xq=acts[gi]["xq"],
                                       gamma=acts[gi]["gamma"], n_out=outs[i]["n_out"],
                                       y=outs[i]["y"], acc=outs[i]["acc"]) for i in grp], fmt, n, m)

    def snapshot():
        torch.cuda.synchronize()
        snap = [{key: to_np(v).copy() for key, v in o.items() if key in ("beta", "packed", "meta", "y", "acc")
                 and v is not None} for o in outs]
        snap += [{key: to_np(v).copy() for key, v in a.items()} for a in acts]
        return snap

    def clear():
        for o in outs:
            for key in ("beta", "packed", "meta", "y", "acc"):
                if o[key] is not None:
                    o[key].zero_()
        for a in acts:
            a["xq"].zero_()
            a["gamma"].zero_()

    say(f"graph eager fmt={fmt} {n}:{m} m_tok={m_tok}")
    step()
    eager = snapshot()
    for i, (no, k) in enumerate(shapes):
        gi = 0 if i in groups[0] else 1
        r = oracle_forward(bits[i], xs_np[gi], n, m)
        assert eager[i]["beta"][0] == r["beta"]
        assert np.array_equal(eager[i]["acc"], r["acc"])
        check_y(eager[i]["y"], r["y"], r["acc"])
        want = O.pack_dense2(r["codes"]) if fmt == FMT_DENSE2 else r["nm"]
        assert np.array_equal(packed_rows(eager[i]["packed"], no, k, fmt, n, m), want)

    g = torch.cuda.CUDAGraph()
    clear()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        clear()                                     # eager work between replays
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        got = snapshot()
        for a, b in zip(got, eager):
            for key in b:
                assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (rep, key)
        if rep == 1:                                # an eager step between replays
            step()
            torch.cuda.synchronize()


@pytest.mark.parametrize("m_tok", [3, 40])
def test_group_scale_graph_replays_match_eager(m_tok):
    """Group scales in a graph: beta per row (one wave per group), beta per
    block of rows x features (partial sums through the workspace), the
    products with beta per row (GEMV or GEMM epilogue) and with beta per
    block and gamma per feature block; every replay equals the eager step."""
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    rng = np.random.default_rng([42, m_tok])
    n_out, k, rpg, bk_rows, kg = 300, 1024, 1, 128, 256
    bits = synth.gaussian_masters(rng, n_out, k, outlier_frac=0.01)
    x_np = synth.gaussian_acts(rng, m_tok, k, hot_channels=2)
    w, x = to_dev(bits), to_dev(x_np)
    pb = sbl.sbl_packed_bytes(n_out, k, 6, 8, FMT_NM)
    gr, gk = -(-n_out // bk_rows), k // kg
    buf = dict(
        beta_r=torch.empty(n_out, device="cuda"), packed_r=torch.empty(pb, dtype=torch.uint8, device="cuda"),
        meta_r=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda"),
        beta_b=torch.empty((gr, gk), device="cuda"), packed_b=torch.empty(pb, dtype=torch.uint8, device="cuda"),
        meta_b=torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda"),
        xq=torch.empty((m_tok, k), dtype=torch.int8, device="cuda"), gamma=torch.empty(m_tok, device="cuda"),
        xqk=torch.empty((m_tok, k), dtype=torch.int8, device="cuda"), gammak=torch.empty((m_tok, gk), device="cuda"),
        y_r=torch.empty((m_tok, n_out), device="cuda"), y_b=torch.empty((m_tok, n_out), device="cuda"))
    ws_r = torch.empty(sbl.sbl_workspace_bytes_grouped(n_out, k, rpg), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(sbl.sbl_workspace_bytes_blocked(n_out, k, bk_rows, kg), dtype=torch.uint8, device="cuda")

    def step():
        sbl.sbl_quant_weights_grouped(w, 6, 8, rpg, buf["beta_r"], ws_r, fmt=FMT_NM, packed=buf["packed_r"],
                                      meta=buf["meta_r"])
        sbl.sbl_quant_weights_blocked(w, 6, 8, bk_rows, kg, buf["beta_b"], ws_b, fmt=FMT_NM, packed=buf["packed_b"],
                                      meta=buf["meta_b"])
        sbl.sbl_quant_acts(x, buf["xq"], buf["gamma"])
        sbl.sbl_linear_grouped(buf["packed_r"], buf["meta_r"], FMT_NM, 6, 8, buf["beta_r"], rpg, buf["xq"],
                               buf["gamma"], n_out, buf["y_r"])
        sbl.sbl_quant_acts_kgrouped(x, kg, buf["xqk"], buf["gammak"])
        sbl.sbl_linear_blocked(buf["packed_b"], buf["meta_b"], FMT_NM, 6, 8, buf["beta_b"], bk_rows, buf["xqk"],
                               buf["gammak"], kg, n_out, buf["y_b"])

    def snapshot():
        torch.cuda.synchronize()
        return {key: to_np(v).copy() for key, v in buf.items()}

    say(f"group-scale graph eager m_tok={m_tok}")
    step()
    eager = snapshot()
    betas, keep, codes = O.quant_weights_grouped(bits, 6, 8, rpg)
    assert np.array_equal(eager["beta_r"], betas)
    q, g = O.quant_acts(x_np)
    acc = O.contract(codes, q)
    check_y(eager["y_r"], O.rescale_grouped(acc, betas, rpg, g), acc)
    bb, keepb, codesb = O.quant_weights_blocked(bits, 6, 8, bk_rows, kg)
    assert np.array_equal(eager["beta_b"], bb)
    qk, gk_ref = O.quant_acts_kgrouped(x_np, kg)
    _, yb = O.linear_kgrouped(codesb, qk, bb, bk_rows, gk_ref, kg)
    assert np.array_equal(eager["y_b"], yb)

    graph = torch.cuda.CUDAGraph()
    for v in buf.values():
        v.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for v in buf.values():                      # eager work between replays
            v.zero_()
        torch.cuda.synchronize()
        say(f"group-scale graph replay {rep}")
        graph.replay()
        got = snapshot()
        for key, want in eager.items():
            assert np.array_equal(got[key].view(np.uint8), want.view(np.uint8)), (rep, key)
        if rep == 1:
            step()
            torch.cuda.synchronize()
