#!/usr/bin/env python3
"""Benchmark of the Sparse-BitLinear hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for
each of the 7 matrices of a transformer block (q, k, v, o, gate, up, down)
  sbl_quant_weights      exact absmean beta + N:M mask from the BF16 masters +
                         ternary codes + packing (the per-training-step recompute)
  sbl_linear_acts_batch  per input of the block (q/k/v, o, gate/up, down): its
                         per-token absmax int8 quantization and the ternary x
                         int8 products + fp32 rescale that read it (one fused
                         GEMV launch at decode sizes)
Default workload: decode of a 0.7B-class block (hidden 1536, FFN 4096), one
token, 6:8 N:M format.  Inputs are seeded synthetic data resident in HBM; the
steps rotate over enough distinct copies (>= 512 MB) that the 256 MB
Infinity Cache cannot serve a step from the previous one.

Printed: one JSON line.  `value` is the step's algorithmic bytes (BF16
masters read once, packed codes written and read, activations, outputs) per
second; the `roofline*` objects give per-kernel rates from HIP-event timing of
back-to-back launches; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sparse-BitLinear GEMV weight GB/s + prefill int8 TOPS, as % of MI355X peak"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0

FORMATS = {"dense2": (0, 6, 8), "nm68": (1, 6, 8), "nm24": (1, 2, 4)}

WORKLOADS = {
    # name: (synth workload, hidden, ffn, m_tok, description)
    "decode_0p7b": ("b0p7", 1536, 4096, 1,
                    "Decode GEMV, M=1 token, 0.7B-class block: hidden 1536, FFN 4096"),
    "decode_3b": ("b3", 3200, 8640, 1, "Decode GEMV, 3B-class block: hidden 3200, FFN 8640"),
    "prefill_3b": ("b3_prefill", 3200, 8640, 2048,
                   "Prefill GEMM, M=2048 tokens, 3B-class block: hidden 3200, FFN 8640"),
    "train_13b": ("b13", 5120, 13824, 4096,
                  "Training-step path, 13B-class block: hidden 5120, FFN 13824, M=4096"),
    "decode_70b": ("b70", 8192, 28672, 1, "Decode GEMV, M=1, 70B-class block: hidden 8192, FFN 28672"),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_0p7b", choices=sorted(WORKLOADS))
    p.add_argument("--fmt", default="nm68", choices=sorted(FORMATS))
    p.add_argument("--m-tok", type=int, default=None)
    p.add_argument("--pool-mb", type=float, default=560.0,
                   help="minimum bytes of distinct BF16 master copies the steps rotate over")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-group-scales", action="store_true", help="skip the group-scale timings")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill GEMM measurement")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-qw-sweep", action="store_true", help="skip the weight-preparation sweep")
    p.add_argument("--no-gemv-sweep", action="store_true",
                   help="skip the GEMV weight-bandwidth table over the decode configurations")
    p.add_argument("--copy-calibration-mb", type=float, default=0.0,
                   help="before the run, copy a buffer of this many MB 3 times (a known-size copy "
                        "kernel for scaling hardware byte counters)")
    return p.parse_args()


def recorded_traffic(call, workload, fmt):
    """HBM bytes per call from the committed counter summary (profiles/traffic.json),
    or None when there is none for this workload and format or when any kernel
    source it was taken with has changed since (its SHA-256 differs)."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            rec = json.load(fh)[call]
        if rec.get("workload") != workload or rec.get("format") != fmt:
            return None
        for path, digest in rec["sources_sha256"].items():
            with open(os.path.join(ROOT, path), "rb") as fh:
                if hashlib.sha256(fh.read()).hexdigest() != digest:
                    return None
        return rec["bytes_per_call"]
    except (OSError, KeyError, ValueError):
        return None


def block(h, f):
    import synth
    return synth.block_shapes(h, f)


class Timer:
    """HIP events on torch's current stream (every libsbl launch goes there)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs and is measured on one GPU (asked for --gpus {args.gpus}); "
              "sharding across GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from sparse_linear_layers_absmean_amd import sbl

    sbl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mb > 0:
        nb = int(args.copy_calibration_mb * 1e6) // 16 * 16
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wname, h, f, m_tok, desc = WORKLOADS[args.workload]
    if args.m_tok:
        m_tok = args.m_tok
    fmt, n, m = FORMATS[args.fmt]
    mats = block(h, f)
    block_w = sum(no * k for _, no, k in mats)
    copies = max(2, int(np.ceil(args.pool_mb * 1e6 / (2 * block_w))))
    copies = min(copies, 64)

    # ---------------- inputs: seeded synthetic, resident in HBM
    t0 = time.time()
    masters = [[torch.from_numpy(synth.workload_masters(wname, i, no, k, copy=c).view(np.int16)).to(dev)
                for i, (_, no, k) in enumerate(mats)] for c in range(copies)]
    # a block's matrices read 4 inputs: q/k/v share one, o one, gate/up one, down one
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    xs = [[torch.from_numpy(synth.workload_acts(wname, grp[0], m_tok, mats[grp[0]][2], copy=c)).to(dev)
           for grp in groups] for c in range(copies)]
    gen_s = time.time() - t0

    def alloc_out(no, k):
        pb = sbl.sbl_packed_bytes(no, k, n, m, fmt)
        return dict(beta=torch.empty(1, dtype=torch.float32, device=dev),
                    packed=torch.empty(pb, dtype=torch.uint8, device=dev),
                    meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev) if fmt == 1 else None,
                    y=torch.empty((m_tok, no), dtype=torch.float32, device=dev), n_out=no)

    outs = [[alloc_out(no, k) for (_, no, k) in mats] for _ in range(copies)]
    acts = [[dict(xq=torch.empty((m_tok, mats[grp[0]][2]), dtype=torch.int8, device=dev),
                  gamma=torch.empty(m_tok, dtype=torch.float32, device=dev)) for grp in groups]
            for _ in range(copies)]
    wss = [[sbl.new_workspace(no, k, dev) for (_, no, k) in mats] for _ in range(copies)]

    def items_of(c, gi, pool=None):
        src = outs[c] if pool is None else pool
        return [dict(src[i], xq=acts[c][gi]["xq"], gamma=acts[c][gi]["gamma"]) for i in groups[gi]]

    def qw_all(c, flags=0):
        sbl.sbl_quant_weights_batch(
            [dict(w=masters[c][i], beta=outs[c][i]["beta"], packed=outs[c][i]["packed"],
                  meta=outs[c][i]["meta"], workspace=wss[c][i]) for i in range(len(mats))],
            n, m, fmt, flags=flags)

    def qa_all(c):
        for gi in range(len(groups)):
            sbl.sbl_quant_acts(xs[c][gi], acts[c][gi]["xq"], acts[c][gi]["gamma"])

    def la_all(c, pool=None):
        # per input: its quantization and the products that read it (one fused
        # launch for decode-sized inputs, else sbl_quant_acts + sbl_linear_batch)
        src = outs[c] if pool is None else pool
        for gi in range(len(groups)):
            sbl.sbl_linear_acts_batch(xs[c][gi], acts[c][gi]["xq"], acts[c][gi]["gamma"],
                                      [src[i] for i in groups[gi]], fmt, n, m)

    def step(c):
        qw_all(c)
        la_all(c)

    # ---------------- algorithmic bytes
    def packed_b(no, k):
        return sbl.sbl_packed_bytes(no, k, n, m, fmt) + max(0, sbl.sbl_meta_bytes(no, k, fmt))

    qw_bytes = sum(2 * no * k + packed_b(no, k) for _, no, k in mats)
    qa_bytes = sum(m_tok * mats[grp[0]][2] * 5 + 4 * m_tok for grp in groups)
    lin_bytes = sum(packed_b(no, k) + m_tok * k + 4 * m_tok + 4 * m_tok * no + 4 for _, no, k in mats)
    step_bytes = qw_bytes + qa_bytes + lin_bytes
    weight_bytes = sum(packed_b(no, k) for _, no, k in mats)

    # ---------------- HIP graphs: one per rotation copy, so that host launch
    # overhead stays out of the timed region (the step has no memset nodes)
    def capture(fn):
        fn()                                  # eager run first: every kernel loaded
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    step_graphs = [capture(lambda c=c: step(c)) for c in range(copies)]

    # ---------------- whole-step timing
    for s in range(args.warmup):
        step_graphs[s % copies].replay()
    torch.cuda.synchronize()
    tm = Timer()
    tm.start()
    for s in range(args.steps):
        step_graphs[s % copies].replay()
    step_ms = tm.stop_ms() / args.steps
    torch.cuda.synchronize()

    # ---------------- per-call rates: graphs of one call kind, replayed back to back
    def time_graphs(graphs, reps):
        for r in range(min(reps, len(graphs))):
            graphs[r % len(graphs)].replay()
        torch.cuda.synchronize()
        tm.start()
        for r in range(reps):
            graphs[r % len(graphs)].replay()
        return tm.stop_ms() / reps

    # GEMV pool: distinct packed buffers totalling >= 512 MB (cold Infinity Cache)
    gemv_copies = max(copies, int(np.ceil(560e6 / weight_bytes)))
    gemv_pool = []
    for c in range(gemv_copies):
        gemv_pool.append([dict(o, packed=o["packed"].clone(),
                               meta=o["meta"].clone() if o["meta"] is not None else None)
                          for o in outs[c % copies]])

    def lin_all(c):
        for gi in range(len(groups)):
            sbl.sbl_linear_batch(items_of(c % copies, gi, gemv_pool[c % gemv_copies]), fmt, n, m)

    qw_graphs = [capture(lambda c=c: qw_all(c)) for c in range(copies)]
    qw2_graphs = [capture(lambda c=c: qw_all(c, sbl.SBL_QW_TWO_PASS)) for c in range(copies)]
    qa_graphs = [capture(lambda c=c: qa_all(c)) for c in range(copies)]
    lin_graphs = [capture(lambda c=c: lin_all(c)) for c in range(gemv_copies)]
    la_graphs = [capture(lambda c=c: la_all(c % copies, gemv_pool[c % gemv_copies])) for c in range(gemv_copies)]

    reps = max(20, args.steps)
    qw_ms = time_graphs(qw_graphs, reps)
    qw2_ms = time_graphs(qw2_graphs, reps)
    qa_ms = time_graphs(qa_graphs, reps)
    lin_ms = time_graphs(lin_graphs, max(reps, 2 * gemv_copies))
    la_ms = time_graphs(la_graphs, max(reps, 2 * gemv_copies))

    def roof(bytes_per, ms, kernel, launches, traffic=None):
        gbps = bytes_per / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
                "launches_per_step": launches, "avg_launch_us": round(ms * 1e3 / launches, 3)}

    # the step's two calls, then (for reference) the same work as separate calls
    per_call = {
        "sbl_quant_weights": roof(qw_bytes, qw_ms, "sbl_quant_weights_batch over the 7 matrices in one launch: "
                                  "resident_kernel (masters held in registers while the exact beta completes)",
                                  1, recorded_traffic("sbl_quant_weights", args.workload, args.fmt)),
        "sbl_quant_weights_two_pass": roof(qw_bytes, qw2_ms, "the same call with SBL_QW_TWO_PASS: "
                                           "absmean_partial + mask_pack kernels (masters read twice)", 1),
        "sbl_linear_acts_batch": roof(qa_bytes + lin_bytes, la_ms,
                                      "gemv_kernel with the activation quantization fused in "
                                      "(grouped: qkv, o, gate+up, down)", len(groups)),
        "sbl_quant_acts": roof(qa_bytes, qa_ms, "quant_acts_kernel (separate call)", len(groups)),
        "sbl_linear": roof(lin_bytes, lin_ms, "gemv_kernel (separate call; grouped: qkv, o, gate+up, down)",
                           len(groups)),
    }
    dominant = max(["sbl_quant_weights", "sbl_linear_acts_batch"],
                   key=lambda kk: {"sbl_quant_weights": qw_ms, "sbl_linear_acts_batch": la_ms}[kk])
    gemv_gbps = weight_bytes / (lin_ms * 1e-3) / 1e9

    # ---------------- GEMV weight bandwidth over the decode configurations
    gemv = None
    read_peak = None
    if not args.no_gemv_sweep:
        gemv = gemv_sweep(torch, np, sbl, dev, synth)
        read_peak = stream_read_peak(torch, dev, tm)
        for row in gemv:
            row["frac_of_measured_stream"] = round(row["weight_GBps"] / read_peak["reference_GBps"], 4)
    qw_sweep = None if args.no_qw_sweep else weight_prep_sweep(torch, np, sbl, dev, synth, tm)

    # ---------------- prefill GEMM (3B block, M = 2048 tokens), int8 ops
    prefill = prefill_24 = backward = None
    if not args.no_prefill:
        prefill = bench_prefill(torch, np, synth, sbl, dev, tm)
        prefill_24 = bench_prefill(torch, np, synth, sbl, dev, tm, n=2, m=4)
        backward = bench_backward(torch, np, synth, sbl, dev, tm)
    group_scales = None if args.no_group_scales else bench_group_scales(torch, np, sbl, dev, synth, tm)
    library_gemm = None if args.no_prefill else library_gemm_reference(torch, dev, tm)

    # ---------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(np, synth, wname, mats, m_tok, n, m, fmt, args.cpu_seconds, step_bytes)

    value = step_bytes / (step_ms * 1e-3) / 1e9
    # the GEMV's roofline at the largest decode configuration (70B block, M = 1,
    # this run's format) when the sweep ran; else the step's own GEMV launches
    roofline_gemv = {"bound": "hbm", "achieved": round(gemv_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "workload": desc, "note": "packed weight bytes / sbl_linear_batch time"}
    if gemv:
        big = [g for g in gemv if g["block"] == "70b" and g["format"] == args.fmt and g["m_tok"] == 1]
        if big:
            roofline_gemv = {"bound": "hbm", "achieved": big[0]["weight_GBps"], "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": big[0]["frac"], "traffic": None,
                             "workload": "Decode GEMV, M=1, 70B-class block (hidden 8192, FFN 28672), "
                                         f"{args.fmt}, 4 grouped launches",
                             "note": "packed weight bytes (codes + metadata) / time of the block's launches"}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,0.02) BF16 masters, N(0,1) fp32 activations)",
        "config": {"workload": desc, "format": args.fmt, "m_tok": m_tok, "matrices": len(mats),
                   "block_weights": block_w, "rotation_copies": copies,
                   "step_algorithmic_bytes": step_bytes},
        "roofline": dict(per_call[dominant], call=dominant),
        "roofline_gemv": roofline_gemv,
        "per_call": per_call,
        "gemv": gemv,
        "measured_stream": read_peak,
        "measured_library_gemm": library_gemm,
        "weight_prep": qw_sweep,
        "prefill": prefill,
        "prefill_2of4_sparse_mfma": prefill_24,
        "backward": backward,
        "group_scales": group_scales,
        "cpu_baseline": cpu,
        "input_gen_s": round(gen_s, 1),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


def weight_prep_sweep(torch, np, sbl, dev, synth, tm):
    """sbl_quant_weights_batch over whole blocks (7 matrices, 6:8 N:M output), the per-step
    weight preparation: algorithmic bytes (masters read once + packed codes and metadata
    written) per second.  Masters are N(0, 0.02) BF16 drawn on the device; each block
    rotates over >= 2 distinct copies totalling >= 600 MB; HIP graphs, HIP events."""
    n, m, fmt = 6, 8, 1
    cases = [("0p7b", 1536, 4096), ("3b", 3200, 8640), ("13b", 5120, 13824)]
    out = []
    for wl, h, f in cases:
        mats = synth.block_shapes(h, f)
        bw = sum(no * k for _, no, k in mats)
        copies = max(2, int(np.ceil(600e6 / (2 * bw))))
        g = torch.Generator(device=dev).manual_seed(5)
        pool = []
        for c in range(copies):
            its = []
            for _, no, k in mats:
                w = (torch.randn((no, k), generator=g, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
                its.append(dict(w=w, beta=torch.empty(1, device=dev),
                                packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8,
                                                   device=dev),
                                meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev),
                                workspace=sbl.new_workspace(no, k, dev)))
            pool.append(its)
        graphs = []
        for c in range(copies):
            sbl.sbl_quant_weights_batch(pool[c], n, m, fmt)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                sbl.sbl_quant_weights_batch(pool[c], n, m, fmt)
            graphs.append(gr)
        reps = max(20, 2 * copies)
        for r in range(copies):
            graphs[r].replay()
        torch.cuda.synchronize()
        tm.start()
        for r in range(reps):
            graphs[r % copies].replay()
        us = tm.stop_ms() / reps * 1e3
        alg = sum(2 * no * k + sbl.sbl_packed_bytes(no, k, n, m, fmt) + no * k // 8 for _, no, k in mats)
        gbps = alg / (us * 1e-6) / 1e9
        out.append({"block": wl, "weights": bw, "us_per_call": round(us, 2), "alg_GBps": round(gbps, 1),
                    "frac": round(gbps / HBM_PEAK_GBPS, 4),
                    "path": "one launch (resident_kernel)" if bw * 2 <= 67e6 else "two launches (absmean + mask_pack)"})
        del pool, graphs
        torch.cuda.empty_cache()
    return out


def bench_group_scales(torch, np, sbl, dev, synth, tm, rpg=128, kg=320, n=6, m=8):
    """Group scales on a 3B-class block (hidden 3200, FFN 8640), 6:8 N:M, M = 1: weight
    preparation with beta per block of rows (rows_per_group 1 and rpg), and the decode
    products with beta per row group (sbl_linear_grouped) and with gamma per block of kg
    features as well (sbl_quant_acts_kgrouped + sbl_linear_kgrouped), beside the per-matrix
    sbl_linear (kg = 320 = 5 x 64 divides both k = 3200 and k = 8640).  Each block's calls are
    one HIP graph; every block uses distinct buffers from a pool of >= 600 MB.
    Rates are algorithmic bytes: masters read + packed codes and metadata written for the
    weights, packed codes and metadata read for the products."""
    fmt = 1
    mats = synth.block_shapes(3200, 8640)
    bw = sum(no * k for _, no, k in mats)
    g = torch.Generator(device=dev).manual_seed(7)
    pb = [sbl.sbl_packed_bytes(no, k, n, m, fmt) for _, no, k in mats]
    wbytes = sum(pb) + sum(no * k // 8 for _, no, k in mats)

    def timed(fn, copies, reps):
        graphs = []
        for c in range(copies):
            fn(c)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn(c)
            graphs.append(gr)
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        tm.start()
        for r in range(reps):
            graphs[r % copies].replay()
        us = tm.stop_ms() / reps * 1e3
        del graphs
        return us

    out = {"workload": f"3B-class block (hidden 3200, FFN 8640), {n}:{m} N:M, M=1", "weight_prep": [],
           "products": []}
    copies = max(2, int(np.ceil(600e6 / (2 * bw))))
    masters = [[(torch.randn((no, k), generator=g, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
                for _, no, k in mats] for _ in range(copies)]
    outs = [[dict(packed=torch.empty(pb[i], dtype=torch.uint8, device=dev),
                  meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev)) for i, (_, no, k) in enumerate(mats)]
            for _ in range(copies)]
    for r in (1, rpg):
        betas = [torch.empty(-(-no // r), device=dev) for _, no, k in mats]
        wss = [torch.empty(sbl.sbl_workspace_bytes_grouped(no, k, r), dtype=torch.uint8, device=dev)
               for _, no, k in mats]

        def prep(c):
            for i, (_, no, k) in enumerate(mats):
                sbl.sbl_quant_weights_grouped(masters[c][i], n, m, r, betas[i], wss[i], fmt=fmt,
                                              packed=outs[c][i]["packed"], meta=outs[c][i]["meta"])
        us = timed(prep, copies, max(10, 2 * copies))
        gbps = (2 * bw + wbytes) / (us * 1e-6) / 1e9
        out["weight_prep"].append({"rows_per_group": r, "groups": sum(-(-no // r) for _, no, k in mats),
                                   "us_per_block": round(us, 1), "alg_GBps": round(gbps, 1),
                                   "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    del masters
    torch.cuda.empty_cache()
    # products: the rpg-grouped betas of the last preparation; a pool of packed copies
    pcopies = max(2, int(np.ceil(600e6 / wbytes)))
    pool = [[{k2: v.clone() for k2, v in o.items()} for o in outs[0]] for _ in range(pcopies)]
    beta1 = [b[:1].contiguous() for b in betas]
    xs = [torch.randn((1, k), generator=g, device=dev) for _, no, k in mats]
    acts = [sbl.quant_acts(x) for x in xs]
    gq = [(torch.empty((1, k), dtype=torch.int8, device=dev), torch.empty((1, k // kg), device=dev))
          for _, no, k in mats]
    ys = [torch.empty((1, no), device=dev) for _, no, k in mats]
    accs = [torch.empty((1, no), dtype=torch.int32, device=dev) for _, no, k in mats]

    def plain(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_linear(pool[c][i]["packed"], pool[c][i]["meta"], fmt, n, m, beta1[i], acts[i][0], acts[i][1],
                           no, ys[i], None)

    def grouped(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_linear_grouped(pool[c][i]["packed"], pool[c][i]["meta"], fmt, n, m, betas[i], rpg,
                                   acts[i][0], acts[i][1], no, ys[i], accs[i])

    def kgrouped(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_quant_acts_kgrouped(xs[i], kg, gq[i][0], gq[i][1])
            sbl.sbl_linear_kgrouped(pool[c][i]["packed"], pool[c][i]["meta"], fmt, n, m, betas[i], rpg,
                                    gq[i][0], gq[i][1], kg, no, ys[i])

    for name, fn, what in (("sbl_linear", plain, "per-matrix beta and gamma (one launch per matrix)"),
                           ("sbl_linear_grouped", grouped, f"beta per {rpg} rows: GEMV + grouped rescale"),
                           ("sbl_linear_kgrouped", kgrouped,
                            f"beta per {rpg} rows, gamma per {kg} features: activation quant + product")):
        us = timed(fn, pcopies, max(20, 2 * pcopies))
        gbps = wbytes / (us * 1e-6) / 1e9
        out["products"].append({"call": name, "scales": what, "us_per_block": round(us, 1),
                                "weight_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    del pool, outs
    torch.cuda.empty_cache()
    return out


def stream_read_peak(torch, dev, tm):
    """Measured streaming rates for reference (library kernels, not part of the path),
    HIP events around 10 runs each: torch's fp32 sum over 2 GB (bytes read), and a
    1 GB device-to-device copy (bytes read + written)."""
    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(10):
            fn()
        return tm.stop_ms() / 10

    a = torch.ones(512 << 20, dtype=torch.float32, device=dev)
    sum_gbps = (2 << 30) / (timed(lambda: a.sum()) * 1e-3) / 1e9
    del a
    src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_gbps = (2 << 30) / (timed(lambda: dst.copy_(src)) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"sum_fp32_GBps": round(sum_gbps, 1), "copy_GBps": round(copy_gbps, 1),
            "reference_GBps": round(max(sum_gbps, copy_gbps), 1)}


def library_gemm_reference(torch, dev, tm):
    """Measured matrix-core rates of library GEMMs (references, not part of the path), HIP events
    around 10 runs each, at the 3B-class gate shape with 2048 tokens (2048 x 3200 by 3200 x 8640):
    int8 x int8 -> int32 (torch._int_mm) for the prefill GEMM, and BF16 (torch.matmul, fp32
    accumulation) for the backward's products."""
    m_tok, k, n_out = 2048, 3200, 8640
    flops = 2 * m_tok * k * n_out
    out = {"shape": f"{m_tok} x {k} by {k} x {n_out}"}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(10):
            fn()
        return tm.stop_ms() / 10

    g = torch.Generator(device=dev).manual_seed(3)
    try:
        a = torch.randint(-127, 128, (m_tok, k), generator=g, device=dev, dtype=torch.int8)
        b = torch.randint(-1, 2, (n_out, k), generator=g, device=dev, dtype=torch.int8).t()
        ms = timed(lambda: torch._int_mm(a, b))
        out["int8_TOPS"] = round(flops / (ms * 1e-3) / 1e12, 1)
        out["int8_frac"] = round(flops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
    except (RuntimeError, AttributeError) as e:
        out["int8_error"] = str(e).splitlines()[0][:160]
    a = torch.randn((m_tok, k), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((k, n_out), generator=g, device=dev).to(torch.bfloat16)
    ms = timed(lambda: torch.matmul(a, b))
    out["bf16_TFLOPS"] = round(flops / (ms * 1e-3) / 1e12, 1)
    out["bf16_frac"] = round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    del a, b
    torch.cuda.empty_cache()
    return out


def gemv_sweep(torch, np, sbl, dev, synth):
    """Packed-weight GB/s of the grouped GEMV (sbl_linear_batch, 4 launches per
    block: q/k/v, o, gate/up, down) for the decode configurations.  The packed
    bytes are seeded random (the GEMV's time does not depend on the code
    values); every block uses distinct buffers from a pool of >= 600 MB, so the
    256 MB Infinity Cache cannot serve one launch from the previous one.  Each
    block's 4 launches are one HIP graph; HIP events bracket the replays."""
    cases = [("0p7b", 1536, 4096, 1), ("3b", 3200, 8640, 1), ("3b", 3200, 8640, 4),
             ("3b", 3200, 8640, 8), ("70b", 8192, 28672, 1)]
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    out = []
    for wl, h, f, m_tok in cases:
        mats = synth.block_shapes(h, f)
        for fname, (fmt, n, m) in FORMATS.items():
            nbytes = [sbl.sbl_packed_bytes(no, k, n, m, fmt) for _, no, k in mats]
            mbytes = [no * k // 8 if fmt == 1 else 0 for _, no, k in mats]
            block_bytes = sum(nbytes) + sum(mbytes)
            copies = max(2, int(np.ceil(600e6 / block_bytes)))
            gen = torch.Generator(device=dev).manual_seed(7)
            pool = []
            for _ in range(copies):
                items = []
                for i, (_, no, k) in enumerate(mats):
                    packed = torch.randint(0, 256, (nbytes[i],), dtype=torch.uint8, device=dev, generator=gen)
                    if fmt == 0:
                        packed &= 0x55                            # 2-bit fields u in {0, 1}
                    meta = (torch.randint(0, 256, (no, k // 8), dtype=torch.uint8, device=dev, generator=gen)
                            if fmt == 1 else None)
                    items.append(dict(packed=packed, meta=meta, beta=torch.full((1,), 0.02, device=dev),
                                      n_out=no, y=torch.empty((m_tok, no), device=dev)))
                pool.append(items)
            xs = [torch.randint(-127, 128, (m_tok, mats[grp[0]][2]), dtype=torch.int8, device=dev,
                                generator=gen) for grp in groups]
            gam = torch.ones(m_tok, device=dev)

            def run(c):
                for gi, grp in enumerate(groups):
                    sbl.sbl_linear_batch([dict(pool[c][i], xq=xs[gi], gamma=gam) for i in grp], fmt, n, m)

            graphs = []
            for c in range(copies):
                run(c)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    run(c)
                graphs.append(g)
            reps = max(40, 2 * copies)
            for r in range(copies):
                graphs[r].replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for r in range(reps):
                graphs[r % copies].replay()
            b.record()
            b.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            gbps = block_bytes / (us * 1e-6) / 1e9
            # all HBM bytes of the block's products: weights, int8 activations, gamma, fp32 outputs
            hbm = block_bytes + sum(m_tok * mats[g_[0]][2] + 4 * m_tok for g_ in groups) + \
                sum(4 * m_tok * no for _, no, _k in mats)
            out.append({"block": wl, "format": fname, "m_tok": m_tok, "weight_bytes": block_bytes,
                        "us_per_block": round(us, 2), "weight_GBps": round(gbps, 1),
                        "hbm_GBps": round(hbm / (us * 1e-6) / 1e9, 1),
                        "frac": round(gbps / HBM_PEAK_GBPS, 4)})
            del pool, graphs, xs
            torch.cuda.empty_cache()
    return out


def bench_prefill(torch, np, synth, sbl, dev, tm, n=6, m=8):
    """3B-class block at M = 2048 tokens, N:M n:m weights: sbl_linear (GEMM) TOPS.  2:4 runs on
    the sparse MFMA; its TOPS count the dense-equivalent 2*M*N*K ops and are priced against the
    dense int8 peak."""
    wname, h, f, m_tok = "b3_prefill", 3200, 8640, 2048
    fmt = 1
    mats = synth.block_shapes(h, f)
    items = []
    for i, (_, no, k) in enumerate(mats):
        w = torch.from_numpy(synth.workload_masters(wname, i, no, k).view(np.int16)).to(dev)
        o = sbl.quant_weights(w, n, m, fmt=fmt)
        x = torch.from_numpy(synth.workload_acts(wname, i, m_tok, k)).to(dev)
        xq, gamma = sbl.quant_acts(x)
        y = torch.empty((m_tok, no), dtype=torch.float32, device=dev)
        items.append((o, xq, gamma, y, no, k))
        del w, x

    groups = [[0, 1, 2], [3], [4, 5], [6]]          # q/k/v, o, gate/up, down

    def run():
        for grp in groups:
            sbl.sbl_linear_batch([dict(packed=items[i][0]["packed"], meta=items[i][0]["meta"],
                                       beta=items[i][0]["beta"], xq=items[i][1], gamma=items[i][2],
                                       n_out=items[i][4], y=items[i][3]) for i in grp], fmt, n, m)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    reps = 20
    tm.start()
    for _ in range(reps):
        run()
    ms = tm.stop_ms() / reps
    ops = sum(2 * m_tok * no * k for *_, no, k in items)
    tops = ops / (ms * 1e-3) / 1e12
    kernel = "gemm24_kernel (v_smfmac_i32_16x16x128_i8)" if (n, m) == (2, 4) else "gemm_kernel (v_mfma_i32_32x32x32_i8)"
    return {"workload": f"Prefill GEMM, M=2048 tokens, 3B-class block (hidden 3200, FFN 8640), {n}:{m} N:M",
            "kernel": kernel,
            "ms_per_block": round(ms, 4), "int8_TOPS": round(tops, 2),
            "useful_TOPS": round(tops * n / m, 2),
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": None}}


BF16_PEAK_TFLOPS = 2500.0


def bench_backward(torch, np, synth, sbl, dev, tm, n=6, m=8):
    """Backward of a 3B-class block at M = 2048 tokens, 6:8 weights: sbl_linear_backward (dX and dW
    of the 7 matrices) on the BF16 matrix cores.  Algorithmic flops 2*M*N*K per gradient; dW runs
    three BF16 products per step (x_hat split exactly into three parts), counted separately."""
    wname, h, f, m_tok = "b3_prefill", 3200, 8640, 2048
    fmt = 1
    mats = synth.block_shapes(h, f)
    g = torch.Generator(device=dev).manual_seed(11)
    items = []
    for i, (_, no, k) in enumerate(mats):
        w = torch.from_numpy(synth.workload_masters(wname, i, no, k).view(np.int16)).to(dev)
        o = sbl.quant_weights(w, n, m, fmt=fmt)
        x = torch.from_numpy(synth.workload_acts(wname, i, m_tok, k)).to(dev)
        xq, gamma = sbl.quant_acts(x)
        dy = (torch.randn((m_tok, no), generator=g, device=dev) * 0.05).to(torch.bfloat16)
        dx = torch.empty((m_tok, k), dtype=torch.float32, device=dev)
        dw = torch.empty((no, k), dtype=torch.float32, device=dev)
        items.append((o, x, xq, gamma, dy, dx, dw, no, k))
        del w

    def run(which):
        for o, x, xq, gamma, dy, dx, dw, no, k in items:
            sbl.sbl_linear_backward(dy, o["packed"], o["meta"], fmt, n, m, o["beta"], x, xq, gamma,
                                    dx=dx if which in ("dx", "both") else None,
                                    dw=dw if which in ("dw", "both") else None)

    res = {}
    for which in ("dx", "dw", "both"):
        for _ in range(2):
            run(which)
        torch.cuda.synchronize()
        reps = 5
        tm.start()
        for _ in range(reps):
            run(which)
        res[which] = tm.stop_ms() / reps
    flops = sum(2 * m_tok * no * k for *_, no, k in items)
    tf = {w: (flops * (2 if w == "both" else 1)) / (res[w] * 1e-3) / 1e12 for w in res}
    mfma_tf_dw = 3 * flops / (res["dw"] * 1e-3) / 1e12
    return {"workload": f"Backward (dX and dW), M=2048 tokens, 3B-class block (hidden 3200, FFN 8640), {n}:{m} N:M",
            "kernel": "backward_dx_kernel, backward_dw_kernel (v_mfma_f32_32x32x16_bf16)",
            "ms_per_block": {w: round(v, 3) for w, v in res.items()},
            "algorithmic_TFLOPS": {w: round(v, 1) for w, v in tf.items()},
            "dw_mfma_TFLOPS": round(mfma_tf_dw, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf["both"], 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf["both"] / BF16_PEAK_TFLOPS, 4), "traffic": None}}


def cpu_baseline(np, synth, wname, mats, m_tok, n, m, fmt, budget_s, step_bytes):
    """The CPU oracle, untuned, on the same workload: whole blocks until the
    budget is spent.  Each stage is one oracle call, timed on its own, in the
    order the oracle's quant_weights and linear compose them."""
    from threadpoolctl import threadpool_limits

    from oracle import sbl_oracle as O
    done_bytes, blocks, t_total, weights, ops = 0, 0, 0.0, 0, 0
    stages = dict.fromkeys(("beta", "mask", "codes", "pack", "quant_acts", "contract", "rescale"), 0.0)

    def timed(name, fn, *a):
        t = time.perf_counter()
        r = fn(*a)
        stages[name] += time.perf_counter() - t
        return r

    with threadpool_limits(1):
        while t_total < budget_s and blocks < 3:
            for i, (_, no, k) in enumerate(mats):
                bits = synth.workload_masters(wname, i, no, k)
                first = {0: 0, 1: 0, 2: 0, 3: 3, 4: 4, 5: 4, 6: 6}[i]    # shared block inputs
                x = synth.workload_acts(wname, first, m_tok, k)
                beta = timed("beta", O.absmean_beta, bits)
                keep = timed("mask", O.nm_keep, bits, n, m)
                codes = timed("codes", lambda: (O.ternarize(bits, beta) * keep.astype(np.int8)).astype(np.int8))
                if fmt == 1:
                    timed("pack", lambda: (O.to_panels(O.pack_nm(codes, keep, n, m), 16 * n // m),
                                           O.to_panels(O.pack_bitmap(keep), 8)))
                else:
                    timed("pack", lambda: O.to_panels(O.pack_dense2(codes), 16))
                q, gamma = timed("quant_acts", O.quant_acts, x)
                acc = timed("contract", O.contract, codes, q)
                timed("rescale", O.rescale, acc, beta, gamma)
                weights += no * k
                ops += 2 * m_tok * no * k
            blocks += 1
            done_bytes += step_bytes
            t_total = sum(stages.values())
    gbps = done_bytes / t_total / 1e9
    try:
        model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except (OSError, StopIteration):
        model = None
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{blocks} full block step(s) of the same workload ({len(mats)} matrices), "
                      f"{t_total:.1f} s single-threaded NumPy",
            "stages_s": {k: round(v, 4) for k, v in stages.items()},
            "weights_per_s": round(weights / t_total, 1), "ops_per_s": round(ops / t_total, 1),
            "host_cpus": len(os.sched_getaffinity(0)), "host_cpu_model": model}


if __name__ == "__main__":
    main()
