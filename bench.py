#!/usr/bin/env python3
"""Benchmark of the Sparse-BitLinear hot path on one MI355X.

Headline (`value`): decode of a 70B-class transformer block (hidden 8192,
FFN 28672: q, k, v, o 8192x8192, gate, up 28672x8192, down 8192x28672), one
token, 6:8 Sparse-BitLinear weights.  The codes (ternary, masked 6:8) are
stored 2 bits per weight (DENSE2): on MI355X, whose matrix cores have no 6:8
mode, that is both the smaller storage (the N:M codes + bitmap take 2.5 bits
per weight) and the cheaper decode; the same step with the N:M storage is
measured beside it (`headline_nm68`).  A step is the block's decode pass:
for each of its 4 inputs (q/k/v share one, o, gate/up share one, down)
`sbl_linear_acts_batch` quantizes the token (per-token absmax int8) and runs
the ternary x int8 products with the fp32 rescale, one fused GEMV launch per
input.  The weights were prepared before the timed region by
`sbl_quant_weights_batch` (exact absmean beta, 6:8 mask from the BF16
masters, ternary codes, packing), as a decoder prepares them once at load.
`value` is the packed weight bytes (codes, and metadata for N:M) streamed per
second.
Steps rotate over distinct copies of the packed weights (>= 560 MB), so the
256 MB Infinity Cache cannot serve a step from the previous one; one HIP graph
holds a pass over all copies (as a model's decode graph holds all its
layers), so a graph's own launch cost is shared by several steps.

Side measurements in the same line: prefill GEMMs (3B-class block, 2048
tokens, 6:8 / DENSE2 on the dense int8 MFMA, 2:4 on the sparse MFMA; 13B-class
block, 4096 tokens), the 13B training-step path (per-step weight preparation
+ forward GEMMs), the weight-preparation sweep, the whole path on a 0.7B-class
block, the GEMV table over every decode configuration, the backward, the group
scales, library reference rates, the chip's measured streaming-read and int8
MFMA peaks (each roofline is also given as a fraction of the measured peak of
its bound), and the CPU oracle on a bounded sample of the headline workload.

Printed: one JSON line.  `--sections` selects parts (for profiler runs);
`--record-traffic` turns two rocprofv3 counter runs into profiles/traffic.json.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sparse-BitLinear GEMV weight GB/s + prefill int8 TOPS, as % of MI355X peak"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0           # dense int8 matrix cores
INT8_SPARSE_PEAK_TOPS = 10000.0   # 2:4 structured-sparse int8 matrix cores (dense-equivalent ops)
BF16_PEAK_TFLOPS = 2500.0

FORMATS = {"dense2": (0, 6, 8), "nm68": (1, 6, 8), "nm24": (1, 2, 4)}
GROUPS = [[0, 1, 2], [3], [4, 5], [6]]          # q/k/v, o, gate/up, down share an input

BLOCKS = {
    # name: (synth workload, hidden, ffn, description)
    "0p7b": ("b0p7", 1536, 4096, "0.7B-class block (hidden 1536, FFN 4096)"),
    "3b": ("b3", 3200, 8640, "3B-class block (hidden 3200, FFN 8640)"),
    "13b": ("b13", 5120, 13824, "13B-class block (hidden 5120, FFN 13824)"),
    "70b": ("b70", 8192, 28672, "70B-class block (hidden 8192, FFN 28672)"),
}
SECTIONS = ("peaks", "headline", "gemv", "prefill", "act_quant", "train13b", "weight_prep", "step0p7b",
            "backward", "group_scales", "references", "cpu")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--block", default="70b", choices=sorted(BLOCKS), help="headline decode block")
    p.add_argument("--fmt", default="dense2", choices=sorted(FORMATS),
                   help="headline format (the other N:M one is measured beside it)")
    p.add_argument("--m-tok", type=int, default=1)
    p.add_argument("--sections", default=",".join(SECTIONS),
                   help="comma list of parts to run (default: all): " + ",".join(SECTIONS))
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration-mb", type=float, default=0.0,
                   help="before the run, copy a buffer of this many MB 3 times (a known-size copy "
                        "for scaling hardware byte counters)")
    p.add_argument("--record-traffic", metavar="KEY", default=None,
                   help="do not run: read two rocprofv3 counter runs (--fetch-dir, --write-dir) and "
                        "record KEY's bytes per launch in profiles/traffic.json")
    p.add_argument("--trace-summary", metavar="DIR", default=None,
                   help="do not run: summarize a rocprofv3 --kernel-trace --stats output directory "
                        "(per-kernel table; with --kernel/--count/--launches, the timed launches)")
    p.add_argument("--fetch-dir")
    p.add_argument("--write-dir")
    p.add_argument("--kernel", help="kernel-name prefix of the launches to count (--record-traffic)")
    p.add_argument("--launches", type=int, help="launches of that kernel per step (--record-traffic)")
    p.add_argument("--count", type=int,
                   help="count the last COUNT launches of that kernel (--record-traffic; default "
                        "launches x steps: the timed steps, which end the profiled run)")
    p.add_argument("--prefill-cases", default="3b:nm68,3b:dense2,3b:nm24,13b:nm68,13b:dense2",
                   help="prefill cases block:format, in this order")
    p.add_argument("--prep-blocks", default="0p7b,3b,13b", help="blocks of the weight-preparation sweep")
    p.add_argument("--summary", help="text summary to write under profiles/ (--record-traffic)")
    p.add_argument("--command", help="the profiled command, quoted in the summary (--record-traffic)")
    return p.parse_args()


# --------------------------------------------------------------------------- traffic records

TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join("sparse_linear_layers_absmean_amd", "csrc")
# the sources each measured kernel is built from (its file and the headers it
# includes), plus the header and C ABI that configure every launch: a traffic
# record holds while these files are unchanged
_COMMON_SOURCES = ["sbl_internal.h", "sbl_api.hip"]
KERNEL_SOURCES = {
    "gemv_kernel": ["k_linear.hip", "sbl_actq.h", "sbl_decode.h"],
    "quant_acts": ["k_quant_acts.hip", "sbl_actq.h"],
    "gemm_kernel": ["k_gemm.hip", "k_linear.hip", "sbl_decode.h"],
    "gemm24_kernel": ["k_gemm24.hip", "k_gemm.hip", "k_linear.hip", "sbl_decode.h"],
    "absmean_partial_kernel": ["k_beta.hip", "sbl_partial.h", "sbl_beta.h", "sbl_select.h"],
    "absmean_final_kernel": ["k_beta.hip", "sbl_partial.h", "sbl_beta.h", "sbl_select.h"],
    "mask_pack_fast_kernel": ["k_maskpack.hip", "sbl_partial.h", "sbl_beta.h", "sbl_select.h"],
    "resident_kernel": ["k_maskpack.hip", "sbl_partial.h", "sbl_beta.h", "sbl_select.h"],
}


def _sources_sha(kernels):
    """SHA-256 of the sources of the comma-separated kernel name prefixes."""
    files = set(_COMMON_SOURCES)
    for name in kernels.split(","):
        files.update(KERNEL_SOURCES[name])
    out = {}
    for f in sorted(files):
        rel = os.path.join(CSRC, f)
        with open(os.path.join(ROOT, rel), "rb") as fh:
            out[rel] = hashlib.sha256(fh.read()).hexdigest()
    return out


def recorded_traffic(key, field="bytes_per_launch"):
    """HBM bytes per launch (or per step) recorded for `key` in
    profiles/traffic.json, or None when there is no record or a source of its
    kernels has changed since (SHA-256)."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)[key]
        if rec["sources_sha256"] != _sources_sha(rec["kernels"]):
            return None
        return rec[field]
    except (OSError, KeyError, ValueError):
        return None


def _counter_rows(d):
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _short_name(full, args_too=False):
    """Kernel name without return type, namespaces and (unless args_too)
    template arguments: 'void sbl::(anonymous namespace)::gemv_kernel<1, 1, 2, true>(...)'
    -> 'gemv_kernel' (or 'gemv_kernel<1, 1, 2, true>')."""
    nm = full.replace("(anonymous namespace)::", "").replace("void ", "").strip()
    nm = nm.split("(")[0].split("::")[-1]
    return nm if args_too else nm.split("<")[0]


def trace_summary(args):
    """Text summary of a kernel-trace run: every kernel's calls and durations
    (from the --stats table), then, for --kernel prefixes, the last --count
    dispatches (the timed steps) with their mean duration per launch and per
    step of --launches launches."""
    import csv
    d = args.trace_summary
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    out = [f"# Kernel time: {args.record_traffic or os.path.basename(d.rstrip('/'))}", "",
           "Command (MI355X, one GPU):",
           f"    cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- {args.command}", ""]
    if stats:
        with open(stats[0]) as fh:
            rows = list(csv.DictReader(fh))
        out.append(f"{'kernel':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:25]:
            out.append(f"{_short_name(r['Name'], True)[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                       f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    if trace and args.kernel:
        with open(trace[0]) as fh:
            rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
        prefixes = args.kernel.split(",")
        mine = [r for r in rows if any(_short_name(r["Kernel_Name"]).startswith(p) for p in prefixes)]
        use = mine[-args.count:]
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in use]
        span = (int(use[-1]["End_Timestamp"]) - int(use[0]["Start_Timestamp"])) / 1e3
        steps = len(use) // args.launches
        out += ["", f"Timed launches: the last {len(use)} dispatches of {args.kernel} "
                    f"({args.launches} per step, {steps} steps).",
                f"  mean kernel duration per launch: {sum(durs) / len(durs):.2f} us "
                f"(kernel time per step {sum(durs) / steps:.2f} us)",
                f"  first start to last end: {span:.1f} us = {span / steps:.2f} us per step "
                f"(kernel time plus the gaps between dependent launches)"]
        per_pos = {}
        for i, (r, t) in enumerate(zip(use, durs)):
            per_pos.setdefault(i % args.launches, []).append((_short_name(r["Kernel_Name"], True), t,
                                                               r.get("Grid_Size_X") or r.get("Grid_Size")))
        for pos, v in sorted(per_pos.items()):
            out.append(f"  launch {pos}: {v[0][0][:60]} grid {v[0][2]}: mean {sum(t for _, t, _ in v) / len(v):.2f} us")
    text = "\n".join(out) + "\n"
    if args.summary:
        with open(os.path.join(ROOT, args.summary), "w") as fh:
            fh.write(text)
    print(text)


def record_traffic(args):
    """Bytes per launch of the counted kernels from a FETCH_SIZE run and a
    WRITE_SIZE run of the same command, each scaled by what the counter reads
    for the known copy of --copy-calibration-mb (the first dispatch of the
    blit kernel that copies it).  --kernel is a comma list of kernel-name
    prefixes; the counted dispatches are the last --count of those kernels
    (default launches x steps: the timed steps, which end the run), and
    --launches of them make one step."""
    prefixes = args.kernel.split(",")
    res = {}
    for name, d in (("FETCH_SIZE", args.fetch_dir), ("WRITE_SIZE", args.write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        per_dispatch = {}
        for r in rows:
            per_dispatch.setdefault(r["Dispatch_Id"], [r, 0.0])[1] += float(r["Counter_Value"])
        ordered = sorted(per_dispatch.values(), key=lambda rv: int(rv[0]["Dispatch_Id"]))
        copies = [v for r, v in ordered if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit("calibration copy not found (run with --copy-calibration-mb)")
        cal_bytes = float(args.copy_calibration_mb) * 1e6 // 16 * 16
        factor = cal_bytes / (copies[0] * 1024.0)     # a copy reads and writes its size once
        base = [(_short_name(r["Kernel_Name"]), r, v) for r, v in ordered]
        mine = [(r, v) for nm, r, v in base if any(nm.startswith(p) for p in prefixes)]
        count = args.count or args.launches * args.steps
        if len(mine) < count:
            raise SystemExit(f"only {len(mine)} launches of {args.kernel} in {d}")
        use = mine[-count:]
        kib = sum(v for _, v in use)
        res[name] = dict(factor=factor, bytes_per_launch=kib * 1024.0 * factor / count,
                         copy_kib=copies[0], launches=count,
                         kernels=sorted({_short_name(r["Kernel_Name"], True) for r, _ in use}))
    per_launch = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    try:
        with open(TRAFFIC_JSON) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {}
    allrec[args.record_traffic] = {
        "kernels": args.kernel, "launches_per_step": args.launches,
        "bytes_per_launch": round(per_launch), "bytes_per_step": round(per_launch * args.launches),
        "read_bytes_per_launch": round(res["FETCH_SIZE"]["bytes_per_launch"]),
        "write_bytes_per_launch": round(res["WRITE_SIZE"]["bytes_per_launch"]),
        "fetch_factor": round(res["FETCH_SIZE"]["factor"], 4), "write_factor": round(res["WRITE_SIZE"]["factor"], 4),
        "summary": args.summary, "sources_sha256": _sources_sha(args.kernel)}
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
    if args.summary:
        f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
        with open(os.path.join(ROOT, args.summary), "w") as fh:
            fh.write(f"# HBM traffic: {args.record_traffic}\n\n")
            fh.write("Commands (two counter passes of the same run, MI355X):\n")
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                fh.write(f"    cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- {args.command}\n")
            fh.write(f"\nCalibration: the {args.copy_calibration_mb:g} MB device copy (copyBuffer blit kernel) reads "
                     f"{f['copy_kib']:.1f} KiB\nby FETCH_SIZE and writes {w['copy_kib']:.1f} KiB by WRITE_SIZE, so "
                     f"bytes = FETCH_SIZE*1024*{f['factor']:.4f} and WRITE_SIZE*1024*{w['factor']:.4f}.\n\n")
            fh.write(f"Counted: the last {f['launches']} launches of {', '.join(f['kernels'])} "
                     f"({args.launches} per step: the timed steps).\n")
            fh.write(f"Per launch (average): read {f['bytes_per_launch'] / 1e6:.3f} MB, "
                     f"written {w['bytes_per_launch'] / 1e6:.3f} MB, total {per_launch / 1e6:.3f} MB; "
                     f"per step {per_launch * args.launches / 1e6:.3f} MB.\n")
    print(json.dumps(allrec[args.record_traffic]))


# --------------------------------------------------------------------------- timing helpers

class Timer:
    """HIP events on torch's current stream (every libsbl call here is issued there,
    graph replays included)."""

    def __init__(self, torch):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def timed_steps(torch, tm, fn, copies, steps, warm=None):
    """ms per call of fn(c), timing exactly `steps` calls that rotate over the
    copies c = 0, 1, ...: one HIP graph holds a pass over all copies (so the
    per-replay launch cost of a graph is shared by `copies` steps, as in a
    model whose decode graph holds every layer), a second one the remainder."""
    fn(0)
    torch.cuda.synchronize()

    def graph(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(n):
                fn(c)
        return g

    full = graph(copies)
    rem = graph(steps % copies) if steps % copies else None
    for _ in range(max(1, -(-(copies if warm is None else warm) // copies))):
        full.replay()
    torch.cuda.synchronize()
    tm.start()
    for _ in range(steps // copies):
        full.replay()
    if rem is not None:
        rem.replay()
    ms = tm.stop_ms() / steps
    del full, rem
    return ms


def rot_copies(per_copy_bytes, floor=560e6, cap=64):
    return int(min(cap, max(2, -(-floor // per_copy_bytes))))


def mats_of(block):
    import synth
    _, h, f, _ = BLOCKS[block]
    return synth.block_shapes(h, f)


def synth_masters(block, mats):
    """The block's BF16 masters from the seeded CPU generators, one thread per matrix."""
    from concurrent.futures import ThreadPoolExecutor

    import synth
    wname = BLOCKS[block][0] if block != "3b" else "b3_prefill"
    with ThreadPoolExecutor(len(mats)) as ex:
        return list(ex.map(lambda i: synth.workload_masters(wname, i, mats[i][1], mats[i][2]), range(len(mats))))


def device_masters(torch, dev, gen, no, k):
    """N(0, 0.02) masters rounded to BF16, drawn on the device (same distribution as
    the CPU generators; used where drawing ~1e9 values on the host would take minutes)."""
    return (torch.randn((no, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)


def prepare_packed(torch, sbl, dev, masters, mats, n, m, fmt):
    """sbl_quant_weights_batch over the block (7 matrices, one call); returns per-matrix
    dicts with beta, packed and meta."""
    outs, items = [], []
    for (_, no, k), w in zip(mats, masters):
        o = dict(beta=torch.empty(1, dtype=torch.float32, device=dev),
                 packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device=dev),
                 meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev) if fmt == 1 else None, n_out=no)
        outs.append(o)
        items.append(dict(w=w, beta=o["beta"], packed=o["packed"], meta=o["meta"],
                          workspace=sbl.new_workspace(no, k, dev)))
    sbl.sbl_quant_weights_batch(items, n, m, fmt)
    torch.cuda.synchronize()
    return outs


def packed_bytes(sbl, no, k, n, m, fmt):
    return sbl.sbl_packed_bytes(no, k, n, m, fmt) + max(0, sbl.sbl_meta_bytes(no, k, fmt))


def clone_packed(outs):
    return [dict(o, packed=o["packed"].clone(), meta=o["meta"].clone() if o["meta"] is not None else None)
            for o in outs]


# --------------------------------------------------------------------------- headline: decode step

def bench_decode_step(torch, np, sbl, dev, tm, args):
    """The decode pass of one block (4 fused activation-quant + GEMV launches) over
    packed weights prepared by sbl_quant_weights_batch; graph replays over rotating
    copies of the packed weights."""
    import synth
    fmt, n, m = FORMATS[args.fmt]
    mats = mats_of(args.block)
    m_tok = args.m_tok
    gen = torch.Generator(device=dev).manual_seed(1)
    if args.block == "70b":
        masters = [device_masters(torch, dev, gen, no, k) for _, no, k in mats]
        master_src = "N(0,0.02) BF16 masters drawn on the device (torch, seed 1)"
    else:
        masters = [torch.from_numpy(b.view(np.int16)).to(dev) for b in synth_masters(args.block, mats)]
        master_src = f"seeded synthetic masters ({BLOCKS[args.block][0]} recipe)"
    outs = prepare_packed(torch, sbl, dev, masters, mats, n, m, fmt)
    del masters
    torch.cuda.empty_cache()
    wbytes = sum(packed_bytes(sbl, no, k, n, m, fmt) for _, no, k in mats)
    copies = rot_copies(wbytes)
    pool = [outs] + [clone_packed(outs) for _ in range(copies - 1)]
    wname = BLOCKS[args.block][0]
    xs = [torch.from_numpy(synth.workload_acts(wname, grp[0], m_tok, mats[grp[0]][2])).to(dev) for grp in GROUPS]
    acts = [dict(xq=torch.empty((m_tok, x.shape[1]), dtype=torch.int8, device=dev),
                 gamma=torch.empty(m_tok, dtype=torch.float32, device=dev)) for x in xs]
    ys = [torch.empty((m_tok, no), dtype=torch.float32, device=dev) for _, no, _k in mats]

    def step(c):
        for gi, grp in enumerate(GROUPS):
            sbl.sbl_linear_acts_batch(xs[gi], acts[gi]["xq"], acts[gi]["gamma"],
                                      [dict(pool[c][i], y=ys[i]) for i in grp], fmt, n, m)

    step_ms = timed_steps(torch, tm, step, copies, args.steps, warm=args.warmup)
    # kernel launches per step: one fused GEMV per input, plus a standalone
    # quantizer for inputs above 16384 values (the call's documented rule)
    launches = len(GROUPS) + sum(1 for g in GROUPS if m_tok * mats[g[0]][2] > 16384)
    alg = wbytes + sum(m_tok * mats[g[0]][2] * 5 + 4 * m_tok for g in GROUPS) + \
        sum(4 * m_tok * no for _, no, _k in mats)
    gbps = wbytes / (step_ms * 1e-3) / 1e9
    achieved = alg / (step_ms * 1e-3) / 1e9
    key = f"gemv_decode_{args.block}_{args.fmt}_m{m_tok}"
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": recorded_traffic(key),
            "kernel": "gemv_kernel with the activation quantization fused in (sbl_linear_acts_batch; "
                      "quant_acts_kernel first for inputs above 16384 values)",
            "call": "sbl_linear_acts_batch", "launches_per_step": launches,
            "traffic_per_step": recorded_traffic(key, "bytes_per_step"),
            "alg_bytes_per_launch": round(alg / launches), "avg_launch_us": round(step_ms * 1e3 / launches, 3),
            "note": "algorithmic bytes (packed weights + metadata, fp32 input read, int8 input and gamma "
                    "written, fp32 outputs) per launch / average launch time (HIP events around the timed "
                    "graph replays, gaps included); traffic: counter bytes per launch (profiles/traffic.json)"}
    del pool
    torch.cuda.empty_cache()
    return dict(step_ms=step_ms, gbps=gbps, wbytes=wbytes, copies=copies, roofline=roof,
                master_src=master_src, weights=sum(no * k for _, no, k in mats))


# --------------------------------------------------------------------------- GEMV table

def gemv_sweep(torch, np, sbl, dev, tm):
    """Packed-weight GB/s of the GEMV for the decode configurations: grouped (sbl_linear_batch:
    4 launches per block, matrices sharing an input in one launch) and, for the 3B and 70B
    blocks at one token, one launch per matrix (7 per block).  The packed bytes are seeded random valid codes (the GEMV's
    time does not depend on their values); blocks rotate over >= 600 MB of distinct
    buffers; each block's 4 launches are one HIP graph."""
    # (block, tokens, one launch per matrix instead of the grouped launches)
    cases = [("0p7b", 1, False), ("3b", 1, False), ("3b", 4, False), ("3b", 8, False), ("70b", 1, False),
             ("70b", 8, False), ("70b", 16, False), ("3b", 1, True), ("70b", 1, True)]
    out = []
    for blk, m_tok, single in cases:
        mats = mats_of(blk)
        for fname, (fmt, n, m) in FORMATS.items():
            if single and fname == "nm24":
                continue
            nbytes = [sbl.sbl_packed_bytes(no, k, n, m, fmt) for _, no, k in mats]
            mbytes = [no * k // 8 if fmt == 1 else 0 for _, no, k in mats]
            bb = sum(nbytes) + sum(mbytes)
            copies = rot_copies(bb, 600e6)
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
                                generator=gen) for grp in GROUPS]
            gam = torch.ones(m_tok, device=dev)

            def run(c):
                for gi, grp in enumerate(GROUPS):
                    if single:
                        for i in grp:
                            sbl.sbl_linear_batch([dict(pool[c][i], xq=xs[gi], gamma=gam)], fmt, n, m)
                    else:
                        sbl.sbl_linear_batch([dict(pool[c][i], xq=xs[gi], gamma=gam) for i in grp], fmt, n, m)

            us = timed_steps(torch, tm, run, copies, 8 * copies) * 1e3
            gbps = bb / (us * 1e-6) / 1e9
            hbm = bb + sum(m_tok * mats[g_[0]][2] + 4 * m_tok for g_ in GROUPS) + \
                sum(4 * m_tok * no for _, no, _k in mats)
            out.append({"block": blk, "format": fname, "m_tok": m_tok,
                        "launches": f"{len(mats)}, one per matrix" if single else f"{len(GROUPS)}, grouped",
                        "weight_bytes": bb,
                        "us_per_block": round(us, 2), "weight_GBps": round(gbps, 1),
                        "hbm_GBps": round(hbm / (us * 1e-6) / 1e9, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
            del pool, xs
            torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- activation quantization

def bench_act_quant(torch, sbl, dev, tm):
    """sbl_quant_acts alone (per-token absmax int8 quantization) at the decode and prefill
    input shapes of the blocks: algorithmic bytes = fp32 read + int8 written (5 B per
    value) + gamma (4 B per token); N(0,1) inputs drawn on the device; graph replays
    rotating over >= 560 MB of distinct inputs."""
    cases = [(1, 8192), (1, 28672), (8, 28672), (16, 28672),
             (2048, 3200), (2048, 8640), (4096, 5120), (4096, 13824)]
    out = []
    g = torch.Generator(device=dev).manual_seed(13)
    for m_tok, k in cases:
        copies = rot_copies(m_tok * k * 5, cap=256)
        pool = [(torch.randn((m_tok, k), generator=g, device=dev),
                 torch.empty((m_tok, k), dtype=torch.int8, device=dev),
                 torch.empty(m_tok, device=dev)) for _ in range(copies)]
        us = timed_steps(torch, tm, lambda c: sbl.sbl_quant_acts(*pool[c]), copies, max(20, 2 * copies)) * 1e3
        alg = m_tok * k * 5 + 4 * m_tok
        gbps = alg / (us * 1e-6) / 1e9
        out.append({"m_tok": m_tok, "k": k, "us_per_call": round(us, 2), "alg_bytes": alg,
                    "alg_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        del pool
        torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- prefill GEMMs

def bench_prefill(torch, np, sbl, dev, tm, masters_by_block, cases):
    """Prefill products of whole blocks (4 grouped launches of sbl_linear_batch on
    int8 activations from sbl_quant_acts), graph replays rotating over 2 copies of the
    packed weights: 3B-class block at 2048 tokens (6:8 N:M and 6:8-masked DENSE2 on the
    dense int8 MFMA, 2:4 N:M on the 2:4 sparse MFMA) and 13B-class block at 4096 tokens
    (6:8 N:M, DENSE2).  TOPS count the dense-equivalent 2*M*N*K int8 operations; the
    sparse-MFMA path is priced against the sparse peak."""
    import synth
    tokens = {"3b": 2048, "13b": 4096}
    cases = [(c.split(":")[0], tokens[c.split(":")[0]], c.split(":")[1]) for c in cases.split(",")]
    out = []
    for blk, m_tok, fname in cases:
        fmt, n, m = FORMATS[fname]
        mats = mats_of(blk)
        masters = [torch.from_numpy(b.view(np.int16)).to(dev) for b in masters_by_block[blk]]
        outs = prepare_packed(torch, sbl, dev, masters, mats, n, m, fmt)
        del masters
        pool = [outs, clone_packed(outs)]
        wname = "b3_prefill" if blk == "3b" else BLOCKS[blk][0]
        acts = []
        for grp in GROUPS:
            x = torch.from_numpy(synth.workload_acts(wname, grp[0], m_tok, mats[grp[0]][2])).to(dev)
            acts.append(sbl.quant_acts(x))
            del x
        ys = [torch.empty((m_tok, no), dtype=torch.float32, device=dev) for _, no, _k in mats]

        def run(c):
            for gi, grp in enumerate(GROUPS):
                sbl.sbl_linear_batch([dict(pool[c][i], xq=acts[gi][0], gamma=acts[gi][1], y=ys[i]) for i in grp],
                                     fmt, n, m)

        ms = timed_steps(torch, tm, run, 2, 10)
        ops = sum(2 * m_tok * no * k for _, no, k in mats)
        tops = ops / (ms * 1e-3) / 1e12
        sparse = fname == "nm24"
        peak = INT8_SPARSE_PEAK_TOPS if sparse else INT8_PEAK_TOPS
        key = f"gemm_prefill_{blk}_{fname}_m{m_tok}"
        kernel = ("gemm24_kernel (v_smfmac_i32_16x16x128_i8, 2:4 sparse)" if sparse
                  else "gemm_kernel (v_mfma_i32_32x32x32_i8)")
        out.append({"block": blk, "format": fname, "m_tok": m_tok, "kernel": kernel,
                    "workload": f"Prefill GEMM, M={m_tok} tokens, {BLOCKS[blk][3]}, {fname}",
                    "ms_per_block": round(ms, 4), "int8_TOPS": round(tops, 1),
                    "useful_TOPS": round(tops * n / m, 1),
                    "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": peak, "unit": "TOP/s",
                                 "frac": round(tops / peak, 4), "traffic": recorded_traffic(key),
                                 "peak_kind": "int8 2:4 sparse MFMA (dense-equivalent ops)" if sparse
                                 else "int8 dense MFMA",
                                 "avg_launch_us": round(ms * 1e3 / len(GROUPS), 2)},
                    "weights": "graph replays over 2 copies of the packed weights (both fit in the 256 MB Infinity Cache)"})
        del pool, outs, acts, ys
        torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- 13B training-step path

def bench_train13b(torch, np, sbl, dev, tm, masters13, fname="nm68"):
    """The training-step path of a 13B-class block: per-step weight preparation from the
    BF16 masters (exact beta, 6:8 mask with planted near-ties, codes, packing in the
    storage `fname`: N:M codes + bitmap, or DENSE2), the forward products at 4096 tokens
    (activation quantization + GEMM per input) and the layer's backward (dX and dW of
    every matrix from a synthetic BF16 dY).  Graph replays over 2 copies of masters and
    activations."""
    import synth
    fmt, n, m = FORMATS[fname]
    mats = mats_of("13b")
    m_tok = 4096
    copies = 2
    m0 = [torch.from_numpy(b.view(np.int16)).to(dev) for b in masters13]
    x0 = [torch.from_numpy(synth.workload_acts("b13", grp[0], m_tok, mats[grp[0]][2])).to(dev) for grp in GROUPS]
    state = []
    for c in range(copies):
        ms_ = m0 if c == 0 else [t.clone() for t in m0]
        xs = x0 if c == 0 else [t.clone() for t in x0]
        outs = [dict(beta=torch.empty(1, device=dev),
                     packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device=dev),
                     meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev), n_out=no,
                     y=torch.empty((m_tok, no), device=dev)) for _, no, k in mats]
        wss = [sbl.new_workspace(no, k, dev) for _, no, k in mats]
        acts = [dict(xq=torch.empty((m_tok, x.shape[1]), dtype=torch.int8, device=dev),
                     gamma=torch.empty(m_tok, device=dev)) for x in xs]
        state.append((ms_, xs, outs, wss, acts))
    # backward buffers, shared by the copies: dY per matrix, dX per input, dW per matrix
    g = torch.Generator(device=dev).manual_seed(12)
    dys = [(torch.randn((m_tok, no), generator=g, device=dev) * 0.05).to(torch.bfloat16) for _, no, k in mats]
    dxs = [torch.empty((m_tok, k), device=dev) for _, no, k in mats]
    dws = [torch.empty((no, k), device=dev) for _, no, k in mats]
    bws = sbl.new_backward_workspace(m_tok, max(no for _, no, _k in mats), max(k for _, _n, k in mats), dev)
    group_of = {i: gi for gi, grp in enumerate(GROUPS) for i in grp}

    def bwd(c):
        ms_, xs, outs, wss, acts = state[c]
        for i in range(len(mats)):
            gi = group_of[i]
            sbl.sbl_linear_backward(dys[i], outs[i]["packed"], outs[i]["meta"], fmt, n, m, outs[i]["beta"], xs[gi],
                                    acts[gi]["xq"], acts[gi]["gamma"], dx=dxs[i], dw=dws[i], workspace=bws)

    def prep(c):
        ms_, xs, outs, wss, acts = state[c]
        sbl.sbl_quant_weights_batch([dict(w=ms_[i], beta=outs[i]["beta"], packed=outs[i]["packed"],
                                          meta=outs[i]["meta"], workspace=wss[i]) for i in range(len(mats))],
                                    n, m, fmt)

    def fwd(c):
        ms_, xs, outs, wss, acts = state[c]
        for gi, grp in enumerate(GROUPS):
            sbl.sbl_linear_acts_batch(xs[gi], acts[gi]["xq"], acts[gi]["gamma"], [outs[i] for i in grp],
                                      fmt, n, m)

    step_ms = timed_steps(torch, tm, lambda c: (prep(c), fwd(c)), copies, 10)
    prep_us = timed_steps(torch, tm, prep, copies, 20) * 1e3
    fwd_ms = timed_steps(torch, tm, fwd, copies, 10)
    full_ms = timed_steps(torch, tm, lambda c: (prep(c), fwd(c), bwd(c)), copies, 4)
    bwd_ms = timed_steps(torch, tm, bwd, copies, 4)
    weights = sum(no * k for _, no, k in mats)
    prep_alg = sum(2 * no * k + packed_bytes(sbl, no, k, n, m, fmt) for _, no, k in mats)
    ops = 2 * m_tok * weights
    del state, dys, dxs, dws, bws
    torch.cuda.empty_cache()
    storage = "N:M codes + bitmap" if fname == "nm68" else "DENSE2 (2 bits per weight)"
    return {"workload": f"Training-step path, {BLOCKS['13b'][3]}, 6:8 stored {storage}, M=4096 tokens, "
                        "masters with near-ties planted on the keep boundary",
            "ms_per_step": round(step_ms, 4),
            "with_backward_ms_per_step": round(full_ms, 4), "backward_ms": round(bwd_ms, 4),
            "backward_TFLOPS": round(2 * ops / (bwd_ms * 1e-3) / 1e12, 1),
            "backward_frac": round(2 * ops / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "weight_prep_us": round(prep_us, 1),
            "weight_prep_GBps": round(prep_alg / (prep_us * 1e-6) / 1e9, 1),
            "weight_prep_frac": round(prep_alg / (prep_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "forward_ms": round(fwd_ms, 4), "forward_int8_TOPS": round(ops / (fwd_ms * 1e-3) / 1e12, 1),
            "forward_frac": round(ops / (fwd_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "calls": "sbl_quant_weights_batch (7 matrices), then per input sbl_linear_acts_batch "
                     "(quant_acts_kernel + gemm_kernel); with_backward adds per matrix "
                     "sbl_linear_backward_ws (dX and dW, one shared workspace)"}


# --------------------------------------------------------------------------- weight preparation sweep

def weight_prep_sweep(torch, np, sbl, dev, tm, blocks):
    """sbl_quant_weights_batch over whole blocks (7 matrices, 6:8 N:M output), the
    per-step weight preparation: algorithmic bytes (masters read once + packed codes and
    metadata written) per second.  N(0, 0.02) BF16 masters drawn on the device; each
    block rotates over >= 2 distinct copies totalling >= 600 MB; HIP graphs."""
    n, m, fmt = 6, 8, 1
    out = []
    for blk in blocks.split(","):
        mats = mats_of(blk)
        bw = sum(no * k for _, no, k in mats)
        copies = rot_copies(2 * bw, 600e6)
        g = torch.Generator(device=dev).manual_seed(5)
        pool = []
        for c in range(copies):
            pool.append([dict(w=device_masters(torch, dev, g, no, k), beta=torch.empty(1, device=dev),
                              packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8,
                                                 device=dev),
                              meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev),
                              workspace=sbl.new_workspace(no, k, dev)) for _, no, k in mats])
        us = timed_steps(torch, tm, lambda c: sbl.sbl_quant_weights_batch(pool[c], n, m, fmt), copies,
                         max(20, 2 * copies)) * 1e3
        alg = sum(2 * no * k + packed_bytes(sbl, no, k, n, m, fmt) for _, no, k in mats)
        gbps = alg / (us * 1e-6) / 1e9
        counted = recorded_traffic(f"weight_prep_{blk}_nm68", "bytes_per_step")
        out.append({"block": blk, "weights": bw, "us_per_call": round(us, 2), "alg_GBps": round(gbps, 1),
                    "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic_bytes_per_call": counted,
                    "counted_GBps": round(counted / (us * 1e-6) / 1e9, 1) if counted else None,
                    "path": "one launch (resident_kernel)" if bw * 2 <= 67e6 else "two launches (absmean + mask_pack)"})
        del pool
        torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- whole path, 0.7B block

def bench_step0p7b(torch, np, sbl, dev, tm):
    """The whole path on a 0.7B-class block, one token, 6:8 N:M: per step the weight
    preparation of the 7 matrices (one launch) and the 4 fused activation-quant + GEMV
    launches; graph replays rotating over >= 560 MB of master copies.  Rate: all of the
    step's algorithmic bytes (masters read, packed written and read, activations,
    outputs) per second."""
    import synth
    fmt, n, m = FORMATS["nm68"]
    mats = mats_of("0p7b")
    m_tok = 1
    bw = sum(no * k for _, no, k in mats)
    copies = rot_copies(2 * bw)
    base = synth_masters("0p7b", mats)
    st = []
    for c in range(copies):
        masters = [torch.from_numpy(b.view(np.int16)).to(dev) for b in base]
        xs = [torch.from_numpy(synth.workload_acts("b0p7", grp[0], m_tok, mats[grp[0]][2], copy=c)).to(dev)
              for grp in GROUPS]
        outs = [dict(beta=torch.empty(1, device=dev),
                     packed=torch.empty(sbl.sbl_packed_bytes(no, k, n, m, fmt), dtype=torch.uint8, device=dev),
                     meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev), n_out=no,
                     y=torch.empty((m_tok, no), device=dev)) for _, no, k in mats]
        wss = [sbl.new_workspace(no, k, dev) for _, no, k in mats]
        acts = [dict(xq=torch.empty((m_tok, x.shape[1]), dtype=torch.int8, device=dev),
                     gamma=torch.empty(m_tok, device=dev)) for x in xs]
        st.append((masters, xs, outs, wss, acts))

    def step(c):
        masters, xs, outs, wss, acts = st[c]
        sbl.sbl_quant_weights_batch([dict(w=masters[i], beta=outs[i]["beta"], packed=outs[i]["packed"],
                                          meta=outs[i]["meta"], workspace=wss[i]) for i in range(len(mats))],
                                    n, m, fmt)
        for gi, grp in enumerate(GROUPS):
            sbl.sbl_linear_acts_batch(xs[gi], acts[gi]["xq"], acts[gi]["gamma"], [outs[i] for i in grp], fmt, n, m)

    ms = timed_steps(torch, tm, step, copies, 10 * copies)
    pb = sum(packed_bytes(sbl, no, k, n, m, fmt) for _, no, k in mats)
    alg = 2 * bw + 2 * pb + sum(m_tok * mats[g[0]][2] * 5 + 4 * m_tok for g in GROUPS) + \
        sum(4 * m_tok * no for _, no, _k in mats)
    del st
    torch.cuda.empty_cache()
    return {"workload": "Whole path, M=1 token, 0.7B-class block (hidden 1536, FFN 4096), 6:8 N:M: "
                        "weight preparation + fused activation quantization and GEMV",
            "us_per_step": round(ms * 1e3, 2), "alg_bytes": alg,
            "alg_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


# --------------------------------------------------------------------------- backward

def bench_backward(torch, np, sbl, dev, tm, masters3b):
    """Backward of a 3B-class block at 2048 tokens, 6:8 weights: sbl_linear_backward (dX
    and dW of the 7 matrices) on the BF16 matrix cores, with a caller workspace and without.  Algorithmic flops 2*M*N*K per
    gradient; dW runs three BF16 products per step (x_hat split exactly into three parts)."""
    import synth
    fmt, n, m = FORMATS["nm68"]
    m_tok = 2048
    mats = mats_of("3b")
    g = torch.Generator(device=dev).manual_seed(11)
    items = []
    for i, (_, no, k) in enumerate(mats):
        w = torch.from_numpy(masters3b[i].view(np.int16)).to(dev)
        o = sbl.quant_weights(w, n, m, fmt=fmt)
        x = torch.from_numpy(synth.workload_acts("b3_prefill", i, m_tok, k)).to(dev)
        xq, gamma = sbl.quant_acts(x)
        dy = (torch.randn((m_tok, no), generator=g, device=dev) * 0.05).to(torch.bfloat16)
        items.append((o, x, xq, gamma, dy, torch.empty((m_tok, k), device=dev), torch.empty((no, k), device=dev)))
        del w

    # one workspace serves the 7 calls in turn (one stream)
    ws = sbl.new_backward_workspace(m_tok, max(no for _, no, _k in mats), max(k for _, _n, k in mats), dev)

    def run(which, use_ws):
        for o, x, xq, gamma, dy, dx, dw in items:
            sbl.sbl_linear_backward(dy, o["packed"], o["meta"], fmt, n, m, o["beta"], x, xq, gamma,
                                    dx=dx if which in ("dx", "both") else None,
                                    dw=dw if which in ("dw", "both") else None,
                                    workspace=ws if use_ws else None)

    flops = sum(2 * m_tok * no * k for _, no, k in mats)
    out = {}
    for use_ws in (True, False):
        res = {}
        for which in ("dx", "dw", "both"):
            for _ in range(2):
                run(which, use_ws)
            torch.cuda.synchronize()
            tm.start()
            for _ in range(5):
                run(which, use_ws)
            res[which] = tm.stop_ms() / 5
        tf = {w: (flops * (2 if w == "both" else 1)) / (res[w] * 1e-3) / 1e12 for w in res}
        out["workspace" if use_ws else "no_workspace"] = {
            "ms_per_block": {w: round(v, 3) for w, v in res.items()},
            "algorithmic_TFLOPS": {w: round(v, 1) for w, v in tf.items()},
            "dw_mfma_TFLOPS": round(3 * flops / (res["dw"] * 1e-3) / 1e12, 1)}
    del items, ws
    torch.cuda.empty_cache()
    main = out["workspace"]
    tf_both = main["algorithmic_TFLOPS"]["both"]
    return {"workload": "Backward (dX and dW), M=2048 tokens, 3B-class block (hidden 3200, FFN 8640), 6:8 N:M",
            "call": "sbl_linear_backward_ws (one caller workspace; sbl_linear_backward without one: no_workspace)",
            "kernel": "bwd_codes_t/bwd_dy_t/bwd_xhat_t_kernel + bwd_gemm_kernel (v_mfma_f32_32x32x16_bf16); "
                      "without a workspace backward_dx_kernel, backward_dw_kernel",
            **main, "no_workspace": out["no_workspace"],
            "roofline": {"bound": "mfma", "achieved": tf_both, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf_both / BF16_PEAK_TFLOPS, 4), "traffic": None}}


# --------------------------------------------------------------------------- group scales

def bench_group_scales(torch, np, sbl, dev, tm, rpg=128, kg=320, n=6, m=8):
    """Group scales on a 3B-class block, 6:8 N:M, M = 1: weight preparation with beta per
    block of rows (rows_per_group 1 and rpg) and per block of rpg rows x kg features, and
    the decode products with beta per row group, with gamma per block of kg features and
    with both per block, beside the per-matrix sbl_linear.  Each
    block's calls are one HIP graph; every block uses distinct buffers (>= 600 MB)."""
    fmt = 1
    mats = mats_of("3b")
    bw = sum(no * k for _, no, k in mats)
    g = torch.Generator(device=dev).manual_seed(7)
    pb = [sbl.sbl_packed_bytes(no, k, n, m, fmt) for _, no, k in mats]
    wbytes = sum(pb) + sum(no * k // 8 for _, no, k in mats)
    out = {"workload": f"3B-class block (hidden 3200, FFN 8640), {n}:{m} N:M, M=1", "weight_prep": [],
           "products": []}
    copies = rot_copies(2 * bw, 600e6)
    masters = [[device_masters(torch, dev, g, no, k) for _, no, k in mats] for _ in range(copies)]
    outs = [[dict(packed=torch.empty(pb[i], dtype=torch.uint8, device=dev),
                  meta=torch.empty((no, k // 8), dtype=torch.uint8, device=dev)) for i, (_, no, k) in enumerate(mats)]
            for _ in range(copies)]
    # block scales: beta per rpg rows x kg features
    bbetas = [torch.empty((-(-no // rpg), k // kg), device=dev) for _, no, k in mats]
    bwss = [torch.empty(sbl.sbl_workspace_bytes_blocked(no, k, rpg, kg), dtype=torch.uint8, device=dev)
            for _, no, k in mats]

    def prep_blocked(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_quant_weights_blocked(masters[c][i], n, m, rpg, kg, bbetas[i], bwss[i], fmt=fmt,
                                          packed=outs[c][i]["packed"], meta=outs[c][i]["meta"])
    us = timed_steps(torch, tm, prep_blocked, copies, max(10, 2 * copies)) * 1e3
    bouts = [{k2: v.clone() for k2, v in o.items()} for o in outs[0]]     # codes with the block betas
    gbps = (2 * bw + wbytes) / (us * 1e-6) / 1e9
    out["weight_prep"].append({"rows_per_group": rpg, "cols_per_group": kg,
                               "groups": sum(-(-no // rpg) * (k // kg) for _, no, k in mats),
                               "us_per_block": round(us, 1), "alg_GBps": round(gbps, 1),
                               "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    for r in (1, rpg):
        betas = [torch.empty(-(-no // r), device=dev) for _, no, k in mats]
        wss = [torch.empty(sbl.sbl_workspace_bytes_grouped(no, k, r), dtype=torch.uint8, device=dev)
               for _, no, k in mats]

        def prep(c):
            for i, (_, no, k) in enumerate(mats):
                sbl.sbl_quant_weights_grouped(masters[c][i], n, m, r, betas[i], wss[i], fmt=fmt,
                                              packed=outs[c][i]["packed"], meta=outs[c][i]["meta"])
        us = timed_steps(torch, tm, prep, copies, max(10, 2 * copies)) * 1e3
        gbps = (2 * bw + wbytes) / (us * 1e-6) / 1e9
        out["weight_prep"].append({"rows_per_group": r, "groups": sum(-(-no // r) for _, no, k in mats),
                                   "us_per_block": round(us, 1), "alg_GBps": round(gbps, 1),
                                   "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    del masters
    torch.cuda.empty_cache()
    pcopies = rot_copies(wbytes, 600e6)
    pool = [[{k2: v.clone() for k2, v in o.items()} for o in outs[0]] for _ in range(pcopies)]
    bpool = [[{k2: v.clone() for k2, v in o.items()} for o in bouts] for _ in range(pcopies)]
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

    for i in range(len(mats)):
        sbl.sbl_quant_acts_kgrouped(xs[i], kg, gq[i][0], gq[i][1])

    def kgrouped(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_linear_kgrouped(pool[c][i]["packed"], pool[c][i]["meta"], fmt, n, m, betas[i], rpg,
                                    gq[i][0], gq[i][1], kg, no, ys[i])

    def blocked(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_linear_blocked(bpool[c][i]["packed"], bpool[c][i]["meta"], fmt, n, m, bbetas[i], rpg,
                                   gq[i][0], gq[i][1], kg, no, ys[i])

    def kgrouped_q(c):
        for i, (_, no, k) in enumerate(mats):
            sbl.sbl_quant_acts_kgrouped(xs[i], kg, gq[i][0], gq[i][1])
            sbl.sbl_linear_kgrouped(pool[c][i]["packed"], pool[c][i]["meta"], fmt, n, m, betas[i], rpg,
                                    gq[i][0], gq[i][1], kg, no, ys[i])

    # every product row times the products alone on activations quantized beforehand
    for name, fn, what in (("sbl_linear", plain, "per-matrix beta and gamma (one launch per matrix)"),
                           ("sbl_linear_grouped", grouped, f"beta per {rpg} rows, read by the GEMV epilogue"),
                           ("sbl_linear_kgrouped", kgrouped, f"beta per {rpg} rows, gamma per {kg} features"),
                           ("sbl_linear_blocked", blocked, f"beta per {rpg} rows x {kg} features, gamma per {kg} features"),
                           ("sbl_quant_acts_kgrouped + sbl_linear_kgrouped", kgrouped_q,
                            f"the same with the activation quantization per matrix in the step")):
        us = timed_steps(torch, tm, fn, pcopies, max(20, 2 * pcopies)) * 1e3
        gbps = wbytes / (us * 1e-6) / 1e9
        out["products"].append({"call": name, "scales": what, "us_per_block": round(us, 1),
                                "weight_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    del pool, bpool, outs, bouts
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- library references

def measured_peaks(torch, dev, tm):
    """What plain kernels reach on this GPU (libsbl_probe.so, outside the path), HIP
    events around 10 runs each: a streaming read of 1 GB (nontemporal 16-byte loads,
    8 in flight per thread; best of 2048-16384 workgroups of 256 threads) and
    back-to-back independent int8 32x32x32 MFMAs (2048 workgroups of 4 waves)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_linear_layers_absmean_amd", "libsbl_probe.so"))
    lib.sbl_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.sbl_probe_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(10):
            fn()
        return tm.stop_ms() / 10

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed (HIP error {rc})")

    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best, best_grid = 0.0, 0
    for grid in (2048, 4096, 8192, 16384):
        ms = timed(lambda: check(lib.sbl_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, st)))
        gbps = nbytes / (ms * 1e-3) / 1e9
        if gbps > best:
            best, best_grid = gbps, grid
    del buf
    grid, iters = 2048, 2000
    sink = torch.zeros(grid * 256, dtype=torch.int32, device=dev)
    ms = timed(lambda: check(lib.sbl_probe_mfma_i8(sink.data_ptr(), grid, iters, st)))
    tops = grid * 4 * 4 * iters * 65536 / (ms * 1e-3) / 1e12
    del sink
    torch.cuda.empty_cache()
    khz = ctypes.c_int(0)
    clock = khz.value / 1000.0 if lib.sbl_probe_clock_khz(ctypes.byref(khz)) == 0 else None
    return {"peak_engine_clock_MHz": clock,
            "stream_read_GBps": round(best, 1), "stream_read_workgroups": best_grid,
            "stream_read_frac_of_peak": round(best / HBM_PEAK_GBPS, 4),
            "mfma_i8_TOPS": round(tops, 1), "mfma_i8_frac_of_peak": round(tops / INT8_PEAK_TOPS, 4)}


def annotate_measured(line, peaks):
    """Each roofline also as a fraction of the measured peak of its bound."""
    def add(r):
        if not r:
            return
        if r.get("bound") == "hbm" and r.get("unit") == "GB/s":
            r["frac_of_measured"] = round(r["achieved"] / peaks["stream_read_GBps"], 4)
        elif r.get("bound") == "mfma" and r.get("peak") == INT8_PEAK_TOPS:
            r["frac_of_measured"] = round(r["achieved"] / peaks["mfma_i8_TOPS"], 4)
    add(line.get("roofline"))
    for k, v in line.items():
        if k.startswith("headline_") and isinstance(v, dict):
            add(v.get("roofline"))
    for p in line.get("prefill") or []:
        add(p.get("roofline"))


def references(torch, dev, tm):
    """Measured library rates for reference (not part of the path), HIP events around 10
    runs each: torch's fp32 sum over 2 GB (bytes read), a 1 GB device copy (read +
    written), and two GEMMs at the 3B-class gate shape with 2048 tokens (2048 x 3200 by
    3200 x 8640): int8 -> int32 (torch._int_mm) and BF16 (torch.matmul)."""
    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(10):
            fn()
        return tm.stop_ms() / 10

    out = {}
    a = torch.ones(512 << 20, dtype=torch.float32, device=dev)
    out["sum_fp32_GBps"] = round((2 << 30) / (timed(lambda: a.sum()) * 1e-3) / 1e9, 1)
    del a
    src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out["copy_GBps"] = round((2 << 30) / (timed(lambda: dst.copy_(src)) * 1e-3) / 1e9, 1)
    del src, dst
    m_tok, k, n_out = 2048, 3200, 8640
    flops = 2 * m_tok * k * n_out
    out["gemm_shape"] = f"{m_tok} x {k} by {k} x {n_out}"
    g = torch.Generator(device=dev).manual_seed(3)
    try:
        a = torch.randint(-127, 128, (m_tok, k), generator=g, device=dev, dtype=torch.int8)
        b = torch.randint(-1, 2, (n_out, k), generator=g, device=dev, dtype=torch.int8).t()
        t = flops / (timed(lambda: torch._int_mm(a, b)) * 1e-3) / 1e12
        out["int8_TOPS"], out["int8_frac"] = round(t, 1), round(t / INT8_PEAK_TOPS, 4)
    except (RuntimeError, AttributeError) as e:
        out["int8_error"] = str(e).splitlines()[0][:160]
    a = torch.randn((m_tok, k), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((k, n_out), generator=g, device=dev).to(torch.bfloat16)
    t = flops / (timed(lambda: torch.matmul(a, b)) * 1e-3) / 1e12
    out["bf16_TFLOPS"], out["bf16_frac"] = round(t, 1), round(t / BF16_PEAK_TFLOPS, 4)
    del a, b
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(np, args, budget_s):
    """The CPU oracle, untuned, on a bounded sample of the headline workload: the decode
    of 1024 rows of the block's first matrix shape (8192 wide at 70B), one token.
    Untimed, once: the oracle's own weight preparation and packing of those rows (a
    decoder's load time).  Timed, repeated until about budget_s seconds: reading the
    packed format back (the oracle's panel-order and N:M unpacking), the activation
    quantization, the contraction and the rescale."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import sbl_oracle as O
    fmt, n, m = FORMATS[args.fmt]
    _, no, k = mats_of(args.block)[0]
    wname = BLOCKS[args.block][0]
    rows = 1024
    x = synth.workload_acts(wname, 0, args.m_tok, k)
    bits = synth.workload_masters(wname, 0, no, k)[:rows]
    beta, keep, codes = O.quant_weights(bits, n, m)
    if fmt == 1:
        stored = (O.to_panels(O.pack_nm(codes, keep, n, m), 16 * n // m), O.to_panels(O.pack_bitmap(keep), 8))
    else:
        stored = (O.to_panels(O.pack_dense2(codes), 16), None)
    nbytes = sum(a.size for a in stored if a is not None)
    cores = len(os.sched_getaffinity(0))
    stages = dict.fromkeys(("unpack", "quant_acts", "contract", "rescale"), 0.0)
    reps = 0
    with threadpool_limits(cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while sum(stages.values()) < budget_s and reps < 1000:
            t = time.perf_counter()
            if fmt == 1:
                c2 = O.unpack_nm(O.from_panels(stored[0], rows, k * n // (4 * m), 16 * n // m),
                                 O.from_panels(stored[1], rows, k // 8, 8), n, m, k)
            else:
                c2 = O.unpack_dense2(O.from_panels(stored[0], rows, k // 4, 16), k)
            t1 = time.perf_counter()
            q, gamma = O.quant_acts(x)
            t2 = time.perf_counter()
            acc = O.contract(c2, q)
            t3 = time.perf_counter()
            O.rescale(acc, beta, gamma)
            t4 = time.perf_counter()
            for s_, dt in zip(stages, (t1 - t, t2 - t1, t3 - t2, t4 - t3)):
                stages[s_] += dt
            reps += 1
    total = sum(stages.values())
    try:
        model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except (OSError, StopIteration):
        model = None
    return {"value": round(reps * nbytes / total / 1e9, 5), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} decodes of {rows} x {k} rows of the block's first matrix ({args.fmt}, "
                      f"M={args.m_tok}): {total:.1f} s of timed oracle work (NumPy; BLAS contraction on "
                      f"{threads} threads, other stages one thread); packed weight bytes per second",
            "stages_s": {s_: round(v, 4) for s_, v in stages.items()},
            "weights_per_s": round(reps * rows * k / total, 1), "host_cpus": cores, "host_cpu_model": model}


# --------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args)
        return
    if args.record_traffic:
        record_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}): the path runs on one MI355X "
              "here; how it would shard across GPUs is described, not built", file=sys.stderr)
        sys.exit(2)
    sections = set(args.sections.split(","))
    bad = sections - set(SECTIONS)
    if bad:
        raise SystemExit(f"unknown sections: {sorted(bad)}")
    import numpy as np
    import torch

    from sparse_linear_layers_absmean_amd import sbl

    sbl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tm = Timer(torch)
    if args.copy_calibration_mb > 0:
        nb = int(args.copy_calibration_mb * 1e6) // 16 * 16
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t0 = time.time()
    line = {}
    masters = {}
    peaks = measured_peaks(torch, dev, tm) if "peaks" in sections else None
    if peaks:
        line["measured_peaks"] = peaks
    pre_blocks = {c.split(":")[0] for c in args.prefill_cases.split(",")} if "prefill" in sections else set()
    if "backward" in sections or "3b" in pre_blocks:
        masters["3b"] = synth_masters("3b", mats_of("3b"))
    if "train13b" in sections or "13b" in pre_blocks:
        masters["13b"] = synth_masters("13b", mats_of("13b"))
    if "prefill" in sections:
        line["prefill"] = bench_prefill(torch, np, sbl, dev, tm, masters, args.prefill_cases)
    if "train13b" in sections:
        line["train_step_13b"] = bench_train13b(torch, np, sbl, dev, tm, masters["13b"])
        line["train_step_13b_dense2"] = bench_train13b(torch, np, sbl, dev, tm, masters["13b"], "dense2")
    masters.pop("13b", None)
    if "act_quant" in sections:
        line["act_quant"] = bench_act_quant(torch, sbl, dev, tm)
    if "weight_prep" in sections:
        line["weight_prep"] = weight_prep_sweep(torch, np, sbl, dev, tm, args.prep_blocks)
    if "step0p7b" in sections:
        line["step_0p7b"] = bench_step0p7b(torch, np, sbl, dev, tm)
    if "gemv" in sections:
        line["gemv"] = gemv_sweep(torch, np, sbl, dev, tm)
    if "backward" in sections:
        line["backward"] = bench_backward(torch, np, sbl, dev, tm, masters["3b"])
    masters.clear()
    if "group_scales" in sections:
        line["group_scales"] = bench_group_scales(torch, np, sbl, dev, tm)
    if "references" in sections:
        line["measured_library"] = references(torch, dev, tm)
    head = None
    if "headline" in sections:
        # the same step with the weights in the other storage format, then
        # the headline itself last, so that its timed steps end a profiled run
        alt = "nm68" if args.fmt == "dense2" else "dense2"
        other = bench_decode_step(torch, np, sbl, dev, tm, argparse.Namespace(**{**vars(args), "fmt": alt}))
        line["headline_" + alt] = {"format": alt, "value": round(other["gbps"], 1), "unit": "GB/s",
                                    "ms_per_step": round(other["step_ms"], 5),
                                    "frac_of_hbm_peak": round(other["gbps"] / HBM_PEAK_GBPS, 4),
                                    "packed_weight_bytes_per_step": other["wbytes"], "roofline": other["roofline"]}
        head = bench_decode_step(torch, np, sbl, dev, tm, args)
    cpu = cpu_baseline(np, args, args.cpu_seconds) if "cpu" in sections else None
    fmt_desc = {"dense2": "6:8-masked ternary codes packed 2 bits per weight (DENSE2)",
                "nm68": "6:8 N:M: kept ternary codes 2 bits each + 8-bit bitmap per 8 weights",
                "nm24": "2:4 N:M: kept ternary codes 2 bits each + 4-bit bitmap per 4 weights"}[args.fmt]
    desc = f"Decode GEMV, M={args.m_tok} token(s), {BLOCKS[args.block][3]}, {fmt_desc}"
    out = {
        "metric": METRIC,
        "value": round(head["gbps"], 1) if head else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 5) if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic: " + (head["master_src"] if head else "") + ", N(0,1) fp32 activations; "
                "seeded CPU generators elsewhere",
        "config": {"workload": desc, "format": args.fmt, "m_tok": args.m_tok, "matrices": 7,
                   "block_weights": head["weights"] if head else None,
                   "packed_weight_bytes_per_step": head["wbytes"] if head else None,
                   "rotation_copies": head["copies"] if head else None,
                   "step": "per input (q/k/v, o, gate/up, down): sbl_linear_acts_batch = per-token int8 "
                           "quantization + ternary x int8 GEMV + fp32 rescale, one fused launch; weights "
                           "prepared by sbl_quant_weights_batch before timing"},
        "roofline": head["roofline"] if head else None,
        "frac_of_hbm_peak": round(head["gbps"] / HBM_PEAK_GBPS, 4) if head else None,
    }
    out.update(line)
    if peaks:
        annotate_measured(out, peaks)
    out["cpu_baseline"] = cpu
    out["bench_s"] = round(time.time() - t0, 1)
    out["device"] = torch.cuda.get_device_name(0)
    out["device_arch"] = getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
