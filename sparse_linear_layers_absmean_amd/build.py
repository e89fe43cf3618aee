"""Build libsbl.so (all HIP sources + the C ABI) in-tree for gfx950 with hipcc, and the
benchmark's peak probes (libsbl_probe.so)."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsbl.so")
PROBE_LIB = os.path.join(PKG, "libsbl_probe.so")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # IEEE fp32 semantics: correctly rounded division, no contraction, no fast-math
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    # never emit packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsbl)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libsbl.so")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object in parallel (each is its own
    translation unit), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[hipcc(), *compile_flags, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or max(1, min(len(cmds), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the benchmark's peak probes: a library of their own, outside the path
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, os.path.join(PKG, "probe", "peaks.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
