"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
(via the thin binding) and the CPU oracle on the same seeded inputs."""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import sbl_oracle as O

FMT_DENSE2, FMT_NM = 0, 1
Y_RTOL = 1e-6          # fp32 outputs: relative error bound (exact zeros where acc == 0)


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def par_map(fn, args):
    """fn over args on a thread pool, results in order (the oracle's NumPy
    array operations release the interpreter lock)."""
    args = list(args)
    if len(args) <= 1:
        return [fn(a) for a in args]
    with ThreadPoolExecutor(min(_workers(), len(args))) as ex:
        return list(ex.map(fn, args))


def _row_blocks(n_rows: int):
    step = max(16, -(-n_rows // (4 * _workers())))
    return [(r, min(r + step, n_rows)) for r in range(0, n_rows, step)]


def oracle_weight_rows(bits: np.ndarray, beta, n: int, m: int):
    """The oracle's mask and masked codes for a whole matrix, by row blocks
    (rows are independent given beta): (keep bool, codes int8)."""
    def one(rr):
        b = bits[rr[0]:rr[1]]
        keep = O.nm_keep(b, n, m)
        return keep, O.ternarize(b, beta) * keep.astype(np.int8)
    parts = par_map(one, _row_blocks(bits.shape[0]))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_packed_panels(codes: np.ndarray, keep: np.ndarray, fmt: int, n: int, m: int):
    """The oracle's packed stream and N:M metadata (None for DENSE2), in the
    panel-major storage order, flat."""
    def one(rr):
        c, kp = codes[rr[0]:rr[1]], keep[rr[0]:rr[1]]
        return O.pack_dense2(c) if fmt == FMT_DENSE2 else O.pack_nm(c, kp, n, m)
    rows = np.concatenate(par_map(one, _row_blocks(codes.shape[0])))
    packed = O.to_panels(rows, block_bytes(fmt, n, m))
    meta = O.to_panels(O.pack_bitmap(keep), 8) if fmt == FMT_NM else None
    return packed, meta


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_quant_weights(bits: np.ndarray, n: int, m: int, fmt: int):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = bits.shape
    w = to_dev(bits)
    beta = torch.empty(1, dtype=torch.float32, device="cuda")
    mask = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda")
    codes = torch.empty((n_out, k), dtype=torch.int8, device="cuda")
    packed = torch.empty(sbl.sbl_packed_bytes(n_out, k, n, m, fmt), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_out, k // 8), dtype=torch.uint8, device="cuda") if fmt == FMT_NM else None
    ws = sbl.new_workspace(n_out, k)
    sbl.sbl_quant_weights(w, n, m, beta, ws, mask_bits=mask, codes=codes, fmt=fmt, packed=packed,
                          meta=meta)
    return dict(beta=beta, mask=mask, codes=codes, packed=packed, meta=meta)


def gpu_forward(bits: np.ndarray, x: np.ndarray, n: int, m: int, fmt: int):
    import torch
    from sparse_linear_layers_absmean_amd import sbl
    n_out, k = bits.shape
    out = gpu_quant_weights(bits, n, m, fmt)
    xd = to_dev(x.astype(np.float32))
    xq, gamma = sbl.quant_acts(xd)
    y, acc = sbl.linear(out["packed"], out["meta"], fmt, n, m, out["beta"], xq, gamma, n_out,
                        want_acc=True)
    torch.cuda.synchronize()
    res = {key: (to_np(v) if v is not None else None) for key, v in out.items()}
    res.update(xq=to_np(xq), gamma=to_np(gamma), y=to_np(y), acc=to_np(acc))
    return res


def oracle_forward(bits: np.ndarray, x: np.ndarray, n: int, m: int):
    r = O.forward(bits, x, n, m)
    r["bitmap"] = O.pack_bitmap(r["keep"])
    r["dense2"] = O.pack_dense2(r["codes"])
    r["nm"] = O.pack_nm(r["codes"], r["keep"], n, m) if (bits.shape[1] * n // m) % 4 == 0 else None
    r["n"], r["m"] = n, m
    return r


def block_bytes(fmt: int, n: int, m: int) -> int:
    """Bytes of one 64-weight block of the packed stream."""
    return 16 if fmt == FMT_DENSE2 else 16 * n // m


def packed_rows(flat, n_out: int, k: int, fmt: int, n: int, m: int, rows=None):
    """Row-major content of a panel-major packed stream (all rows or `rows`)."""
    b = block_bytes(fmt, n, m)
    return O.from_panels(np.asarray(flat).reshape(-1), n_out, k // 64 * b, b, rows)


def meta_rows(flat, n_out: int, k: int, rows=None):
    """Row-major BITMAP of panel-major N:M metadata (all rows or `rows`)."""
    return O.from_panels(np.asarray(flat).reshape(-1), n_out, k // 8, 8, rows)


def check_y(y_gpu, y_ref, acc_ref):
    nz = acc_ref != 0
    assert np.all(y_gpu[~nz] == 0)
    if nz.any():
        rel = np.abs(y_gpu[nz].astype(np.float64) / y_ref[nz].astype(np.float64) - 1.0)
        assert rel.max() <= Y_RTOL, rel.max()


def compare_all(g, r, fmt: int, n_out: int):
    assert g["beta"][0] == r["beta"], (g["beta"][0], r["beta"])
    assert np.array_equal(g["mask"], r["bitmap"])
    assert np.array_equal(g["codes"], r["codes"])
    k = g["codes"].shape[1]
    if fmt == FMT_DENSE2:
        assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, 8, 8), r["dense2"])
    else:
        n, m = r["n"], r["m"]
        assert np.array_equal(packed_rows(g["packed"], n_out, k, fmt, n, m), r["nm"])
        assert np.array_equal(meta_rows(g["meta"], n_out, k), r["bitmap"])
    assert np.array_equal(g["gamma"], r["gamma"])
    assert np.array_equal(g["xq"], r["q"])
    assert np.array_equal(g["acc"], r["acc"])
    check_y(g["y"], r["y"], r["acc"])
