"""Seeded synthetic inputs for the Sparse-BitLinear workloads.

This module only *draws* inputs: BF16 master weights and fp32 activations
with the shapes and value distributions of the five workloads (a 256x256
unit layer, 0.7B/3B/13B/70B-class transformer blocks).  It holds none of the
layer's arithmetic (no scales, masks, codes or products), so both the CPU
oracle and the HIP path can be fed from it without sharing any method code.

Distributions:
  * master weights: fp32 N(0, 0.02^2), rounded to BF16 (round to nearest even);
    the 3B-class blocks scale a seeded 1% of entries by 10 before rounding;
    the 13B-class training workload then plants exact and near ties on the
    6:8 keep boundary (`plant_ties`).
  * activations: fp32 N(0, 1); the 3B decode workload scales 8 seeded channels
    by 20; the 3B prefill workload draws a seeded 25% of rows from Student-t(4).

Seeds: the unit layer uses seed 0 (weights) and seed 1 (activations); every
other matrix uses numpy.random.default_rng([workload, matrix_index, role])
with role 0 = weights, 1 = activations, 2 = tie planting, and an extra
trailing copy index for the benchmark's rotation pool.
"""

from __future__ import annotations

import numpy as np

ROLE_W, ROLE_X, ROLE_TIES = 0, 1, 2

# Transformer-block matrices as (name, n_out, k) for hidden h and FFN width f.
# The weight layout is [n_out][k], the same orientation as a torch Linear.
def block_shapes(h: int, f: int):
    return [("q", h, h), ("k", h, h), ("v", h, h), ("o", h, h),
            ("gate", f, h), ("up", f, h), ("down", h, f)]


WORKLOADS = {
    # name: (workload id, hidden, ffn)
    "unit256": (1, 256, None),
    "b0p7": (2, 1536, 4096),
    "b3": (3, 3200, 8640),
    "b3_prefill": (4, 3200, 8640),
    "b13": (5, 5120, 13824),
    "b70": (6, 8192, 28672),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to BF16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng_for(workload: int, matrix_index: int, role: int, copy: int | None = None):
    key = [workload, matrix_index, role] if copy is None else [workload, matrix_index, role, copy]
    return np.random.default_rng(key)


def gaussian_masters(rng, n_out: int, k: int, sigma: float = 0.02,
                     outlier_frac: float = 0.0, outlier_scale: float = 10.0) -> np.ndarray:
    w = rng.standard_normal((n_out, k), dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0.0:
        hit = rng.random((n_out, k)) < outlier_frac
        w[hit] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(w)


def plant_ties(bits: np.ndarray, rng, m: int = 8, n: int = 6, frac_exact: float = 0.25,
               frac_near: float = 0.25) -> np.ndarray:
    """Plant exact and near magnitude ties on the n:m keep boundary.

    Groups are m consecutive positions of a row.  The boundary magnitude b of
    a group is its n-th largest |w| (the smallest one an n:m mask keeps).
      * In a seeded `frac_exact` of the groups, three positions take the
        magnitude b: one of the m - n positions below the boundary and two
        others drawn at random (never the position holding b).  Each such
        group then has equal magnitudes on both sides of the boundary.
      * In a disjoint `frac_near` of the groups, one position below the
        boundary takes b + s and another random position b - s, with
        s = +-1 BF16 ulp: the n-th and (n+1)-th largest magnitudes then
        differ by at most one ulp.
    Signs are kept; only the 15 magnitude bits change.
    """
    b = bits.reshape(-1, m).copy()
    g = b.shape[0]
    rows = np.arange(g)
    mag = (b & 0x7FFF).astype(np.int32)
    order = np.argsort(-mag, axis=1, kind="stable")
    src = order[:, n - 1]
    bmag = mag[rows, src]
    u = rng.random(g)
    exact = u < frac_exact
    near = (u >= frac_exact) & (u < frac_exact + frac_near)
    low = order[rows, n + rng.integers(0, m - n, g)]
    keys = rng.random((g, m))
    keys[rows, src] = 2.0
    keys[rows, low] = 2.0
    others = np.argsort(keys, axis=1)[:, :2]
    s = np.where(rng.random(g) < 0.5, -1, 1)

    def put(sel, col, value):
        r, c = rows[sel], col[sel]
        v = np.clip(value[sel], 0, 0x7F7F)
        b[r, c] = (b[r, c] & 0x8000) | v.astype(np.uint16)

    put(exact, low, bmag)
    put(exact, others[:, 0], bmag)
    put(exact, others[:, 1], bmag)
    put(near, low, bmag + s)
    put(near, others[:, 0], bmag - s)
    return b.reshape(bits.shape)


def rare_mixture(rng, n_out: int, k: int) -> np.ndarray:
    """BF16 bit patterns drawn in five equal parts: zeros, subnormals, tiny
    normals (below 2^-31), mid-range normals and large values up to 2^127,
    each with a random sign.  Stresses every range of the scale sums."""
    kind = rng.integers(0, 5, (n_out, k))
    mag = np.select([kind == 0, kind == 1, kind == 2, kind == 3],
                    [0, rng.integers(1, 0x80, (n_out, k)), rng.integers(0x0080, 0x3000, (n_out, k)),
                     rng.integers(0x3000, 0x4000, (n_out, k))],
                    rng.integers(0x4000, 0x7F00, (n_out, k)))
    return (mag | (rng.integers(0, 2, (n_out, k)) << 15)).astype(np.uint16)


def gaussian_acts(rng, m_tok: int, k: int, hot_channels: int = 0, hot_scale: float = 20.0,
                  t_row_frac: float = 0.0, t_nu: float = 4.0) -> np.ndarray:
    x = rng.standard_normal((m_tok, k), dtype=np.float32)
    if t_row_frac > 0.0:
        rows = rng.random(m_tok) < t_row_frac
        nt = int(rows.sum())
        if nt:
            x[rows] = rng.standard_t(t_nu, size=(nt, k)).astype(np.float32)
    if hot_channels > 0:
        ch = rng.choice(k, hot_channels, replace=False)
        x[:, ch] *= np.float32(hot_scale)
    return x


def workload_masters(name: str, matrix_index: int, n_out: int, k: int, copy: int | None = None):
    """BF16 master bits for one matrix of a named workload."""
    wid = WORKLOADS[name][0]
    if name == "unit256":
        rng = np.random.default_rng(0 if copy is None else [0, copy])
        return gaussian_masters(rng, n_out, k)
    rng = rng_for(wid, matrix_index, ROLE_W, copy)
    if name in ("b3", "b3_prefill"):
        return gaussian_masters(rng, n_out, k, outlier_frac=0.01)
    bits = gaussian_masters(rng, n_out, k)
    if name == "b13":
        bits = plant_ties(bits, rng_for(wid, matrix_index, ROLE_TIES, copy))
    return bits


def workload_acts(name: str, matrix_index: int, m_tok: int, k: int, copy: int | None = None):
    """fp32 activations [m_tok][k] for one matrix of a named workload."""
    wid = WORKLOADS[name][0]
    if name == "unit256":
        rng = np.random.default_rng(1 if copy is None else [1, copy])
        return gaussian_acts(rng, m_tok, k)
    rng = rng_for(wid, matrix_index, ROLE_X, copy)
    if name == "b3":
        return gaussian_acts(rng, m_tok, k, hot_channels=8)
    if name == "b3_prefill":
        return gaussian_acts(rng, m_tok, k, t_row_frac=0.25)
    return gaussian_acts(rng, m_tok, k)
