"""Plain CPU oracle for the Sparse-BitLinear (W1.58A8, N:M) forward path.

TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct definition the
HIP kernels are checked against.  Only the test-suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the library never does,
and it shares no code, tables or constants with the GPU path.  Inputs come
from the seeded generators in `synth.py`, which hold none of this arithmetic.

Sources (the method pages; sections, equations and items named per page):
  [SB-es]  "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
           Semi-Structured Sparsity", gist.science Spanish summary,
           "Resumen tecnico", sections 1 (Problema), 2 (Metodologia) and
           3 (Contribuciones Clave; item 3: the training-design ablations).
  [SB-ar]  the same paper, gist.science Arabic summary, section 2
           (Methodology): items "Ternary Quantization", "Dynamic N:M
           Masking", "Mask Generation", "Quant-Then-Mask Order".
  [BN-cpp] "Marco de inferencia de Microsoft lleva modelos de lenguaje
           grande de 1 bit a dispositivos locales" (unite.ai), section
           "Fundamento matematico": activation quantization (item 2) and the
           BitLinear operation (item 3).
  [BN-spec] "Introduccion Detallada al Proyecto BitNet" (aibars.net),
           "Especificaciones Tecnicas": W1.58A8, absmean weights, 8-bit
           activations, no bias.

Readings taken where the pages are silent or garbled (each one is also
listed with its reason in the design notes):
  * beta is ONE scale per weight matrix: the exact mean of |w| over all
    n_out*k BF16 master values (pruned ones included, because quantization
    comes before the mask), rounded once to fp32, nearest-even.  The value
    used for scaling is beta_eff = max(beta, 1e-5f).
  * codes: c = RoundClip(w / beta_eff, -1, 1), round half to even.
  * the N:M groups are m consecutive positions along k inside one output row;
    the mask keeps exactly n per group, the n largest |w| of the BF16 master,
    ties to the lower index; +0 and -0 tie.
  * activations: per token, gamma = max_k |x|, gamma_eff = max(gamma, 1e-5f),
    q = clamp(rint(RN_fp32(Qb * x / gamma_eff)), -127, 127) with Qb = 128 and
    rint rounding half to even.  RN_fp32(Qb*x/gamma) is evaluated as the
    single correctly-rounded fp32 quotient x / (gamma_eff / 128), where the
    divisor is exact.
  * rescale: y = RN_fp32(fp32(acc) * RN_fp32(RN_fp32(beta_eff * gamma_eff) * 2^-7)).
  * byte formats (the pages only speak of "metadata" for the kernel) are
    defined in `pack_dense2`, `pack_bitmap` and `pack_nm` below, and the
    storage order of the packed streams in `to_panels`; they are this
    implementation's choice, not the pages'.

Group scales (`quant_weights_grouped`, `rescale_grouped`): one absmean
beta per block of consecutive output rows instead of one per matrix.
Activation groups (`quant_acts_kgrouped`, `linear_kgrouped`): one gamma per
token and block of kg features; each block's product is rescaled on its own
and the blocks' fp32 results are added in ascending block order.
Block scales (`quant_weights_blocked`): one absmean beta per block of
consecutive output rows x consecutive features (the weight groups of the same
section taken along k as well); `linear_kgrouped` then takes one beta per row
group and feature block, the feature blocks being those of the activations.

Backward (dual straight-through estimator; readings listed with the
function `backward`): the scales are constants, the incoming gradient is
BF16, dX passes only where the activation clamp did not act, and dW reaches
every master (pruned ones included).

Non-finite inputs are a precondition violation: the functions raise.

Pinned by tests/test_oracle_*.py (exact-rational brute force, enumeration of
all C(m, n) subsets, Python-int contraction, closed-form statistics, the
hand-derived 16-weight worked example and format round trips).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

QB = 128                # 2^(b-1) for b = 8 bit activations  [BN-cpp] item 2
Q_CLIP = 127            # symmetric int8 clip  [BN-spec]
EPS_SCALE = np.float32(1e-5)


# --------------------------------------------------------------------------
# BF16 helpers
# --------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> fp32 values (exact: BF16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _check_finite_bf16(bits: np.ndarray) -> None:
    if np.any((np.asarray(bits, dtype=np.uint16) & 0x7F80) == 0x7F80):
        raise ValueError("non-finite BF16 master weight")


# --------------------------------------------------------------------------
# exact rounding of a non-negative rational to fp32
# --------------------------------------------------------------------------

def rational_to_f32(num: int, den: int) -> np.float32:
    """Round num/den (num >= 0, den > 0) to the nearest fp32, ties to even.

    Integer arithmetic only: find the binade, take 24 significant bits (or the
    fixed 2^-149 grid for subnormals), and round on the exact remainder.
    """
    if num < 0 or den <= 0:
        raise ValueError("rational_to_f32 needs num >= 0 and den > 0")
    if num == 0:
        return np.float32(0.0)
    # e = floor(log2(num/den))
    e = num.bit_length() - den.bit_length()
    if (num << max(0, -e)) < (den << max(0, e)):
        e -= 1
    lsb = max(e - 23, -149)          # exponent of the last kept bit
    if lsb >= 0:
        n2, d2 = num, den << lsb
    else:
        n2, d2 = num << (-lsb), den
    q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (q & 1)):
        q += 1
    val = float(q) * 2.0 ** lsb     # exact in fp64 (q <= 2^24)
    if val >= 2.0 ** 128:
        return np.float32(np.inf)
    return np.float32(val)


# --------------------------------------------------------------------------
# a1: beta, the absmean weight scale  [SB-ar] "Ternary Quantization";
#     [BN-spec] absmean weights
# --------------------------------------------------------------------------

def absmean_exact(bits: np.ndarray, keep=None) -> Fraction:
    """Exact mean of |w| over every BF16 value of the matrix, or over the
    values where `keep` is true (the mask-then-quant ablation).

    A finite BF16 magnitude is sig * 2^(max(e,1) - 134) with e the biased
    exponent and sig = mantissa | (e != 0) << 7, i.e. an integer number of
    2^-133 units.  Per-exponent sums of sig are exact in float64 (each sum is
    an integer below 2^53), so the total is an exact Python integer.
    """
    b = np.asarray(bits, dtype=np.uint16).ravel()
    if b.size == 0:
        raise ValueError("empty weight matrix")
    _check_finite_bf16(b)
    if keep is not None:
        b = b[np.asarray(keep, dtype=bool).ravel()]
        if b.size == 0:
            raise ValueError("nothing kept")
    mag = (b & 0x7FFF).astype(np.int64)
    e = mag >> 7
    sig = (mag & 0x7F) | ((e != 0).astype(np.int64) << 7)
    per_e = np.bincount(e, weights=sig.astype(np.float64), minlength=256)
    total = 0
    for ei in range(256):
        s = int(per_e[ei])
        if s:
            total += s << (max(ei, 1) - 1)   # units of 2^-133
    return Fraction(total, b.size << 133)


def absmean_beta(bits: np.ndarray, keep=None) -> np.float32:
    """beta = RN_fp32(mean |w|): one scale per weight matrix (over the kept
    values only when `keep` is given)."""
    f = absmean_exact(bits, keep)
    return rational_to_f32(f.numerator, f.denominator)


def beta_eff(beta) -> np.float32:
    return np.maximum(np.float32(beta), EPS_SCALE)


# --------------------------------------------------------------------------
# a3: ternarization  c = RoundClip(w / beta_eff, -1, 1)
# --------------------------------------------------------------------------

def ternarize(bits: np.ndarray, beta) -> np.ndarray:
    """Ternary codes in {-1, 0, +1} (int8), same shape as `bits`.

    w / beta_eff is formed in float64.  It cannot land on the wrong side of
    +-1/2: when |w| != beta_eff/2 the exact ratio differs from 1/2 by at
    least 2^-25 (both are fp32 grid values), far beyond float64 rounding, and
    when |w| == beta_eff/2 the quotient 1/2 is exact; rint then rounds that
    tie to even (to 0).
    """
    _check_finite_bf16(bits)
    w = bf16_to_f32(bits).astype(np.float64)
    r = np.rint(w / np.float64(beta_eff(beta)))
    return np.clip(r, -1, 1).astype(np.int8)


# --------------------------------------------------------------------------
# a2: N:M mask from the BF16 master magnitudes  [SB-es] section 2 (mask
#     generation from master weights); [SB-ar] "Dynamic N:M Masking",
#     "Mask Generation"
# --------------------------------------------------------------------------

def nm_keep(bits: np.ndarray, n: int, m: int) -> np.ndarray:
    """Boolean keep-mask [n_out][k]: exactly n kept in each group of m along k.

    rank_j = #{i : |w_i| > |w_j|} + #{i < j : |w_i| == |w_j|}; keep_j = rank_j < n.
    """
    b = np.asarray(bits, dtype=np.uint16)
    _check_finite_bf16(b)
    return top_n_keep(np.abs(bf16_to_f32(b)), n, m)


def top_n_keep(mag: np.ndarray, n: int, m: int) -> np.ndarray:
    """The same rank rule for any magnitudes [n_out][k] (|w| of the masters,
    or |c| of the codes for the masks-from-quantized-weights ablation)."""
    mag = np.asarray(mag)
    n_out, k = mag.shape
    if m < 1 or n < 1 or n > m or k % m:
        raise ValueError("bad N:M pattern for this shape")
    mag = mag.reshape(n_out, k // m, m)
    keep = np.empty((n_out, k // m, m), dtype=bool)
    idx = np.arange(m)
    lower = idx[None, :] < idx[:, None]          # lower[j, i] = i < j
    step = max(1, (1 << 22) // max(1, k * m))
    for r0 in range(0, n_out, step):
        a = mag[r0:r0 + step]                     # [R, G, m]
        wj = a[..., :, None]                      # j along axis -2
        wi = a[..., None, :]                      # i along axis -1
        rank = (wi > wj).sum(-1) + ((wi == wj) & lower).sum(-1)
        keep[r0:r0 + step] = rank < n
    return keep.reshape(n_out, k)


# --------------------------------------------------------------------------
# a1-a4 together: quant, then mask  [SB-es] section 2 (quant-then-mask);
# [SB-ar] "Quant-Then-Mask Order"
# --------------------------------------------------------------------------

QUANT_THEN_MASK, MASK_THEN_QUANT, MASK_FROM_CODES = "quant_then_mask", "mask_then_quant", "mask_from_codes"


def quant_weights(bits: np.ndarray, n: int, m: int, order: str = QUANT_THEN_MASK):
    """(beta, keep, codes) with codes = RoundClip(w/beta_eff, -1, 1) * keep.

    order (the pages' training-design ablations, [SB-es] section 3 item 3):
      quant_then_mask  the method: beta over every master, mask from the masters;
      mask_then_quant  mask from the masters first, beta over the kept masters only;
      mask_from_codes  beta over every master, then the mask from |codes|
                       (top n per group, ties to the lower index), instead of
                       from the masters.
    """
    if order == QUANT_THEN_MASK:
        beta = absmean_beta(bits)
        keep = nm_keep(bits, n, m)
        codes = ternarize(bits, beta) * keep.astype(np.int8)
    elif order == MASK_THEN_QUANT:
        keep = nm_keep(bits, n, m)
        beta = absmean_beta(bits, keep)
        codes = ternarize(bits, beta) * keep.astype(np.int8)
    elif order == MASK_FROM_CODES:
        beta = absmean_beta(bits)
        c = ternarize(bits, beta)
        keep = top_n_keep(np.abs(c), n, m)
        codes = c * keep.astype(np.int8)
    else:
        raise ValueError(f"unknown order {order!r}")
    return beta, keep, codes.astype(np.int8)


# --------------------------------------------------------------------------
# a5: byte formats
# --------------------------------------------------------------------------

def pack_dense2(codes: np.ndarray) -> np.ndarray:
    """DENSE2: 2 bits per weight, u = c + 1 in {0,1,2} (3 is never written).

    Row r occupies bytes r*(k/4) .. r*(k/4) + k/4 - 1.  Within it, each run of
    16 weights k = 16b .. 16b+15 fills the 4 bytes 4b .. 4b+3: weight k lives
    in byte 4*(k // 16) + (k % 4), at bit offset 2*((k // 4) % 4).  (So byte
    4b + j holds weights 16b + j + 4s at bit pairs s = 0..3: shifting the
    little-endian word right by 2s and masking 0x03030303 yields the u of
    weights 16b+4s .. 16b+4s+3 in byte order.)
    """
    c = np.asarray(codes, dtype=np.int8)
    n_out, k = c.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    u = (c.astype(np.int16) + 1).astype(np.uint8)
    out = np.zeros((n_out, k // 4), dtype=np.uint8)
    for kk in range(16):
        byte = 4 * np.arange(k // 16) + (kk % 4)
        out[:, byte] |= (u[:, kk::16] << (2 * (kk // 4))).astype(np.uint8)
    return out


def unpack_dense2(packed: np.ndarray, k: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n_out = p.shape[0]
    codes = np.empty((n_out, k), dtype=np.int8)
    for kk in range(16):
        byte = 4 * np.arange(k // 16) + (kk % 4)
        codes[:, kk::16] = ((p[:, byte] >> (2 * (kk // 4))) & 3).astype(np.int16) - 1
    return codes


def pack_bitmap(keep: np.ndarray) -> np.ndarray:
    """Bitmap (mask bits / N:M metadata): byte n*(k/8) + k/8, bit k%8 = kept."""
    kp = np.asarray(keep, dtype=bool)
    n_out, k = kp.shape
    if k % 8:
        raise ValueError("k must be a multiple of 8")
    return np.packbits(kp.reshape(n_out, k // 8, 8), axis=-1, bitorder="little").reshape(n_out, k // 8)


def unpack_bitmap(bitmap: np.ndarray, k: int) -> np.ndarray:
    bm = np.asarray(bitmap, dtype=np.uint8)
    return np.unpackbits(bm, axis=-1, bitorder="little")[:, :k].astype(bool)


def pack_nm(codes: np.ndarray, keep: np.ndarray, n: int, m: int) -> np.ndarray:
    """N:M codes: the kept positions of row r, in ascending k, are numbered
    i = 0 .. k*n/m - 1; byte r*(k*n/(4m)) + i/4, bits 2*(i%4)..+1 hold u = c+1.
    Requires exactly n kept per group (k*n/m must be a multiple of 4)."""
    c = np.asarray(codes, dtype=np.int8)
    kp = np.asarray(keep, dtype=bool)
    n_out, k = c.shape
    per_row = k * n // m
    if k % m or per_row % 4:
        raise ValueError("k*n/m must be a multiple of 4")
    if np.any(kp.reshape(n_out, k // m, m).sum(-1) != n):
        raise ValueError("mask must keep exactly n per group")
    kept_u = (c[kp].astype(np.int16) + 1).astype(np.uint8).reshape(n_out, per_row // 4, 4)
    out = np.zeros((n_out, per_row // 4), dtype=np.uint8)
    for s in range(4):
        out |= (kept_u[..., s] << (2 * s)).astype(np.uint8)
    return out


def unpack_nm(packed: np.ndarray, bitmap: np.ndarray, n: int, m: int, k: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n_out = p.shape[0]
    kept_u = np.stack([(p >> (2 * s)) & 3 for s in range(4)], axis=-1).reshape(n_out, -1)
    keep = unpack_bitmap(bitmap, k)
    codes = np.zeros((n_out, k), dtype=np.int8)
    codes[keep] = (kept_u.astype(np.int16) - 1).astype(np.int8).ravel()
    return codes


# --------------------------------------------------------------------------
# a5: storage order of a packed stream (this implementation's choice, like the
#     byte formats above; the pages fix neither)
# --------------------------------------------------------------------------

PANEL_BLOCKS = 4        # 64-weight blocks per panel: panels are 256 weights wide along k


def to_panels(rows: np.ndarray, block_bytes: int) -> np.ndarray:
    """Panel-major storage of a row-major packed stream.

    `rows` is [n_out][row_bytes], every 64-weight block of a row taking
    `block_bytes` bytes (DENSE2 16, N:M codes 16*n/m, bitmap 8).  The k axis
    is cut into panels of PANEL_BLOCKS blocks; panel p holds, row after row,
    the bytes of blocks 4p .. 4p+3 of every row (a last panel may hold fewer
    blocks).  Returns the flat byte string.
    """
    r = np.asarray(rows, dtype=np.uint8)
    if r.ndim != 2 or r.shape[1] % block_bytes:
        raise ValueError("rows must be [n_out][whole blocks]")
    width = PANEL_BLOCKS * block_bytes
    return np.concatenate([r[:, s:s + width].reshape(-1) for s in range(0, r.shape[1], width)])


def from_panels(flat: np.ndarray, n_out: int, row_bytes: int, block_bytes: int, rows=None) -> np.ndarray:
    """Inverse of `to_panels`: the row-major bytes of all rows, or of `rows`."""
    f = np.asarray(flat, dtype=np.uint8).reshape(-1)
    if f.size != n_out * row_bytes or row_bytes % block_bytes:
        raise ValueError("size mismatch")
    sel = np.arange(n_out) if rows is None else np.asarray(rows, dtype=np.int64)
    width = PANEL_BLOCKS * block_bytes
    out = np.empty((sel.size, row_bytes), dtype=np.uint8)
    for s in range(0, row_bytes, width):
        w = min(width, row_bytes - s)
        base = n_out * s                          # every earlier panel is full
        idx = base + sel[:, None] * w + np.arange(w)[None, :]
        out[:, s:s + w] = f[idx]
    return out


# --------------------------------------------------------------------------
# a6: per-token absmax int8 activation quantization  [BN-cpp] item 2;
#     [BN-spec] 8-bit activations
# --------------------------------------------------------------------------

def quant_acts(x: np.ndarray):
    """(q int8 [m_tok][k], gamma fp32 [m_tok]) with gamma = max_k |x|."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite activation")
    gamma = np.abs(x).max(axis=1).astype(np.float32)
    g_eff = np.maximum(gamma, EPS_SCALE)
    s = (g_eff / np.float32(QB)).astype(np.float32)        # exact power-of-two scaling
    t = (x / s[:, None]).astype(np.float32)                 # one IEEE fp32 division
    q = np.clip(np.rint(t), -Q_CLIP, Q_CLIP).astype(np.int8)
    return q, gamma


# --------------------------------------------------------------------------
# a7-a8: ternary x int8 contraction and rescale  [BN-cpp] item 3
#        y = W~ x~ (beta gamma / Qb); no bias [BN-spec]
# --------------------------------------------------------------------------

def contract(codes: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc[t, r] = sum_k codes[r, k] * q[t, k] (int32).

    The float64 matmul is exact: every partial sum is an integer of magnitude
    at most 127*k < 2^53.
    """
    c = np.asarray(codes, dtype=np.int8)
    qq = np.asarray(q, dtype=np.int8)
    if c.shape[1] != qq.shape[1]:
        raise ValueError("k mismatch")
    acc = qq.astype(np.float64) @ c.astype(np.float64).T
    return np.rint(acc).astype(np.int32)


def rescale(acc: np.ndarray, beta, gamma: np.ndarray) -> np.ndarray:
    """y[t, r] = RN(fp32(acc) * RN(RN(beta_eff * gamma_eff[t]) * 2^-7))."""
    b = beta_eff(beta)
    g = np.maximum(np.asarray(gamma, dtype=np.float32), EPS_SCALE)
    s = ((b * g).astype(np.float32) * np.float32(1.0 / QB)).astype(np.float32)
    return (np.asarray(acc).astype(np.float32) * s[:, None]).astype(np.float32)


def linear(codes: np.ndarray, q: np.ndarray, beta, gamma: np.ndarray):
    acc = contract(codes, q)
    return acc, rescale(acc, beta, gamma)


# --------------------------------------------------------------------------
# Group scales  [BN-cpp] section "Cuantizacion y normalizacion de grupos": the
# scale is computed per group of weights instead of per matrix, so groups need
# no communication.  Reading: a group is a block of rows_per_group consecutive
# output rows (the last one may be shorter); each has its own exact absmean
# beta, and its codes use it.  The mask does not depend on beta.  gamma stays
# per token.
# --------------------------------------------------------------------------

def quant_weights_grouped(bits: np.ndarray, n: int, m: int, rows_per_group: int):
    """(betas fp32 [G], keep bool, codes int8): quant-then-mask with one beta per row group."""
    bits = np.asarray(bits, dtype=np.uint16)
    n_out = bits.shape[0]
    if rows_per_group < 1:
        raise ValueError("rows_per_group must be positive")
    keep = nm_keep(bits, n, m)
    betas, codes = [], np.zeros(bits.shape, np.int8)
    for r0 in range(0, n_out, rows_per_group):
        sl = slice(r0, min(n_out, r0 + rows_per_group))
        b = absmean_beta(bits[sl])
        betas.append(b)
        codes[sl] = ternarize(bits[sl], b)
    codes = (codes * keep).astype(np.int8)
    return np.array(betas, np.float32), keep, codes


def quant_weights_blocked(bits: np.ndarray, n: int, m: int, rows_per_group: int, cols_per_group: int):
    """(betas fp32 [Gr][Gk], keep bool, codes int8): quant-then-mask with one beta per
    block of rows_per_group consecutive rows (the last block may be shorter) and
    cols_per_group consecutive features (a multiple of m dividing k).  Each block's beta
    is the method's exact absmean over the block's masters, and the block's codes use it;
    the mask does not depend on beta."""
    bits = np.asarray(bits, dtype=np.uint16)
    n_out, k = bits.shape
    if rows_per_group < 1 or cols_per_group < 1 or k % cols_per_group or cols_per_group % m:
        raise ValueError("rows_per_group >= 1 and cols_per_group a multiple of m dividing k")
    keep = nm_keep(bits, n, m)
    row_starts = range(0, n_out, rows_per_group)
    col_starts = range(0, k, cols_per_group)
    betas = np.zeros((len(row_starts), len(col_starts)), np.float32)
    codes = np.zeros(bits.shape, np.int8)
    for gi, r0 in enumerate(row_starts):
        for gj, c0 in enumerate(col_starts):
            blk = (slice(r0, min(n_out, r0 + rows_per_group)), slice(c0, c0 + cols_per_group))
            betas[gi, gj] = absmean_beta(bits[blk])
            codes[blk] = ternarize(bits[blk], betas[gi, gj])
    codes = (codes * keep).astype(np.int8)
    return betas, keep, codes


def rescale_grouped(acc: np.ndarray, betas: np.ndarray, rows_per_group: int, gamma: np.ndarray) -> np.ndarray:
    """y[t, r] = RN(fp32(acc) * RN(RN(beta_eff[r // rows_per_group] * gamma_eff[t]) * 2^-7))."""
    acc = np.asarray(acc)
    b = np.maximum(np.asarray(betas, dtype=np.float32), EPS_SCALE)
    b_rows = np.repeat(b, rows_per_group)[:acc.shape[1]]
    g = np.maximum(np.asarray(gamma, dtype=np.float32), EPS_SCALE)
    s = ((g[:, None] * b_rows[None, :]).astype(np.float32) * np.float32(1.0 / QB)).astype(np.float32)
    return (acc.astype(np.float32) * s).astype(np.float32)


def quant_acts_kgrouped(x: np.ndarray, kg: int):
    """Activation groups along k: (q int8 [m_tok][k], gamma fp32 [m_tok][k // kg]),
    gamma[t, j] = max |x| over features [j kg, (j + 1) kg) of token t, and each
    feature quantized with its block's gamma exactly as quant_acts does."""
    x = np.asarray(x, dtype=np.float32)
    t, k = x.shape
    if kg < 1 or k % kg:
        raise ValueError("kg must divide k")
    q = np.zeros((t, k), np.int8)
    gam = np.zeros((t, k // kg), np.float32)
    for j in range(k // kg):
        q[:, j * kg:(j + 1) * kg], gam[:, j] = quant_acts(x[:, j * kg:(j + 1) * kg])
    return q, gam


def linear_kgrouped(codes: np.ndarray, q: np.ndarray, betas: np.ndarray, rows_per_group: int,
                    gamma: np.ndarray, kg: int):
    """(acc int32 [m_tok][n_out][G], y fp32): per feature block j the exact
    product acc_j, rescaled with beta of the row's group (betas [Gr]) or of the
    row's group and block j (betas [Gr][G], block scales) and gamma[t, j] (the two
    roundings of rescale), and the blocks' fp32 results added in ascending j."""
    c = np.asarray(codes, dtype=np.int8)
    qq = np.asarray(q, dtype=np.int8)
    b = np.asarray(betas, dtype=np.float32)
    n_out, k = c.shape
    groups = k // kg
    if b.ndim == 2 and b.shape[1] != groups:
        raise ValueError("block scales need one beta per feature block of the activations")
    acc = np.stack([contract(c[:, j * kg:(j + 1) * kg], qq[:, j * kg:(j + 1) * kg]) for j in range(groups)], axis=2)
    y = np.zeros((qq.shape[0], n_out), np.float32)
    for j in range(groups):
        bj = b if b.ndim == 1 else b[:, j]
        y = (y + rescale_grouped(acc[:, :, j], bj, rows_per_group, np.asarray(gamma)[:, j])).astype(np.float32)
    return acc, y


# --------------------------------------------------------------------------
# Backward of the layer: the dual straight-through estimator
#   [SB-es] section 2, "Estrategia de Entrenamiento" (Dual STE: gradients reach
#   every master weight, the pruned ones included);
#   [SB-ar] section 2, item 3 (quantization STE: identity inside the clipping
#   range; mask STE: dense gradient flow to all masters).
# The scales beta and gamma are treated as constants (no gradient through
# them), the incoming gradient dY is BF16, and the results are fp32.
# --------------------------------------------------------------------------

FP32_UNIT = 2.0 ** -24      # unit roundoff of fp32 (round to nearest)


def clip_pass(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """1.0 where the activation quantizer's clamp did not act, else 0.0.

    The quantizer's STE passes the gradient inside the clipping range: where
    |rint(RN_fp32(128 x / gamma_eff))| <= 127, evaluated exactly as in
    quant_acts (the same fp32 division and half-to-even rint)."""
    x = np.asarray(x, dtype=np.float32)
    g_eff = np.maximum(np.asarray(gamma, dtype=np.float32), EPS_SCALE)
    s = (g_eff / np.float32(QB)).astype(np.float32)
    t = np.rint((x / s[:, None]).astype(np.float32))
    return (np.abs(t) <= Q_CLIP).astype(np.float64)


def dequant_acts(q: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """x_hat[t, k] = RN_fp32(gamma_eff[t] * q[t, k]) * 2^-7 (fp32): the
    activation the forward product used, in real terms."""
    g_eff = np.maximum(np.asarray(gamma, dtype=np.float32), EPS_SCALE)
    prod = (g_eff[:, None] * np.asarray(q, dtype=np.float32)).astype(np.float32)
    return (prod * np.float32(1.0 / QB)).astype(np.float32)


def backward(codes: np.ndarray, beta, x: np.ndarray, q: np.ndarray, gamma: np.ndarray,
             dy_bits: np.ndarray, clip: bool = True):
    """Gradients of the layer y = (beta C) x_hat^T under the dual STE.

      dX[t, k] = beta_eff * sum_n dY[t, n] C[n, k] * clip_pass(x)[t, k]
      dW[n, k] = sum_t dY[t, n] x_hat[t, k]      for EVERY (n, k), pruned or not

    Returned in float64 (the real values), with elementwise bounds for an
    fp32 evaluation whose products are exact and whose L-term sums are
    accumulated in fp32 in any order: |fp32 result - real| <= bound, from
    |sum error| <= (L - 1) u sum|terms| plus one rounding of the result
    (u = 2^-24; dW's sums have 3L terms, x_hat being split exactly into three
    BF16 parts).  Masked dX entries are exactly 0."""
    c = np.asarray(codes, dtype=np.float64)
    dy = bf16_to_f32(np.asarray(dy_bits, dtype=np.uint16)).astype(np.float64)
    if not np.all(np.isfinite(dy)):
        raise ValueError("non-finite gradient")
    if dy.shape[1] != c.shape[0]:
        raise ValueError("n_out mismatch")
    b = float(beta_eff(beta))
    n_out, t = c.shape[0], dy.shape[0]
    s = dy @ c                                          # [m_tok][k]
    s_abs = np.abs(dy) @ np.abs(c)
    mask = clip_pass(x, gamma) if clip else np.ones_like(s)
    dx = b * s * mask
    dx_bound = (n_out + 1) * FP32_UNIT * b * s_abs * mask
    xh = dequant_acts(q, gamma).astype(np.float64)
    dw = dy.T @ xh                                      # [n_out][k]
    dw_bound = (3 * t + 2) * FP32_UNIT * (np.abs(dy).T @ np.abs(xh))
    return dict(dx=dx, dx_bound=dx_bound, dw=dw, dw_bound=dw_bound, clip=mask)


def forward(bits: np.ndarray, x: np.ndarray, n: int, m: int):
    """The whole path for one matrix: returns a dict of every intermediate."""
    beta, keep, codes = quant_weights(bits, n, m)
    q, gamma = quant_acts(x)
    acc, y = linear(codes, q, beta, gamma)
    return dict(beta=beta, keep=keep, codes=codes, q=q, gamma=gamma, acc=acc, y=y)
