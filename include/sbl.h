/*
 * sbl.h -- C ABI of the Sparse-BitLinear (W1.58A8, N:M) forward path for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (BitNet b1.58 with N:M semi-structured sparsity, "Sparse-BitNet"):
 *   beta  = mean |w| over the BF16 master matrix            (absmean scale)
 *   c     = RoundClip(w / max(beta, 1e-5), -1, 1)           (ternary codes)
 *   keep  = top-n of every m consecutive |w| along k, from the BF16 master,
 *           ties to the lower index; codes are masked after quantization
 *   q     = clamp(rint(128 x / max(gamma, 1e-5)), -127, 127),
 *           gamma = max_k |x| per token                    (int8 activations)
 *   acc   = sum_k c[n,k] q[t,k]                             (int32, exact)
 *   y     = acc * (max(beta,1e-5) * max(gamma,1e-5) / 128)  (fp32, no bias)
 * Sources: the Sparse-BitNet paper summaries (gist.science, Spanish and
 * Arabic), section 2 "Methodology" (Sparse-BitLinear: ternary quantization
 * with an absmean scale, dynamic N:M masking from the BF16 master weights,
 * quant-then-mask order, metadata for the hardware kernel); the bitnet.cpp
 * article (unite.ai), "Fundamento matematico" items 2 (activation
 * quantization) and 3 (BitLinear operation); the BitNet project page
 * (aibars.net), "Especificaciones Tecnicas" (W1.58A8, no bias).
 *
 * Conventions for every call:
 *  - Every array pointer is a DEVICE pointer owned by the caller (for example
 *    a PyTorch tensor's data_ptr()).  The library never allocates, frees or
 *    retains caller memory and keeps no mutable global state, so concurrent
 *    calls on different streams are safe.
 *  - Arrays are dense, row-major, 16-byte aligned (scalars: 4-byte aligned).
 *  - Outputs must not alias inputs.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; nothing is read back to the host.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is enqueued and the status is returned.  A failed launch
 *    returns SBL_ERR_LAUNCH and sbl_last_hip_error() (per thread) gives the
 *    HIP error code.  No exception, abort or exit crosses this boundary.
 *  - Non-finite inputs (Inf/NaN) are a precondition violation: results are
 *    unspecified but every kernel still terminates and stays in bounds.
 *  - Shape limits: 64 <= k <= 131072 and k % 64 == 0 (so 127*k < 2^24 and
 *    fp32(acc) is exact); m in {4, 8}; 1 <= n <= m; n_out*k <= 2^34.
 *
 * Byte formats (our own; the pages only say the kernel receives N:M
 * "metadata").  The content of one row:
 *  DENSE2  k/4 bytes, 2 bits per weight holding u = c + 1 in {0,1,2} (3 is
 *          never written).  Weight kk lives in row byte 4*(kk/16) + kk%4, at
 *          bit offset 2*((kk/4)%4): in every 16-weight little-endian word,
 *          (word >> 2s) & 0x03030303 gives the u of weights 4s..4s+3 in byte
 *          order, i.e. an int8 MFMA operand in natural k order after 7 VALU
 *          ops per 16 weights.
 *  BITMAP  k/8 bytes: row byte kk/8, bit kk%8 = 1 when weight kk is kept.
 *          Serves as the mask output and as the N:M metadata.
 *  NM      k*n/(4m) bytes: the kept positions of the row, in ascending k, are
 *          numbered i = 0 .. k*n/m - 1; row byte i/4, bits 2*(i%4)..+1 hold
 *          u = c + 1.  Always used together with its BITMAP metadata.
 * Storage order.  The mask output (mask_bits) and the int8 codes are
 * row-major: [n_out][k/8] and [n_out][k].  The packed stream (`packed`) and
 * the N:M metadata (`meta`) are PANEL-MAJOR: each row's content is a
 * sequence of 64-weight blocks of b bytes (DENSE2 16, NM 16*n/m, BITMAP 8);
 * the k axis is cut into panels of 4 blocks (256 weights), and panel p holds,
 * row after row, the bytes of blocks 4p .. 4p+3 of every row (the last panel
 * holds fewer when k % 256 != 0).  Block kb of row r therefore starts at
 *   (kb/4) * 4*b*n_out  +  r * nb * b  +  (kb%4) * b,
 * where nb is the number of blocks in panel kb/4.  A 16-row decode tile then
 * reads one contiguous run per panel, and a launch sweeps memory in address
 * order.  Sizes are unchanged: sbl_packed_bytes and sbl_meta_bytes.
 */
#ifndef SBL_H
#define SBL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SBL_ABI_VERSION 11

typedef enum {
  SBL_OK = 0,
  SBL_ERR_NULL = 1,        /* a required pointer is NULL                      */
  SBL_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
  SBL_ERR_ALIGN = 3,       /* a pointer is not aligned as required            */
  SBL_ERR_UNSUPPORTED = 4, /* unsupported n:m pattern or format               */
  SBL_ERR_LAUNCH = 5,      /* a HIP launch failed; see sbl_last_hip_error()   */
  SBL_ERR_WORKSPACE = 6    /* workspace missing or smaller than required      */
} sbl_status;

typedef enum {
  SBL_FMT_DENSE2 = 0,      /* 2-bit dense codes, no metadata                  */
  SBL_FMT_NM = 1           /* kept codes only (2 bits each) + BITMAP metadata */
} sbl_format;

typedef void* sbl_stream;  /* a hipStream_t */

/* ABI version of the loaded library (SBL_ABI_VERSION). */
int sbl_abi_version(void);

/* Static text for a status code. */
const char* sbl_status_string(int status);

/* HIP error code of this thread's last SBL_ERR_LAUNCH (0 if none). */
int sbl_last_hip_error(void);

/* Bytes of packed codes for an n_out x k matrix in `fmt` (DENSE2 ignores n, m).
 * Returns -1 for invalid arguments. */
int64_t sbl_packed_bytes(int64_t n_out, int64_t k, int32_t n, int32_t m, int32_t fmt);

/* Bytes of metadata: 0 for DENSE2, n_out*k/8 (the BITMAP) for NM; -1 if invalid. */
int64_t sbl_meta_bytes(int64_t n_out, int64_t k, int32_t fmt);

/* Bytes of device workspace sbl_quant_weights needs for an n_out x k matrix
 * (the exact beta reduction: per workgroup of its first pass an 8-byte
 * partial sum and a 48-byte exact sum of out-of-range magnitudes, rounded up
 * to 4 KB; 56 KB or less up to 2^31 values, 224 KB at 2^34).  Returns -1 for
 * invalid arguments. */
int64_t sbl_workspace_bytes(int64_t n_out, int64_t k);

/* Zero-fill a workspace of `workspace_bytes` bytes (a multiple of 8),
 * enqueued on `stream`.  Optional: every sbl_quant_weights call writes the
 * workspace words it reads, so a workspace carries no state from one call to
 * the next and needs no initialization. */
int sbl_workspace_init(void* workspace, int64_t workspace_bytes, sbl_stream stream);

/* Weight preparation: beta, N:M mask, ternary codes, packing -- one pass of
 * the per-training-step recompute (mask recomputed from the current BF16
 * masters; Sparse-BitNet "dynamic mask recomputation").
 *   w_bf16     [n_out][k] BF16 bit patterns (input).
 *   n, m       the N:M pattern: keep n of every m along k (n == m: no mask).
 *   beta       [1] fp32 output: RN_fp32 of the exact mean of |w| over all
 *              n_out*k values (pruned ones included).  The codes use
 *              max(beta, 1e-5).
 *   mask_bits  [n_out][k/8] BITMAP output, or NULL.
 *   codes      [n_out][k] int8 output in {-1,0,1} (already masked), or NULL.
 *   fmt        format of `packed`.
 *   packed     packed codes output (sbl_packed_bytes), or NULL.
 *   meta       BITMAP metadata output, panel-major, for fmt == SBL_FMT_NM
 *              (required there when packed != NULL); ignored for DENSE2.
 *   The outputs mask_bits, codes, packed and (NM) meta must not share
 *   any byte (SBL_ERR_SHAPE).
 *   workspace  device scratch of at least sbl_workspace_bytes(n_out, k)
 *              bytes, 16-byte aligned, any contents.  Calls sharing one
 *              workspace must be ordered on one stream.
 */
int sbl_quant_weights(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                      float* beta, uint8_t* mask_bits, int8_t* codes,
                      int32_t fmt, uint8_t* packed, uint8_t* meta,
                      void* workspace, int64_t workspace_bytes, sbl_stream stream);

/* One matrix of a grouped weight preparation (the arguments of one
 * sbl_quant_weights call). */
typedef struct {
  const uint16_t* w_bf16;
  int64_t n_out, k;
  float* beta;
  uint8_t* mask_bits;      /* nullable                                       */
  int8_t* codes;           /* nullable                                       */
  uint8_t* packed;         /* nullable                                       */
  uint8_t* meta;           /* NM with packed != NULL: required               */
  void* workspace;         /* sbl_workspace_bytes(n_out, k) bytes, its own   */
  int64_t workspace_bytes;
} sbl_quant_item;

/* Weight preparation of several matrices (e.g. the seven of one transformer
 * block) in two launches per 8 matrices instead of two per matrix, or in one
 * when the 8 (or fewer) matrices fit on the chip at once (about 33M weights
 * on MI355X; patterns dropping at most 2 of a group).  The one-launch path
 * keeps the masters in registers while beta is completed, so it reads them
 * once instead of twice.
 * `items` is a HOST array of `count` (1..256) descriptors sharing the pattern
 * n:m and `fmt`; each is validated as sbl_quant_weights validates its
 * arguments, and workspaces must not overlap (SBL_ERR_WORKSPACE), all before
 * anything is enqueued.  Results are bit-identical to calling
 * sbl_quant_weights on each item. */
int sbl_quant_weights_batch(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                            int32_t fmt, sbl_stream stream);

/* The pages' weight-preparation ablations (Sparse-BitNet summary, Spanish,
 * section 3 "Contribuciones Clave", item 3: the training-design analysis,
 * which finds masks from the continuous masters and the quant-then-mask order
 * better than the alternatives).  Flags of sbl_quant_weights_batch_ex:
 *   SBL_QW_DEFAULT          the method (what sbl_quant_weights_batch does).
 *   SBL_QW_BETA_KEPT        mask-then-quant: the n:m mask comes first (from the
 *                           masters, as usual) and beta is the exact mean of
 *                           |w| over the kept weights only (n_out*k*n/m of
 *                           them); the codes use that beta.
 *   SBL_QW_MASK_FROM_CODES  the mask keeps the n largest |code| of every group
 *                           (codes from beta over every weight; equal |code|
 *                           goes to the lower index) instead of the n largest
 *                           master magnitudes.
 * The two are exclusive.  Outputs and formats are those of
 * sbl_quant_weights_batch.  The variants run slower kernels (per-key
 * selection) than the method's own path, always in two launches.
 * Two more bits select how the method itself runs (same results, bit for bit):
 *   SBL_QW_TWO_PASS         always the two-launch path.
 *   SBL_QW_NO_WAIT          one-launch path: no workgroup waits for another's
 *                           partial sum; each computes the ones not yet there
 *                           from the masters (the fallback that bounds every
 *                           wait, forced; for testing).
 * Unknown bits, or BETA_KEPT with MASK_FROM_CODES, give SBL_ERR_UNSUPPORTED
 * before anything is checked or enqueued. */
enum {
  SBL_QW_DEFAULT = 0,
  SBL_QW_BETA_KEPT = 1,
  SBL_QW_MASK_FROM_CODES = 2,
  SBL_QW_TWO_PASS = 4,
  SBL_QW_NO_WAIT = 8
};
int sbl_quant_weights_batch_ex(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                               int32_t fmt, int32_t flags, sbl_stream stream);

/* Allocation-free weight preparation, for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): sbl_quant_weights_batch with the
 * exact-beta scratch taken from a fixed array inside the library instead of
 * the items' workspaces, whose workspace and workspace_bytes fields are
 * ignored.
 *  - The array holds SBL_NOALLOC_SCRATCH_BYTES (4 MiB) on every GPU the
 *    library runs on, until the process ends.  Item i takes
 *    sbl_workspace_bytes(n_out, k) of it, rounded up to 256 bytes; a batch
 *    needing more in all returns SBL_ERR_WORKSPACE before anything is
 *    enqueued (73 items of up to 2^31 weights each always fit).
 *  - The array of the CURRENT device is used; `stream` must belong to it.
 *    The first call on a device looks up the array's address once; no call
 *    allocates or frees memory.
 *  - Every call on one GPU shares that GPU's array: calls that can overlap
 *    on one GPU (different streams or threads without ordering) race and
 *    give undefined results.  Order them, e.g. on one stream.
 *  - Nothing in the array has to start at zero, and it needs no clearing
 *    between calls: a call reads only words it writes itself, plus one
 *    generation word per item whose starting value does not matter.
 * Validation and errors as sbl_quant_weights_batch; results are
 * bit-identical to it. */
#define SBL_NOALLOC_SCRATCH_BYTES (4 << 20)
int sbl_quant_weights_batch_noalloc(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                                    int32_t fmt, sbl_stream stream);

/* Packing alone: ternary codes (+ mask) -> packed bytes.
 *   codes      [n_out][k] int8 in {-1,0,1} (other values: unspecified bytes).
 *   mask_bits  [n_out][k/8] BITMAP; required for NM, ignored for DENSE2.
 *              NM takes, per group, the codes of the first n kept positions
 *              in ascending k; a group with fewer than n kept bits is padded
 *              with code 0.
 *   packed     output (sbl_packed_bytes), panel-major.
 *   meta       NM only: receives mask_bits in panel-major order, or NULL to skip.
 */
int sbl_pack(const int8_t* codes, const uint8_t* mask_bits, int64_t n_out, int64_t k,
             int32_t n, int32_t m, int32_t fmt, uint8_t* packed, uint8_t* meta,
             sbl_stream stream);

/* Per-token absmax int8 activation quantization.
 *   x      [m_tok][k] fp32 input.
 *   xq     [m_tok][k] int8 output: clamp(rint(x / (max(gamma,1e-5)/128)), -127, 127),
 *          one correctly rounded fp32 division, rint half to even.
 *   gamma  [m_tok] fp32 output: max_k |x[t,k]| (exact).
 * m_tok == 0 is a no-op.
 */
int sbl_quant_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                   sbl_stream stream);

/* Ternary x int8 product with fp32 rescale; no bias.
 *   packed, meta  weights in `fmt` (meta: BITMAP for NM, NULL for DENSE2);
 *                 n, m must be those the weights were packed with.
 *   beta          [1] fp32 (as produced by sbl_quant_weights).
 *   xq, gamma     [m_tok][k] int8 and [m_tok] fp32 (as produced by sbl_quant_acts).
 *   y             [m_tok][n_out] fp32 output:
 *                 RN(fp32(acc) * RN(RN(max(beta,1e-5) * max(gamma,1e-5)) * 2^-7)).
 *   acc           [m_tok][n_out] int32 output (exact sum), or NULL.
 * Decode sizes (m_tok <= 16) run a bandwidth-bound GEMV, larger ones an
 * int8-MFMA GEMM; both give identical bits.  Products whose buffers are too
 * large for those kernels' 32-bit buffer offsets (2 GiB, the last tile's
 * overhang included, e.g. (m_tok + 256) * n_out * 4 bytes of y for the GEMM)
 * run a generic kernel instead: the same bits, more slowly.  m_tok == 0 is
 * a no-op.
 */
int sbl_linear(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
               const float* beta, const int8_t* xq, const float* gamma,
               int64_t m_tok, int64_t n_out, int64_t k, float* y, int32_t* acc,
               sbl_stream stream);

/* One product of a batch (the arguments of one sbl_linear call). */
typedef struct {
  const uint8_t* packed;
  const uint8_t* meta;     /* NM: BITMAP metadata; DENSE2: NULL              */
  const float* beta;
  const int8_t* xq;
  const float* gamma;
  int64_t m_tok, n_out, k;
  float* y;
  int32_t* acc;            /* nullable                                       */
} sbl_linear_item;

/* Several independent products (e.g. the q, k, v projections of one block)
 * in as few launches as possible: decode-sized items (m_tok <= 16) share one
 * bandwidth-bound GEMV launch per 8 items; larger ones each run the GEMM.
 * `items` is a HOST array of `count` (1..256) descriptors, all in format
 * `fmt` with pattern n:m; every item is validated as sbl_linear validates
 * its arguments before anything is enqueued.  Results are bit-identical to
 * calling sbl_linear on each item. */
int sbl_linear_batch(const sbl_linear_item* items, int32_t count, int32_t fmt, int32_t n,
                     int32_t m, sbl_stream stream);

/* Activation quantization and the products that consume it, in one call: the
 * layer input x is quantized exactly as sbl_quant_acts does (bitnet.cpp
 * article, "Fundamento matematico", item 2) and every item's product is
 * computed from it as sbl_linear_batch does (item 3).  Typical use: the q, k
 * and v projections of one input.
 *   x          [m_tok][k] fp32 input shared by every item.
 *   xq, gamma  [m_tok][k] int8 and [m_tok] fp32 OUTPUTS (required), written
 *              as sbl_quant_acts writes them.
 *   items      1..256 products; each must have this m_tok and k; their xq
 *              and gamma fields are ignored (the call uses its own).
 * For decode-sized inputs (m_tok <= 16, at most 8 items, m_tok * k <= 16384
 * values) a single launch quantizes inside the product's workgroups; otherwise
 * the call runs sbl_quant_acts and then sbl_linear_batch.  Validation as those two calls; results (xq, gamma, y,
 * acc) are bit-identical to them. */
int sbl_linear_acts_batch(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                          const sbl_linear_item* items, int32_t count, int32_t fmt, int32_t n, int32_t m,
                          sbl_stream stream);

/* Group scales (BitNet.cpp article, "Cuantizacion y normalizacion de
 * grupos": parameters computed per group instead of per matrix, so groups
 * need no communication).  A group is a block of rows_per_group consecutive
 * output rows (the last may be shorter); G = ceil(n_out / rows_per_group).
 *
 * Workspace bytes for sbl_quant_weights_grouped (-1 if invalid). */
int64_t sbl_workspace_bytes_grouped(int64_t n_out, int64_t k, int64_t rows_per_group);

/* sbl_quant_weights with one beta per row group: beta[g] = RN_fp32 of the
 * exact mean of |w| over group g's rows, and row r's codes use
 * max(beta[r / rows_per_group], 1e-5).  The mask does not depend on beta.
 *   beta       [G] fp32 output.
 *   workspace  sbl_workspace_bytes_grouped(n_out, k, rows_per_group) bytes.
 * Everything else (outputs, formats, validation, errors) as
 * sbl_quant_weights; rows_per_group < 1 or more than 65535 groups gives
 * SBL_ERR_SHAPE, and beta must not overlap the other buffers.
 * rows_per_group = 1: one beta per row. */
int sbl_quant_weights_grouped(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                              int64_t rows_per_group, float* beta, uint8_t* mask_bits, int8_t* codes,
                              int32_t fmt, uint8_t* packed, uint8_t* meta,
                              void* workspace, int64_t workspace_bytes, sbl_stream stream);

/* sbl_linear with one beta per row group:
 *   y[t][r] = RN(fp32(acc[t][r]) * RN(RN(beta_eff[r / rows_per_group] *
 *             gamma_eff[t]) * 2^-7)).
 *   beta       [ceil(n_out / rows_per_group)] fp32 (sbl_quant_weights_grouped).
 *   acc        [m_tok][n_out] int32, nullable (the exact products).
 * The same kernels as sbl_linear, whose epilogues read beta per row.
 * Validation as sbl_linear; rows_per_group < 1 gives SBL_ERR_SHAPE, and y
 * and acc must not overlap beta. */
int sbl_linear_grouped(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                       const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma,
                       int64_t m_tok, int64_t n_out, int64_t k, float* y, int32_t* acc, sbl_stream stream);

/* Activation groups along k (the same article and section): one gamma per
 * token and block of kg consecutive features (kg a multiple of 64 dividing
 * k; k / kg <= 65535, m_tok <= 65535).
 *   gamma      [m_tok][k / kg] fp32 output: gamma[t][j] = max |x| over block j.
 *   xq         [m_tok][k] int8 output: each feature quantized as
 *              sbl_quant_acts does, with its block's gamma.
 * Alignment 4 bytes for x and gamma; buffers must not overlap. */
int sbl_quant_acts_kgrouped(const float* x, int64_t m_tok, int64_t k, int64_t kg, int8_t* xq, float* gamma,
                            sbl_stream stream);

/* Products with activation groups (and beta per row group; rows_per_group
 * >= n_out for one beta per matrix):
 *   y[t][r] = sum over blocks j, in ascending order, in fp32, of
 *             RN(fp32(acc_j[t][r]) * RN(RN(beta_eff[r / rows_per_group] *
 *             gamma_eff[t][j]) * 2^-7)),  acc_j = the exact product of block j.
 * xq and gamma from sbl_quant_acts_kgrouped with the same kg.  Validation as
 * sbl_linear.  A decode kernel: one wave per output row and token, 4 rows
 * per workgroup (the weights are read again for every token; no matrix
 * cores). */
int sbl_linear_kgrouped(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                        const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t kg,
                        int64_t m_tok, int64_t n_out, int64_t k, float* y, sbl_stream stream);

/* Block scales (the same article and section, the weight groups taken
 * along k as well): one beta per block of rows_per_group consecutive output
 * rows x cols_per_group consecutive features (cols_per_group a multiple of 64
 * dividing k; rows_per_group >= 1, the last row block may be shorter; at
 * most 65535 row blocks and 65535 column blocks).
 *   beta[gr][gc] = RN_fp32 of the exact mean of |w| over block (gr, gc); the
 *   codes of the block use max(beta[gr][gc], 1e-5).  The mask does not
 *   depend on beta.
 *   beta       [ceil(n_out / rows_per_group)][k / cols_per_group] fp32 output.
 *   workspace  sbl_workspace_bytes_blocked(n_out, k, rows_per_group,
 *              cols_per_group) bytes (-1: invalid shape).
 * Everything else as sbl_quant_weights_grouped; cols_per_group = k is
 * sbl_quant_weights_grouped. */
int64_t sbl_workspace_bytes_blocked(int64_t n_out, int64_t k, int64_t rows_per_group, int64_t cols_per_group);
int sbl_quant_weights_blocked(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                              int64_t rows_per_group, int64_t cols_per_group, float* beta, uint8_t* mask_bits,
                              int8_t* codes, int32_t fmt, uint8_t* packed, uint8_t* meta,
                              void* workspace, int64_t workspace_bytes, sbl_stream stream);

/* Products with block scales: as sbl_linear_kgrouped, with beta
 * [ceil(n_out / rows_per_group)][k / kg] from sbl_quant_weights_blocked with
 * cols_per_group = kg, so that every feature block j of the activations is
 * one column block of the weights:
 *   y[t][r] = sum over j, ascending, in fp32, of RN(fp32(acc_j[t][r]) *
 *             RN(RN(beta_eff[r / rows_per_group][j] * gamma_eff[t][j]) * 2^-7)).
 * beta must not overlap y. */
int sbl_linear_blocked(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                       const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t kg,
                       int64_t m_tok, int64_t n_out, int64_t k, float* y, sbl_stream stream);

/* Backward of the layer under the dual straight-through estimator
 * (Sparse-BitNet summaries: Spanish section 2, "Estrategia de Entrenamiento",
 * Dual STE; Arabic section 2, item 3): the quantizers pass the gradient as
 * the identity inside their clipping range, and the mask passes it densely
 * to every master weight, the pruned ones included.  beta and gamma are
 * treated as constants.
 *   dy_bf16     [m_tok][n_out] BF16 bit patterns: the gradient of y.
 *   packed, meta, fmt, n, m, beta
 *               the layer's packed weights and scale, as given to sbl_linear
 *               (used for dx; N:M metadata must keep exactly n per group,
 *               as sbl_quant_weights writes it).
 *   x           [m_tok][k] fp32: the layer input (used for dx: the clip mask).
 *   xq, gamma   [m_tok][k] int8 and [m_tok] fp32 from sbl_quant_acts(x)
 *               (gamma for both outputs, xq for dw).
 *   dx          [m_tok][k] fp32 output, or NULL:
 *                 dx = RN(beta_eff * sum_n dy[t][n] c[n][k]) where
 *                 |rint(128 x[t][k] / gamma_eff[t])| <= 127 (evaluated as
 *                 in sbl_quant_acts), else 0.
 *   dw          [n_out][k] fp32 output, or NULL:
 *                 dw = sum_t dy[t][n] x_hat[t][k] for EVERY (n, k), with
 *                 x_hat = RN_fp32(gamma_eff[t] * xq[t][k]) * 2^-7.
 * Products are exact and sums are accumulated in fp32, in an unspecified
 * order (error at most (L + 1) * 2^-24 * sum|terms| for L terms; dw's sums
 * have 3 m_tok terms, x_hat being split exactly into three BF16 parts).
 * Requires m_tok >= 1, n_out % 8 == 0 (SBL_ERR_SHAPE), k % 64 == 0;
 * alignment 16 bytes for dy_bf16, packed, meta and xq, 4 for the rest;
 * outputs must not overlap each other or any input (SBL_ERR_SHAPE).  With
 * both outputs NULL the call does nothing. */
int sbl_linear_backward(const uint16_t* dy_bf16, int64_t m_tok, int64_t n_out, int64_t k,
                        const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                        const float* beta, const float* x, const int8_t* xq, const float* gamma,
                        float* dx, float* dw, sbl_stream stream);

/* Bytes of device scratch that sbl_linear_backward_ws needs at these sizes
 * (for both outputs), or -1 for sizes sbl_linear_backward rejects.  It holds
 * the codes transposed as BF16 (k x n_out, n_out rounded up to 64), dy
 * transposed (n_out x m_tok, both rounded up to 64) and the three BF16 parts
 * of x_hat transposed (3 x k x m_tok): about 2 k n_out + 2 n_out m_tok +
 * 6 k m_tok bytes. */
int64_t sbl_backward_workspace_bytes(int64_t m_tok, int64_t n_out, int64_t k);

/* sbl_linear_backward (the same operation, results within the same bounds;
 * the same argument checks and status codes) with a caller workspace: the
 * ternary codes are decoded and the operands transposed once per call into
 * `workspace`, so that both gradients run as plain BF16 contractions.
 *   workspace        device memory, 256-byte aligned (SBL_ERR_ALIGN), owned by
 *                    the caller, of workspace_bytes >=
 *                    sbl_backward_workspace_bytes(m_tok, n_out, k) bytes
 *                    (else SBL_ERR_SHAPE); NULL: SBL_ERR_NULL.  Its contents
 *                    need no initialisation and are scratch after the call;
 *                    it must not overlap any input or output (SBL_ERR_SHAPE),
 *                    and calls in flight at the same time need their own.
 * Rows longer than 2^22 values (n_out or m_tok rounded up to 64) take the
 * kernels of sbl_linear_backward and leave the workspace unused. */
int sbl_linear_backward_ws(const uint16_t* dy_bf16, int64_t m_tok, int64_t n_out, int64_t k,
                           const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                           const float* beta, const float* x, const int8_t* xq, const float* gamma,
                           float* dx, float* dw, void* workspace, int64_t workspace_bytes, sbl_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* SBL_H */
