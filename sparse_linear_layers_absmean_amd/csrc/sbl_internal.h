// Internal declarations shared by the HIP translation units of libsbl.
// Not part of the public ABI (that is include/sbl.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: nontemporal hint)
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Buffer resource over `bytes` (< 2^32) bytes at p: raw buffer loads past the
// end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Workspace of the exact beta reduction of one matrix, in 64-bit words
// (written by the absmean pass of every call, read after it; no state is
// carried from one call to the next):
//   [0, nb)           fast-window partial sum of absmean workgroup i (units of
//                     2^-38); bit 63 set when the workgroup also met values
//                     outside the window
//   [lb + 6i, +6)     lb = nb rounded up to 8: for a flagged workgroup i, the
//                     exact sum of its out-of-window magnitudes as 12
//                     little-endian 32-bit limbs (units of 2^-133); not
//                     written for other workgroups
__host__ __device__ __forceinline__ int64_t ws_limb_base(int64_t nb) { return (nb + 7) / 8 * 8; }
constexpr int kWsLimbWords = 6;
// The one-launch (resident) weight preparation uses the same two regions for
// its nb slots, then one generation word and nb slot tags (a slot is
// complete for a call when its tag is that call's; k_maskpack.hip):
__host__ __device__ __forceinline__ int64_t ws_res_gen(int64_t nb) { return ws_limb_base(nb) + kWsLimbWords * nb; }
__host__ __device__ __forceinline__ int64_t ws_res_words(int64_t nb) { return ws_res_gen(nb) + 1 + nb; }
// Its workgroups of 256 threads hold at most 2 chunks of 64 weights per thread.
constexpr int kResChunksPerThread = 2;
constexpr int64_t kResChunksPerWg = 256 * kResChunksPerThread;

// Partition of the absmean pass over a matrix of `total` BF16 values: nb
// workgroups of kAbsThreads threads, vpt 16-byte vectors per thread.  A thread
// adds at most 2^14 fast-window values (vpt <= 2048), which keeps its fp64
// partial sums exact.
constexpr int kAbsThreads = 256;
constexpr int kAbsMinVpt = 8;      // one batch of 8 loads per thread at least
constexpr int kAbsMaxSlots = 1024; // partial sums per matrix while vpt <= 2048
struct AbsmeanPlan {
  int64_t nb, vpt;
};
inline AbsmeanPlan absmean_plan(int64_t total) {
  const int64_t nvec = total / 8;
  const int64_t per_wg = (int64_t)kAbsThreads * kAbsMinVpt;
  AbsmeanPlan p{(nvec + per_wg - 1) / per_wg, kAbsMinVpt};
  if (p.nb > kAbsMaxSlots) {  // big matrices: longer threads, at most 1024 slots (4096 at 2^34)
    p.vpt = (nvec + kAbsMaxSlots * kAbsThreads - 1) / (kAbsMaxSlots * kAbsThreads);
    p.vpt = (p.vpt + 7) / 8 * 8;                        // whole batches of 8 loads
    if (p.vpt > 2048) p.vpt = 2048;
    p.nb = (nvec + kAbsThreads * p.vpt - 1) / (kAbsThreads * p.vpt);
  }
  if (p.nb < 1) p.nb = 1;
  return p;
}
inline int64_t workspace_bytes_for(int64_t total) {
  const int64_t nb = absmean_plan(total).nb;
  const int64_t bytes = 8 * (ws_limb_base(nb) + kWsLimbWords * nb);
  return (bytes + 4095) / 4096 * 4096;
}

// Weights handled by one thread of the mask/pack kernels (one 128-byte BF16 chunk).
constexpr int kChunk = 64;

// Panel-major storage of a packed stream (DENSE2 or N:M codes, N:M metadata).
// A row's stream is a sequence of 64-weight blocks of `b` bytes each; the k
// axis is cut into panels of kPanelBlocks blocks (256 weights), and panel p
// stores, row after row, the bytes of blocks kPanelBlocks*p ... of every row
// (the last panel may hold fewer blocks).  Byte offset of block kb of `row`:
constexpr int kPanelBlocks = 4;
__host__ __device__ __forceinline__ int64_t panel_offset(int64_t n_out, int64_t nkb, int64_t b, int64_t row,
                                                         int64_t kb) {
  const int64_t p = kb / kPanelBlocks;
  const int64_t nb = nkb - kPanelBlocks * p < kPanelBlocks ? nkb - kPanelBlocks * p : kPanelBlocks;
  return p * kPanelBlocks * b * n_out + row * nb * b + (kb - kPanelBlocks * p) * b;
}

// One matrix of a grouped weight-preparation launch.
struct QDesc {
  const u32x4* w;         // BF16 masters as 16-byte vectors (8 values each)
  int64_t nvec;           // n_out*k/8
  int64_t count;          // values beta averages over: n_out*k, or the kept ones (n_out*k*n/m)
  int64_t nb, vpt;        // absmean partition (AbsmeanPlan); one launch: nb slots of vpt chunks
  float* beta;
  uint64_t* ws;
  int64_t ws_words;       // workspace size
  int64_t beta_rows;      // > 0: group scales, beta[row / beta_rows] (mask/pack kernels, beta complete)
  uint8_t* mask;          // nullable outputs
  int8_t* codes;
  uint8_t* packed;
  uint8_t* meta;
  int64_t n_out;          // rows; k / 64 blocks per row (panel layout of packed, meta)
  int32_t nkb;
  int32_t fmt;            // format of `packed`
  int32_t beta_kblocks;   // group scales: 0 one beta per row group; > 0 per row group and block of
                          // beta_kblocks k-blocks, beta[(row / beta_rows) * (nkb / beta_kblocks) + kb / beta_kblocks]
};

// group scales: index of the beta of chunk c (64 weights: row c / nkb, k-block c % nkb)
__host__ __device__ __forceinline__ int64_t chunk_beta_index(const QDesc& d, int64_t c) {
  const int64_t row = c / d.nkb;
  if (d.beta_kblocks <= 0) return row / d.beta_rows;
  return (row / d.beta_rows) * (d.nkb / d.beta_kblocks) + (c - row * d.nkb) / d.beta_kblocks;
}
constexpr int kMaxQDesc = 8;
struct QBatch {
  QDesc d[kMaxQDesc];
  int64_t start[kMaxQDesc + 1];   // first workgroup of each item in the current launch
  int32_t count;
  int32_t beta_ready;             // mask/pack: beta already in d.beta (else finalized per workgroup)
};

// Weight preparation in stream order: the absmean pass (partial sums), then
// the mask/pack pass.  A mask/pack launch of about one round of workgroups
// finalizes beta at the start of each workgroup; a larger one (and a call
// that wants only beta) is preceded by the one-workgroup-per-matrix finalize
// kernel, and reads beta (batch.beta_ready).  Each fills batch.start for its
// own grid; launch_mask_pack returns its workgroup count in *grid when
// `dry` (nothing launched).
hipError_t launch_absmean_partial(QBatch& batch, hipStream_t s);
// The mask-then-quant variant: only the magnitudes the n:m mask keeps are summed.
hipError_t launch_absmean_partial_kept(QBatch& batch, int n, int m, hipStream_t s);
hipError_t launch_absmean_final(QBatch& batch, hipStream_t s);
// One launch for the whole weight preparation of a batch that fits on the
// chip at once (returns false, launching nothing, when it does not or the
// pattern drops more than two of a group): every thread keeps its masters in
// registers while the partial sums of its matrix are completed.  max_ticks
// bounds the wait for other workgroups' partial sums; the missing ones are
// then computed directly (0: at once).  Fills batch.start and sets d.nb to
// the one-launch partition.
bool launch_resident(QBatch& batch, int n, int m, uint32_t max_ticks, hipStream_t s, hipError_t* err);
// mask_from_codes: the mask keeps the n largest |code| per group (ties to the
// lower index) instead of the n largest master magnitudes.
hipError_t launch_mask_pack(QBatch& batch, int n, int m, hipStream_t s, bool dry = false, int64_t* grid = nullptr,
                            bool mask_from_codes = false);

hipError_t launch_workspace_init(uint64_t* ws, int64_t words, hipStream_t s);

hipError_t launch_pack(const int8_t* codes, const uint8_t* mask, int64_t n_out, int64_t k, int n, int m,
                       int fmt, uint8_t* packed, uint8_t* meta, hipStream_t s);

hipError_t launch_quant_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                             hipStream_t s);

struct LinearArgs {
  const uint8_t* packed;
  const uint8_t* meta;
  const float* beta;
  const int8_t* xq;
  const float* gamma;
  int64_t m_tok, n_out, k;
  float* y;
  int32_t* acc;
  int64_t beta_rows = 0;          // > 0: beta per block of beta_rows output rows, beta[row / beta_rows]
};

// token counts up to this run the grouped GEMV; larger ones the GEMM
constexpr int64_t kGemvMaxTokens = 16;

hipError_t launch_linear_batch(const LinearArgs* items, int count, int fmt, int n, int m,
                               hipStream_t s);

// Activation quantization of x into xq / gamma and the products of every item
// from them (each item: m_tok x k activations, xq / gamma set to these).  For
// decode-sized inputs that fit, one GEMV launch does both.
hipError_t launch_linear_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                              const LinearArgs* items, int count, int fmt, int n, int m, hipStream_t s);

// any shape, any n:m (one wave per 16 rows x 16 tokens)
hipError_t launch_linear_generic(const LinearArgs& a, int fmt, int n, int m, hipStream_t s);

// up to 8 products with m_tok > kGemvMaxTokens in one launch, DENSE2 (kind 0),
// N:M 6:8 (kind 1) or 2:4 (kind 2)
hipError_t launch_gemm_group(const LinearArgs* items, int count, int kind, hipStream_t s);

// whether the GEMM's 32-bit buffer offsets cover this product
bool gemm_fits(const LinearArgs& a, int kind);

// N:M 2:4 products on the sparse MFMA (v_smfmac_i32_16x16x128_i8); called by
// launch_gemm_group for kind 2
hipError_t launch_gemm24_group(const LinearArgs* items, int count, hipStream_t s);

// Group scales (k_grouped.hip): one exact absmean beta per block of
// rows_per_group output rows x cols_per_group features (cols_per_group = k:
// row groups).  Groups are numbered row group first: g = gr * gk + gc.
// Workspace: one region of `region` words per group (the absmean slot
// layout of one group).
struct GroupPlan {
  int64_t groups, nb, vpt, region;   // region: words per group
  int64_t gr, gk;                    // row groups, column groups (groups = gr * gk)
};
inline GroupPlan group_plan(int64_t n_out, int64_t k, int64_t rows_per_group, int64_t cols_per_group) {
  const int64_t rpg = rows_per_group < n_out ? rows_per_group : n_out;
  const AbsmeanPlan p = absmean_plan(rpg * cols_per_group);
  const int64_t gr = (n_out + rpg - 1) / rpg, gk = k / cols_per_group;
  return GroupPlan{gr * gk, p.nb, p.vpt, ws_limb_base(p.nb) + kWsLimbWords * p.nb, gr, gk};
}
// beta[g] for every group (partial sums, then one finalizing workgroup per
// group, or the partial-sum workgroup itself when one holds the group)
hipError_t launch_grouped_beta(const uint16_t* w, int64_t n_out, int64_t k, int64_t rows_per_group,
                               int64_t cols_per_group, float* beta, uint64_t* ws, hipStream_t s);

// Activation groups along k (kg features per gamma; kg % 64 == 0, k % kg == 0)
hipError_t launch_quant_acts_kgrouped(const float* x, int64_t m_tok, int64_t k, int64_t kg, int8_t* xq, float* gamma,
                                      hipStream_t s);
// beta_per_block: beta [row groups][k / kg] (block scales) instead of [row groups]
hipError_t launch_linear_kgrouped(const uint8_t* packed, const uint8_t* meta, int fmt, int n, int m, const float* beta,
                                  int64_t rows_per_group, bool beta_per_block, const int8_t* xq, const float* gamma,
                                  int64_t kg, int64_t m_tok, int64_t n_out, int64_t k, float* y, hipStream_t s);

// Backward of the layer (k_backward.hip): dx and/or dw (each nullable).
struct BackwardArgs {
  const uint16_t* dy;             // [m_tok][n_out] BF16
  int64_t m_tok, n_out, k;        // n_out % 8 == 0, k % 64 == 0
  const uint8_t* packed;          // dx: the layer's packed weights
  const uint8_t* meta;
  int32_t fmt, n, m;
  const float* beta;
  const float* x;                 // dx: the layer input (clip mask)
  const int8_t* xq;               // dw: its int8 codes
  const float* gamma;
  float* dx;                      // [m_tok][k]
  float* dw;                      // [n_out][k]
};
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
// the same gradients through a caller workspace of backward_ws_bytes bytes
int64_t backward_ws_bytes(int64_t m_tok, int64_t n_out, int64_t k);
hipError_t launch_backward_ws(const BackwardArgs& a, void* ws, hipStream_t s);

}  // namespace sbl
