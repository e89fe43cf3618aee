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

// Workspace of the exact beta reduction of one matrix, in 64-bit words.
//   [0, 256)       per-exponent sums of BF16 significands (values outside the
//                  fast window), exact integers; accumulated with atomics by
//                  the partial-sum kernel, read and zero-filled again by the
//                  finalize kernel (so it must be zero before the first use)
//   [256, 256+nb)  one fast-window partial sum per workgroup of the partial-sum
//                  kernel (units of 2^-38), overwritten by every call
constexpr int kWsBins = 0;
constexpr int kWsSlots = 256;

// Partition of the absmean pass over a matrix of `total` BF16 values: nb
// workgroups of kAbsThreads threads, vpt 16-byte vectors per thread.  A thread
// adds at most 2^14 fast-window values (vpt <= 2048), which keeps its fp64
// partial sums exact.
constexpr int kAbsThreads = 256;
struct AbsmeanPlan {
  int64_t nb, vpt;
};
inline AbsmeanPlan absmean_plan(int64_t total) {
  const int64_t nvec = total / 8;
  const int64_t per_wg = (int64_t)kAbsThreads * 8;
  AbsmeanPlan p{(nvec + per_wg - 1) / per_wg, 8};
  if (p.nb > 1024) {          // big matrices: longer threads, at most 1024 slots (4096 at 2^34)
    p.vpt = (nvec + 1024 * kAbsThreads - 1) / (1024 * kAbsThreads);
    p.vpt = (p.vpt + 7) / 8 * 8;                        // whole batches of 8 loads
    if (p.vpt > 2048) p.vpt = 2048;
    p.nb = (nvec + kAbsThreads * p.vpt - 1) / (kAbsThreads * p.vpt);
  }
  if (p.nb < 1) p.nb = 1;
  return p;
}
inline int64_t workspace_bytes_for(int64_t total) {
  const int64_t bytes = 8 * (kWsSlots + absmean_plan(total).nb);
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
  int64_t nb, vpt;        // absmean partition (AbsmeanPlan)
  float* beta;
  uint64_t* ws;
  uint8_t* mask;          // nullable outputs
  int8_t* codes;
  uint8_t* packed;
  uint8_t* meta;
  int64_t n_out;          // rows; k / 64 blocks per row (panel layout of packed, meta)
  int32_t nkb;
  int32_t fmt;            // format of `packed`
};
constexpr int kMaxQDesc = 8;
struct QBatch {
  QDesc d[kMaxQDesc];
  int64_t start[kMaxQDesc + 1];   // first workgroup of each item in the current launch
  int32_t count;
};

// The three launches of weight preparation, in stream order.  Each fills
// batch.start for its own grid.
hipError_t launch_absmean_partial(QBatch& batch, hipStream_t s);
hipError_t launch_absmean_final(QBatch& batch, hipStream_t s);
hipError_t launch_mask_pack(QBatch& batch, int n, int m, hipStream_t s);

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

}  // namespace sbl
