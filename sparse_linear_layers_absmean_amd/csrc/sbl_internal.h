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

// Workspace of the exact beta reduction, in 64-bit words.
//   [0, 256)  per-exponent sums of BF16 significands (values outside the
//             fast window), exact integers
//   256, 257  fast-window sum in units of 2^-38: low word, carry count
//   258       number of finished workgroups (last one computes beta)
constexpr int kWsBins = 0;
constexpr int kWsFastLo = 256;
constexpr int kWsFastHi = 257;
constexpr int kWsCount = 258;
constexpr int kWsWords = 260;
constexpr int64_t kWorkspaceBytes = 4096;

// Weights handled by one thread of the mask/pack kernels (one 128-byte BF16 chunk).
constexpr int kChunk = 64;

hipError_t launch_workspace_init(uint64_t* ws, hipStream_t s);

hipError_t launch_beta(const uint16_t* w, int64_t total, uint64_t* ws, float* beta,
                       hipStream_t s);

hipError_t launch_mask_pack(const uint16_t* w, int64_t total, int n, int m, const float* beta,
                            uint8_t* mask, int8_t* codes, int fmt, uint8_t* packed,
                            uint8_t* meta, hipStream_t s);

hipError_t launch_pack(const int8_t* codes, const uint8_t* mask, int64_t total, int n, int m,
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

// any shape, any n:m (one wave per 16 rows x 16 tokens)
hipError_t launch_linear_generic(const LinearArgs& a, int fmt, int n, int m, hipStream_t s);

// up to 8 products with m_tok > kGemvMaxTokens in one launch, DENSE2 (kind 0),
// N:M 6:8 (kind 1) or 2:4 (kind 2)
hipError_t launch_gemm_group(const LinearArgs* items, int count, int kind, hipStream_t s);

// whether the GEMM's 32-bit buffer offsets cover this product
bool gemm_fits(const LinearArgs& a, int kind);

}  // namespace sbl
