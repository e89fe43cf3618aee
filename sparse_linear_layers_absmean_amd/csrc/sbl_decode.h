// Device helpers shared by the GEMV and GEMM kernels: weight decode into int8
// MFMA operands (DENSE2 word decode, N:M table + v_perm scatter), the rescale,
// and the grouped-launch descriptors.  Included by k_linear.hip and k_gemm.hip.
#pragma once

#include "sbl_internal.h"

namespace sbl {
namespace dec {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

enum Kind { kDense2 = 0, kNm68 = 1, kNm24 = 2 };

__device__ __forceinline__ v4i dense2_quad(uint32_t w) {
  v4i a;
  a[0] = (int32_t)(w & 0x03030303u);
  a[1] = (int32_t)((w >> 2) & 0x03030303u);
  a[2] = (int32_t)((w >> 4) & 0x03030303u);
  a[3] = (int32_t)((w >> 6) & 0x03030303u);
  return a;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ float out_scale_g(const float* beta, float gamma) {
  const float b = fmaxf(beta[0], 1e-5f);
  const float g = fmaxf(gamma, 1e-5f);
  return (b * g) * 0.0078125f;   // RN(RN(beta*gamma) * 2^-7); the power of two is exact
}

__device__ __forceinline__ float out_scale(const float* beta, const float* gamma, int64_t t) {
  return out_scale_g(beta, gamma[t]);
}

// beta of output row `row` (< n_out): one per matrix (beta_rows = 0) or one
// per block of beta_rows consecutive rows (group scales)
__device__ __forceinline__ const float* row_beta(const float* beta, int32_t beta_rows, int64_t row) {
  return beta_rows > 0 ? beta + (uint32_t)row / (uint32_t)beta_rows : beta;
}

// LDS lookup tables of the N:M decode
struct NmLut {
  uint32_t spread[256];   // byte of 4 codes (2 bits each) -> 4 int8 c = u - 1
  uint32_t sel[256][2];   // bitmap byte -> v_perm selectors for 8 output bytes
};

template <int KIND>
__device__ void build_lut(NmLut& L) {
  for (int x = threadIdx.x; x < 256; x += blockDim.x) {
    uint32_t sp = 0;
    for (int i = 0; i < 4; ++i) sp |= ((((uint32_t)x >> (2 * i)) & 3u) - 1u & 0xFFu) << (8 * i);
    L.spread[x] = sp;
    uint32_t s0 = 0, s1 = 0;
    int ra = 0, rb = 0;
    for (int p = 0; p < 8; ++p) {
      uint32_t sel = 0x0Cu;                        // v_perm: constant zero byte
      const bool kept = (x >> p) & 1;
      if (KIND == kNm68) {
        if (kept && ra < 6) sel = (uint32_t)ra++;
      } else {                                     // two 4-groups: codes 0,1 then 2,3
        if (p < 4) { if (kept && ra < 2) sel = (uint32_t)ra++; }
        else { if (kept && rb < 2) sel = (uint32_t)(2 + rb++); }
      }
      if (p < 4) s0 |= sel << (8 * p);
      else s1 |= sel << (8 * (p - 4));
    }
    L.sel[x][0] = s0;
    L.sel[x][1] = s1;
  }
}

struct LinDesc {
  const uint8_t* packed;
  const uint8_t* meta;
  const int8_t* xq;
  const float* gamma;
  const float* beta;
  float* y;
  int32_t* acc;
  int64_t n_out;
  int32_t k;
  int32_t m_tok;
  int32_t tiles_n;        // GEMM: row tiles of this matrix
  int32_t beta_rows;      // > 0: beta per block of beta_rows output rows (group scales)
  // GEMV with the activation quantization fused in: fp32 input, and the
  // quantized activations and scales to publish (nullable; written once)
  const float* x;
  int8_t* xq_out;
  float* gamma_out;
};

inline LinDesc to_desc(const LinearArgs& a) {
  LinDesc d;
  d.packed = a.packed; d.meta = a.meta; d.xq = a.xq; d.gamma = a.gamma; d.beta = a.beta;
  d.y = a.y; d.acc = a.acc; d.n_out = a.n_out; d.k = (int32_t)a.k; d.m_tok = (int32_t)a.m_tok;
  d.tiles_n = 0;
  d.beta_rows = (int32_t)a.beta_rows;
  d.x = nullptr; d.xq_out = nullptr; d.gamma_out = nullptr;
  return d;
}

constexpr int kMaxDesc = 8;
struct LinBatch {
  LinDesc d[kMaxDesc];
  int32_t start[kMaxDesc + 1];
  int32_t count;
};

// Raw A data of one lane for one 64-weight k-block of one tile.
template <int KIND> struct ARaw;
template <> struct ARaw<kDense2> { u32x4 w; };
template <> struct ARaw<kNm68> { uint32_t c[3]; uint32_t m[2]; };
template <> struct ARaw<kNm24> { uint32_t c[2]; uint32_t m[2]; };

template <int KIND>
__device__ __forceinline__ void load_a(ARaw<KIND>& a, const LinDesc& d, int64_t row, int kb, bool ok) {
  const int64_t k = d.k;
  if constexpr (KIND == kDense2) {
    if (ok) a.w = ld16(d.packed + row * (k / 4) + (int64_t)kb * 16);
    else a.w = u32x4{0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};   // u = 1: code 0
  } else if constexpr (KIND == kNm68) {
    if (ok) {
      const uint32_t* c = reinterpret_cast<const uint32_t*>(d.packed + row * (3 * k / 16) + (int64_t)kb * 12);
      const uint32_t* m = reinterpret_cast<const uint32_t*>(d.meta + row * (k / 8) + (int64_t)kb * 8);
      a.c[0] = c[0]; a.c[1] = c[1]; a.c[2] = c[2];
      a.m[0] = m[0]; a.m[1] = m[1];
    } else {
      a.c[0] = a.c[1] = a.c[2] = 0; a.m[0] = a.m[1] = 0;   // nothing kept: all zero
    }
  } else {
    if (ok) {
      const uint32_t* c = reinterpret_cast<const uint32_t*>(d.packed + row * (k / 8) + (int64_t)kb * 8);
      const uint32_t* m = reinterpret_cast<const uint32_t*>(d.meta + row * (k / 8) + (int64_t)kb * 8);
      a.c[0] = c[0]; a.c[1] = c[1];
      a.m[0] = m[0]; a.m[1] = m[1];
    } else {
      a.c[0] = a.c[1] = 0; a.m[0] = a.m[1] = 0;
    }
  }
}

// 16 weights (operand i of the k-block) as 4 dwords of int8 bytes in k order
template <int KIND>
__device__ __forceinline__ v4i decode_a(const ARaw<KIND>& a, int i, const NmLut& L) {
  if constexpr (KIND == kDense2) {
    return dense2_quad(a.w[i]);
  } else if constexpr (KIND == kNm68) {
    const uint64_t lo64 = (uint64_t)a.c[0] | ((uint64_t)a.c[1] << 32);
    const uint64_t hi64 = (uint64_t)a.c[1] | ((uint64_t)a.c[2] << 32);
    v4i r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int G = 2 * i + h;                       // group of 8 within the k-block
      const uint32_t c12 = (12 * G + 12 <= 64) ? (uint32_t)(lo64 >> (12 * G))
                                                : (uint32_t)(hi64 >> (12 * G - 32));
      const uint32_t mb = (a.m[G >> 2] >> (8 * (G & 3))) & 0xFFu;
      const uint32_t lo = L.spread[c12 & 0xFFu];
      const uint32_t hi = L.spread[(c12 >> 8) & 0xFu];
      r[2 * h] = (int32_t)__builtin_amdgcn_perm(hi, lo, L.sel[mb][0]);
      r[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(hi, lo, L.sel[mb][1]);
    }
    return r;
  } else {
    v4i r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int P = 2 * i + h;                       // byte of codes = two 4-groups
      const uint32_t x = (a.c[P >> 2] >> (8 * (P & 3))) & 0xFFu;
      const uint32_t mb = (a.m[P >> 2] >> (8 * (P & 3))) & 0xFFu;
      const uint32_t v = L.spread[x];
      r[2 * h] = (int32_t)__builtin_amdgcn_perm(v, v, L.sel[mb][0]);
      r[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(v, v, L.sel[mb][1]);
    }
    return r;
  }
}

}  // namespace dec
}  // namespace sbl
