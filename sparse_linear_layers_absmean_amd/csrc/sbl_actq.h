// Per-token int8 activation quantization step, shared by the standalone
// quantizer and the GEMV's fused quantization.
//
// bitnet.cpp article, "Fundamento matematico", item 2: x is scaled by
// Qb / gamma (Qb = 128, gamma = max |x| of the token) and clipped; 8-bit
// activations per the BitNet specification.  The reading implemented here:
//   s = max(gamma, 1e-5) / 128            (exact: a power-of-two scaling)
//   q = clamp(rint(RN(x / s)), -127, 127) (one IEEE division, rint half to even)
//
// Evaluation without a division per element.  With r = RN(1/s) and
// y = RN(x * r), y = (x/s)(1 + d1)(1 + d2) with |d1|, |d2| <= 2^-24, so for
// |x/s| <= 128 (always: |x| <= gamma) |y - x/s| <= 2^-16, and RN(x/s) is
// within 2^-18 of x/s.  Hence |y - RN(x/s)| < 2^-15: when y is farther than
// 2^-15 from every half-integer, rint(y) = rint(RN(x/s)) (no half-integer lies
// between them, and RN(x/s) is not a tie).  Otherwise the exact quotient is
// formed with the IEEE division.  The result is identical to one division
// per element; the slow path is taken for about 6e-5 of the values.
#pragma once

#include "sbl_internal.h"

namespace sbl {
namespace actq {

struct Step {
  float s;   // max(gamma, 1e-5) / 128
  float r;   // RN(1 / s)
};

__device__ __forceinline__ Step make_step(float gamma) {
  const float s = fmaxf(gamma, 1e-5f) * 0.0078125f;
  return Step{s, 1.0f / s};
}

// q of one value, as a byte (two's complement)
__device__ __forceinline__ uint32_t q_byte(float v, const Step& st) {
  const float y = v * st.r;
  float n = rintf(y);
  const float f = y - floorf(y);                   // exact: |y| <= 128
  if (fabsf(f - 0.5f) <= 0x1p-15f) n = rintf(v / st.s);
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return (uint32_t)((int32_t)n) & 0xFFu;
}

// four values -> four bytes, little-endian
__device__ __forceinline__ uint32_t q_word(float4 v, const Step& st) {
  return q_byte(v.x, st) | (q_byte(v.y, st) << 8) | (q_byte(v.z, st) << 16) | (q_byte(v.w, st) << 24);
}

__device__ __forceinline__ float absmax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace actq
}  // namespace sbl
