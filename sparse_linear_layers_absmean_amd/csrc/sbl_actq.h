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

__device__ __forceinline__ uint32_t clamp_byte(float n) {
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return (uint32_t)((int32_t)n) & 0xFFu;
}

// Rounded quotient of one value: rint(x * r), and whether it lies within
// 2^-15 of a half-integer (then only the IEEE quotient decides).
__device__ __forceinline__ float q_fast(float v, const Step& st, bool& near) {
  const float y = v * st.r;
  const float f = y - floorf(y);                   // exact: |y| <= 128
  near = near || fabsf(f - 0.5f) <= 0x1p-15f;
  return rintf(y);
}

// q of one value, as a byte (two's complement)
__device__ __forceinline__ uint32_t q_byte(float v, const Step& st) {
  bool near = false;
  float n = q_fast(v, st, near);
  if (near) n = rintf(v / st.s);
  return clamp_byte(n);
}

// four values -> four bytes, little-endian.  The exact quotients are formed
// only when some lane of the wave has a value near a rounding boundary (one
// uniform branch per four values).
__device__ __forceinline__ uint32_t q_word(float4 v, const Step& st) {
  bool nx = false, ny = false, nz = false, nw = false;
  float a = q_fast(v.x, st, nx), b = q_fast(v.y, st, ny), c = q_fast(v.z, st, nz), d = q_fast(v.w, st, nw);
  if (__any(nx || ny || nz || nw)) {
    a = nx ? rintf(v.x / st.s) : a;
    b = ny ? rintf(v.y / st.s) : b;
    c = nz ? rintf(v.z / st.s) : c;
    d = nw ? rintf(v.w / st.s) : d;
  }
  return clamp_byte(a) | (clamp_byte(b) << 8) | (clamp_byte(c) << 16) | (clamp_byte(d) << 24);
}

__device__ __forceinline__ float absmax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace actq
}  // namespace sbl
