// Per-token absmax int8 activation quantization.
//
// bitnet.cpp article, "Fundamento matematico", item 2: activations are scaled
// by Qb/gamma with gamma = ||x||_inf and clipped to (-Qb+eps, Qb-eps), Qb =
// 2^(b-1); BitNet spec: 8-bit activations.  Per token (one row of x):
//   gamma = max_k |x|                      (exact, any order)
//   s     = max(gamma, 1e-5) / 128         (exact power-of-two scaling)
//   q     = clamp(rint(x / s), -127, 127)  (one IEEE fp32 division, rint to even)
// One workgroup per token: a wavefront max-reduction, then a second sweep
// over the row (now L2-resident) that writes 4 int8 per 16-byte load.
#include "sbl_internal.h"

namespace sbl {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t q_byte(float v, float s) {
  const float r = rintf(v / s);
  const float c = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)((int32_t)c) & 0xFFu;
}

__global__ __launch_bounds__(kThreads) void quant_acts_kernel(const float4* __restrict__ x, int64_t k4,
                                                              uint32_t* __restrict__ xq,
                                                              float* __restrict__ gamma) {
  const int64_t row = blockIdx.x;
  const float4* xr = x + row * k4;
  float mx = 0.0f;
  for (int64_t i = threadIdx.x; i < k4; i += kThreads) {
    const float4 v = xr[i];
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  float g = wmax[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) g = fmaxf(g, wmax[i]);
  const float s = fmaxf(g, 1e-5f) * 0.0078125f;
  uint32_t* qr = xq + row * k4;
  for (int64_t i = threadIdx.x; i < k4; i += kThreads) {
    const float4 v = xr[i];
    qr[i] = q_byte(v.x, s) | (q_byte(v.y, s) << 8) | (q_byte(v.z, s) << 16) | (q_byte(v.w, s) << 24);
  }
  if (threadIdx.x == 0) gamma[row] = g;
}

}  // namespace

hipError_t launch_quant_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                             hipStream_t s) {
  hipLaunchKernelGGL(quant_acts_kernel, dim3((unsigned)m_tok), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(x), k / 4, reinterpret_cast<uint32_t*>(xq),
                     gamma);
  return hipGetLastError();
}

}  // namespace sbl
