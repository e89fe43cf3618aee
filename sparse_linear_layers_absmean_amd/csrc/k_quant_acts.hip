// Per-token absmax int8 activation quantization.
//
// bitnet.cpp article, "Fundamento matematico", item 2: activations are scaled
// by Qb/gamma with gamma = ||x||_inf and clipped to (-Qb+eps, Qb-eps), Qb =
// 2^(b-1); BitNet spec: 8-bit activations.  Per token (one row of x):
//   gamma = max_k |x|                      (exact, any order)
//   s     = max(gamma, 1e-5) / 128         (exact power-of-two scaling)
//   q     = clamp(rint(x / s), -127, 127)  (the IEEE quotient, rint to even;
//                                           evaluated as in sbl_actq.h)
// One workgroup per token.  Every thread issues the loads of all its 16-byte
// pieces of the row at once and keeps them in registers (up to PER pieces),
// so a row costs one memory round trip; the wavefront max-reduction and the
// quantization then run from registers.  Rows longer than THREADS*PER pieces
// take a second sweep over the row (by then in L2).  Decode-sized batches use
// 1024-thread workgroups (a few tokens must still fill many waves), larger
// batches 256-thread ones.  A decode-sized token of 16384-32768 values is
// split over 8 workgroups: each reads the whole row for gamma (the other
// workgroups' reads hit in L2) and quantizes and stores one eighth of it
// (70B-class down projection, 28672 values: 6.1 -> 4.9 us).
#include "sbl_actq.h"

namespace sbl {

namespace {

template <int THREADS, int PER>
__global__ __launch_bounds__(THREADS) void quant_acts_kernel(const float4* __restrict__ x, int64_t k4,
                                                             uint32_t* __restrict__ xq,
                                                             float* __restrict__ gamma) {
  constexpr int kWaves = THREADS / 64;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const float4* xr = x + row * k4;
  uint32_t* qr = xq + row * k4;
  const bool held = k4 <= (int64_t)THREADS * PER;
  // batches of 128+ tokens (256-thread workgroups) stream their rows once:
  // nontemporal cache policy (2048 x 8640: 20.2 -> 18.2 us, 4096 x 13824:
  // 56.6 -> 49.0 us); a decode token keeps the default (1 x 8192 was 0.2 us
  // slower with it)
  constexpr int kAux = THREADS == 256 ? 2 : 0;
  // pieces past the row read zeros (buffer loads), so every load is issued
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xr, held ? k4 * 16 : 0);
  float4 v[PER];
  float mx = 0.0f;
  if (held) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + i * THREADS) * 16u, 0, kAux));
#pragma unroll
    for (int i = 0; i < PER; ++i) mx = fmaxf(mx, actq::absmax4(v[i]));
  } else {
    for (int64_t i = tid; i < k4; i += 4 * THREADS) {
      float4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = i + u * THREADS < k4 ? xr[i + u * THREADS] : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = fmaxf(mx, actq::absmax4(w[u]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  __shared__ float wmax[kWaves];
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  float g = wmax[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) g = fmaxf(g, wmax[i]);
  const actq::Step st = actq::make_step(g);
  if (held) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t idx = tid + (int64_t)i * THREADS;
      if (idx < k4) qr[idx] = actq::q_word(v[i], st);
    }
  } else {
    for (int64_t i = tid; i < k4; i += THREADS) qr[i] = actq::q_word(xr[i], st);
  }
  if (tid == 0) gamma[row] = g;
}

// One token split over SPLIT workgroups (blockIdx.x = part, blockIdx.y =
// token): every workgroup reduces gamma over the whole row (held in
// registers: k4 <= THREADS * PER), then quantizes and stores part `part` of
// the row; workgroup 0 writes gamma.  All of them compute the same gamma.
template <int THREADS, int PER, int SPLIT>
__global__ __launch_bounds__(THREADS) void quant_acts_split_kernel(const float4* __restrict__ x, int64_t k4,
                                                                   uint32_t* __restrict__ xq,
                                                                   float* __restrict__ gamma) {
  constexpr int kWaves = THREADS / 64;
  const int64_t row = blockIdx.y;
  const int part = blockIdx.x;
  const int tid = threadIdx.x;
  const float4* xr = x + row * k4;
  uint32_t* qr = xq + row * k4;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xr, k4 * 16);
  float4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i)
    v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + i * THREADS) * 16u, 0, 0));
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) mx = fmaxf(mx, actq::absmax4(v[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  __shared__ float wmax[kWaves];
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  float g = wmax[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) g = fmaxf(g, wmax[i]);
  const actq::Step st = actq::make_step(g);
  const int64_t per = (k4 + SPLIT - 1) / SPLIT, i0 = part * per;
  const int64_t i1 = i0 + per < k4 ? i0 + per : k4;
  for (int64_t i = i0 + tid; i < i1; i += THREADS) qr[i] = actq::q_word(xr[i], st);
  if (tid == 0 && part == 0) gamma[row] = g;
}

}  // namespace

hipError_t launch_quant_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                             hipStream_t s) {
  const float4* x4 = reinterpret_cast<const float4*>(x);
  uint32_t* q4 = reinterpret_cast<uint32_t*>(xq);
  if (m_tok < 128 && k >= 16384 && k <= 1024 * 8 * 4)
    hipLaunchKernelGGL((quant_acts_split_kernel<1024, 8, 8>), dim3(8, (unsigned)m_tok), dim3(1024), 0, s, x4, k / 4,
                       q4, gamma);
  else if (m_tok < 128)
    hipLaunchKernelGGL((quant_acts_kernel<1024, 8>), dim3((unsigned)m_tok), dim3(1024), 0, s, x4, k / 4, q4, gamma);
  else if (k <= 256 * 4 * 4)   // register slots sized to the row: fewer registers, more rows resident
    hipLaunchKernelGGL((quant_acts_kernel<256, 4>), dim3((unsigned)m_tok), dim3(256), 0, s, x4, k / 4, q4, gamma);
  else if (k <= 256 * 8 * 4)
    hipLaunchKernelGGL((quant_acts_kernel<256, 8>), dim3((unsigned)m_tok), dim3(256), 0, s, x4, k / 4, q4, gamma);
  else
    hipLaunchKernelGGL((quant_acts_kernel<256, 16>), dim3((unsigned)m_tok), dim3(256), 0, s, x4, k / 4, q4, gamma);
  return hipGetLastError();
}

}  // namespace sbl
