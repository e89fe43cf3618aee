// Group scales (BitNet.cpp article, "Cuantizacion y normalizacion de grupos":
// the quantization parameters are computed per group of weights rather than
// per matrix, so groups need no communication).  A group is a block of
// rows_per_group consecutive output rows; each has its own exact absmean
// beta (the method's "Ternary Quantization" scale, restricted to the group),
// and its rows' codes and outputs use it.
//
//  * group_partial_kernel: workgroup (w, g) adds the magnitudes of slice w of
//    group g's rows exactly (sbl_partial.h) into slot w of the group's
//    workspace region; every group uses the partition of a full group.
//  * group_final_kernel: one workgroup per group rounds the exact mean once
//    (sbl_beta.h) into beta[g].
//  * The mask/pack kernel then reads beta per row group (QDesc.beta_rows).
//  * rescale_grouped_kernel: the products' epilogue with beta per row group,
//    from the int32 products.
#include "sbl_partial.h"

namespace sbl {

namespace {

using namespace part;

__global__ __launch_bounds__(kAbsThreads) void group_partial_kernel(const u32x4* __restrict__ w, int64_t n_out,
                                                                    int64_t k, int64_t rpg, GroupPlan plan,
                                                                    uint64_t* ws) {
  const int64_t g = blockIdx.y, wg = blockIdx.x;
  const int64_t r0 = g * rpg;
  const int64_t rows = n_out - r0 < rpg ? n_out - r0 : rpg;
  const int64_t nvec = rows * k / 8;                      // this group's 16-byte vectors
  const int vpt = (int)plan.vpt;
  const int64_t first = wg * kAbsThreads * vpt;
  int64_t span = nvec - first;
  span = span < 0 ? 0 : (span > (int64_t)kAbsThreads * vpt ? (int64_t)kAbsThreads * vpt : span);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + r0 * k / 8 + (span > 0 ? first : 0), span * 16);
  __shared__ unsigned long long bins[256];
  bins[threadIdx.x] = 0;
  __syncthreads();
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
  for (int j = 0; j < vpt; j += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rw, (threadIdx.x + (j + u) * kAbsThreads) * 16, 0, 0));
#pragma unroll
    for (int u = 0; u < 8; ++u) consume(v[u], acc0, acc1, bins, rare);
  }
  publish_partial(ws + g * plan.region, plan.nb, wg, acc0, acc1, rare, bins);
}

__global__ __launch_bounds__(kAbsThreads) void group_final_kernel(const u32x4* w, int64_t n_out, int64_t k,
                                                                  int64_t rpg, GroupPlan plan, uint64_t* ws,
                                                                  float* beta) {
  const int64_t g = blockIdx.x;
  const int64_t rows = n_out - g * rpg < rpg ? n_out - g * rpg : rpg;
  QDesc d = {};
  d.w = w;
  d.nvec = rows * k / 8;
  d.count = rows * k;
  d.nb = plan.nb;
  d.vpt = plan.vpt;
  d.ws = ws + g * plan.region;
  d.beta = beta + g;
  (void)beta::workgroup_beta(d, true);
}

__global__ void rescale_grouped_kernel(const int32_t* __restrict__ acc, const float* __restrict__ beta, int64_t rpg,
                                       const float* __restrict__ gamma, int64_t m_tok, int64_t n_out,
                                       float* __restrict__ y) {
  const int64_t total = m_tok * n_out, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / n_out, r = i - t * n_out;
    const float s = (fmaxf(beta[r / rpg], 1e-5f) * fmaxf(gamma[t], 1e-5f)) * (1.0f / 128.0f);
    y[i] = (float)acc[i] * s;
  }
}

}  // namespace

hipError_t launch_grouped_beta(const uint16_t* w, int64_t n_out, int64_t k, int64_t rows_per_group, float* beta,
                               uint64_t* ws, hipStream_t s) {
  const GroupPlan plan = group_plan(n_out, k, rows_per_group);
  const int64_t rpg = rows_per_group < n_out ? rows_per_group : n_out;
  const u32x4* wv = reinterpret_cast<const u32x4*>(w);
  hipLaunchKernelGGL(group_partial_kernel, dim3((unsigned)plan.nb, (unsigned)plan.groups), dim3(kAbsThreads), 0, s,
                     wv, n_out, k, rpg, plan, ws);
  hipLaunchKernelGGL(group_final_kernel, dim3((unsigned)plan.groups), dim3(kAbsThreads), 0, s, wv, n_out, k, rpg,
                     plan, ws, beta);
  return hipGetLastError();
}

hipError_t launch_rescale_grouped(const int32_t* acc, const float* beta, int64_t rows_per_group, const float* gamma,
                                  int64_t m_tok, int64_t n_out, float* y, hipStream_t s) {
  const int64_t total = m_tok * n_out;
  int64_t blocks = (total + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks);
  hipLaunchKernelGGL(rescale_grouped_kernel, dim3((unsigned)blocks), dim3(256), 0, s, acc, beta, rows_per_group, gamma,
                     m_tok, n_out, y);
  return hipGetLastError();
}

}  // namespace sbl
