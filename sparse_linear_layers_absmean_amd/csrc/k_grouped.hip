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

// Activation groups along k: workgroup (j, t) quantizes features
// [j kg, (j + 1) kg) of token t with that block's own gamma = max |x| over the
// block, exactly as the per-token quantizer does over a whole row:
// s = max(gamma, 1e-5) / 128 (exact), q = clamp(rint(x / s), -127, 127).
__global__ __launch_bounds__(256) void quant_acts_kgrouped_kernel(const float* __restrict__ x, int64_t k, int64_t kg,
                                                                  int8_t* __restrict__ xq, float* __restrict__ gamma) {
  const int64_t j = blockIdx.x, t = blockIdx.y, groups = k / kg;
  const float* xr = x + t * k + j * kg;
  float mx = 0.0f;
  for (int64_t i = threadIdx.x; i < kg; i += 256) mx = fmaxf(mx, fabsf(xr[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  const float g = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float sc = fmaxf(g, 1e-5f) * 0.0078125f;
  int8_t* qr = xq + t * k + j * kg;
  for (int64_t i = threadIdx.x; i < kg; i += 256) {
    const float r = rintf(xr[i] / sc);
    qr[i] = (int8_t)(int32_t)fminf(fmaxf(r, -127.0f), 127.0f);
  }
  if (threadIdx.x == 0) gamma[t * groups + j] = g;
}

// Products with activation groups: one single-wave workgroup per (output row,
// token).  A pass covers one panel (4 k-blocks): lanes 16c .. 16c+15 take
// k-block 4p + c, 4 consecutive weights each, and the 16 lanes' int32 sums
// make that k-block's exact product, kept in LDS.  Then lane j adds up the
// k-blocks of feature block j (an exact int32 sum) and rescales it with beta
// of the row's group and gamma[t][j] (the two roundings of the per-matrix
// epilogue), and lane 0 adds the blocks' fp32 results in ascending j.
constexpr int kKgPanels = 8;       // panels whose loads are issued together

// The 4 codes (as int, -1/0/+1) of weights 4e .. 4e+3 of k-block kb of `row`.
// N:M: the kept codes of a block are stored in ascending position, 2 bits
// each; those of the 4 weights are consecutive, so they lie in 2 bytes.  Each
// lane loads byte e of its block's codes (with the keep bitmap and the
// activations, all independent loads); the two bytes a lane needs then come
// from the 16 lanes of its block by cross-lane reads.
struct KgLoad {
  uint32_t w;        // DENSE2: the word holding the 4 fields; N:M: code byte e, then the lane's 2 code bytes
  uint64_t keep;     // N:M: the block's keep bitmap
  uint32_t x;        // the 4 int8 activations
};

__device__ __forceinline__ KgLoad kg_issue(const uint8_t* packed, const uint8_t* meta, const int8_t* xr,
                                           int64_t n_out, int nkb, int fmt, int n, int m, int64_t row, int kb, int e) {
  KgLoad L = {0u, 0ull, 0u};
  if (kb < nkb) {
    L.x = *reinterpret_cast<const uint32_t*>(xr + 64 * (int64_t)kb + 4 * e);
    if (fmt == 0) {
      L.w = *reinterpret_cast<const uint32_t*>(packed + panel_offset(n_out, nkb, 16, row, kb) + 4 * (e >> 2));
    } else {
      const uint2 mv = *reinterpret_cast<const uint2*>(meta + panel_offset(n_out, nkb, 8, row, kb));
      L.keep = (uint64_t)mv.x | ((uint64_t)mv.y << 32);
      if (e < 16 * n / m) L.w = packed[panel_offset(n_out, nkb, 16 * n / m, row, kb) + e];
    }
  }
  return L;
}

// N:M: gather the lane's 2 code bytes (uniform in the wave: every lane takes part)
__device__ __forceinline__ void kg_gather(KgLoad& L, int n, int m, int lane) {
  const int e = lane & 15, p0 = 4 * e, g0 = p0 / m * m;
  const int idx0 = p0 / m * n + __popcll((L.keep >> g0) & ((1ull << (p0 - g0)) - 1ull));
  // idx0 can be the block's code count when none of the 4 is kept (n <= 4 of
  // 8): both byte indexes stay inside the block, and then no field is used
  const int last = (16 * n / m) - 1;                      // the block's last code byte
  const int b0 = (idx0 >> 2) <= last ? (idx0 >> 2) : last;
  const int b1 = b0 + 1 <= last ? b0 + 1 : last;
  const int base = lane & ~15;
  const uint32_t v0 = (uint32_t)__shfl((int)L.w, base + b0, 64), v1 = (uint32_t)__shfl((int)L.w, base + b1, 64);
  L.w = (v0 | (v1 << 8)) >> (2 * (idx0 & 3));
}

__device__ __forceinline__ int kg_dot(const KgLoad& L, int fmt, int e) {
  int s = 0, j = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c;
    if (fmt == 0) {
      c = (int)((L.w >> (8 * i + 2 * (e & 3))) & 3u) - 1;
    } else {
      const bool kept = (L.keep >> (4 * e + i)) & 1u;
      c = kept ? (int)((L.w >> (2 * j)) & 3u) - 1 : 0;
      j += kept ? 1 : 0;
    }
    s += c * (int)(int8_t)(L.x >> (8 * i));
  }
  return s;
}

__global__ __launch_bounds__(64) void linear_kgrouped_kernel(const uint8_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ meta, int fmt, int n, int m,
                                                             const float* __restrict__ beta, int64_t rpg,
                                                             const int8_t* __restrict__ xq,
                                                             const float* __restrict__ gamma, int64_t kg,
                                                             int64_t n_out, int64_t k, float* __restrict__ y) {
  extern __shared__ int32_t kbsum[];                       // [nkb] k-block sums, then [groups] fp32 terms
  const int lane = threadIdx.x, c = lane >> 4, e = lane & 15;
  const int64_t row = blockIdx.x, t = blockIdx.y;
  const int nkb = (int)(k / 64);
  const int groups = (int)(k / kg), bpg = (int)(kg / 64);
  const int8_t* xr = xq + t * k;
  for (int kb0 = 0; kb0 < nkb; kb0 += 4 * kKgPanels) {
    KgLoad L[kKgPanels];
#pragma unroll
    for (int u = 0; u < kKgPanels; ++u)
      L[u] = kg_issue(packed, meta, xr, n_out, nkb, fmt, n, m, row, kb0 + 4 * u + c, e);
#pragma unroll
    for (int u = 0; u < kKgPanels; ++u) {
      const int kb = kb0 + 4 * u + c;
      if (fmt != 0) kg_gather(L[u], n, m, lane);
      int s = kb < nkb ? kg_dot(L[u], fmt, e) : 0;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);   // within the 16 lanes
      if (e == 0 && kb < nkb) kbsum[kb] = s;
    }
  }
  __syncthreads();
  float* term = reinterpret_cast<float*>(kbsum + nkb);
  const float b = fmaxf(beta[row / rpg], 1e-5f);
  for (int j = lane; j < groups; j += 64) {
    int s = 0;
    for (int i = 0; i < bpg; ++i) s += kbsum[j * bpg + i];
    const float sc = (b * fmaxf(gamma[t * groups + j], 1e-5f)) * (1.0f / 128.0f);
    term[j] = (float)s * sc;
  }
  __syncthreads();
  if (lane == 0) {
    float yacc = 0.0f;
    for (int j = 0; j < groups; ++j) yacc = yacc + term[j];
    y[t * n_out + row] = yacc;
  }
}

}  // namespace

hipError_t launch_quant_acts_kgrouped(const float* x, int64_t m_tok, int64_t k, int64_t kg, int8_t* xq, float* gamma,
                                      hipStream_t s) {
  hipLaunchKernelGGL(quant_acts_kgrouped_kernel, dim3((unsigned)(k / kg), (unsigned)m_tok), dim3(256), 0, s, x, k, kg,
                     xq, gamma);
  return hipGetLastError();
}

hipError_t launch_linear_kgrouped(const uint8_t* packed, const uint8_t* meta, int fmt, int n, int m, const float* beta,
                                  int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t kg,
                                  int64_t m_tok, int64_t n_out, int64_t k, float* y, hipStream_t s) {
  // LDS: k/64 int32 block sums and k/kg fp32 terms, at most 2 * 2048 words
  const size_t lds = (size_t)(k / 64 + k / kg) * 4;
  hipLaunchKernelGGL(linear_kgrouped_kernel, dim3((unsigned)n_out, (unsigned)m_tok), dim3(64), lds, s, packed, meta,
                     fmt, n, m, beta, rows_per_group, xq, gamma, kg, n_out, k, y);
  return hipGetLastError();
}

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
