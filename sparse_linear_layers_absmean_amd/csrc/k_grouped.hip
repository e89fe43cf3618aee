// Group scales (BitNet.cpp article, "Cuantizacion y normalizacion de grupos":
// the quantization parameters are computed per group of weights rather than
// per matrix, so groups need no communication).  A group is a block of
// rows_per_group consecutive output rows x cols_per_group consecutive
// features (cols_per_group = k: whole rows); each has its own exact absmean
// beta (the method's "Ternary Quantization" scale, restricted to the group),
// and its weights' codes and products use it.
//
//  * group_partial_kernel: workgroup (w, gr, gc) adds the magnitudes of
//    slice w of group (gr, gc) exactly (sbl_partial.h) into slot w of the
//    group's workspace region; every group uses the partition of a full group.
//  * group_final_kernel: one workgroup per group rounds the exact mean once
//    (sbl_beta.h) into beta[g].
//  * group_wave_kernel: groups of at most 2048 16-byte vectors (one absmean
//    workgroup's worth) instead take one wave each, 4 per workgroup, which
//    sums them exactly in registers and rounds beta[g] itself: one launch,
//    no workspace traffic, no workgroup-wide reductions.
//  * The mask/pack kernel then reads beta per chunk's group (QDesc.beta_rows,
//    beta_kblocks), and the products' epilogues read it per row
//    (LinearArgs.beta_rows) or per row and feature block (the
//    activation-group product).
#include "sbl_partial.h"

namespace sbl {

namespace {

using namespace part;

__global__ __launch_bounds__(kAbsThreads) void group_partial_kernel(const u32x4* __restrict__ w, int64_t n_out,
                                                                    int64_t k, int64_t rpg, int64_t cpg,
                                                                    GroupPlan plan, uint64_t* ws) {
  const int64_t gr = blockIdx.y, gc = blockIdx.z, wg = blockIdx.x;
  const int64_t g = gr * plan.gk + gc;
  const int64_t r0 = gr * rpg;
  const int64_t rows = n_out - r0 < rpg ? n_out - r0 : rpg;
  const int64_t nvec = rows * cpg / 8;                    // this group's 16-byte vectors
  const int vpt = (int)plan.vpt;
  const int64_t first = wg * kAbsThreads * vpt;
  int64_t span = nvec - first;
  span = span < 0 ? 0 : (span > (int64_t)kAbsThreads * vpt ? (int64_t)kAbsThreads * vpt : span);
  __shared__ unsigned long long bins[256];
  bins[threadIdx.x] = 0;
  __syncthreads();
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
  if (cpg == k) {
    // whole rows: the group's vectors are contiguous (one buffer over the slice)
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + r0 * k / 8 + (span > 0 ? first : 0), span * 16);
    for (int j = 0; j < vpt; j += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rw, (threadIdx.x + (j + u) * kAbsThreads) * 16, 0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u) consume(v[u], acc0, acc1, bins, rare);
    }
  } else {
    // a block of columns: vector i of the slice is vector i % vpr of the
    // group's row i / vpr (vpr vectors per row); past the slice: zeros
    const uint32_t vpr = (uint32_t)(cpg / 8);
    const u32x4* base = w + r0 * (k / 8) + gc * vpr;
    for (int j = 0; j < vpt; j += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = (uint32_t)threadIdx.x + (uint32_t)(j + u) * kAbsThreads;
        const uint32_t gi = (uint32_t)first + i;
        v[u] = i < (uint32_t)span ? base[(int64_t)(gi / vpr) * (k / 8) + gi % vpr] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) consume(v[u], acc0, acc1, bins, rare);
    }
  }
  publish_partial(ws + g * plan.region, plan.nb, wg, acc0, acc1, rare, bins);
}

// One wave per group of at most kWaveGroupVecs vectors: every lane adds at
// most 32 vectors (256 values, far below the 2^14 of the fast-window bound)
// into its fp64 sums and the wave's own exponent bins; lane 0 then forms the
// exact total (fast-window units of 2^-38, and the bins as a multi-word
// integer in units of 2^-133 when the wave met out-of-window values) and
// rounds the quotient once, as the workspace path's finalize does.
constexpr int kWaveGroups = 4;                 // waves (groups) per workgroup
constexpr int64_t kWaveGroupVecs = 2048;

__global__ __launch_bounds__(64 * kWaveGroups) void group_wave_kernel(const u32x4* __restrict__ w, int64_t n_out,
                                                                      int64_t k, int64_t rpg, int64_t cpg,
                                                                      GroupPlan plan, float* __restrict__ beta) {
  __shared__ unsigned long long bins_all[kWaveGroups][256];
  __shared__ uint32_t limbs_all[kWaveGroups][beta::kLimbs + 2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned long long* bins = bins_all[wave];
#pragma unroll
  for (int i = 0; i < 4; ++i) bins[lane + 64 * i] = 0;
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * kWaveGroups + wave;
  const bool live = g < plan.groups;                 // waves past the last group only join the barriers
  const int64_t gr = live ? g / plan.gk : 0, gc = live ? g % plan.gk : 0;
  const int64_t r0 = gr * rpg;
  const int64_t rows = n_out - r0 < rpg ? n_out - r0 : rpg;
  const uint32_t nvec = live ? (uint32_t)(rows * cpg / 8) : 0u;
  const uint32_t vpr = (uint32_t)(cpg / 8);          // vectors per row of the group
  const u32x4* base = w + r0 * (k / 8) + gc * vpr;
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
  for (uint32_t j0 = 0; j0 < nvec; j0 += 64 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = j0 + (uint32_t)lane + 64u * u;
      v[u] = i < nvec ? base[(int64_t)(i / vpr) * (k / 8) + i % vpr] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) consume(v[u], acc0, acc1, bins, rare);
  }
  // both sums are exact multiples of 2^-38 below 2^15
  unsigned long long units = (unsigned long long)(acc0 * 0x1p38) + (unsigned long long)(acc1 * 0x1p38);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) units += __shfl_xor(units, off, 64);
  const bool wave_rare = __ballot(rare != 0) != 0;
  __syncthreads();                                   // the wave's bin atomics are done
  if (!live || lane != 0) return;
  const uint64_t count = (uint64_t)(rows * cpg);
  float b;
  if (!wave_rare) {
    b = beta::round_quotient_fast((uint32_t)units, units >> 32, count);
  } else {
    uint32_t* limbs = limbs_all[wave];
    for (int i = 0; i < beta::kLimbs + 2; ++i) limbs[i] = 0;
    for (int e = 0; e < 256; ++e) beta::add_shifted(limbs, bins[e], max(e, 1) - 1);   // significand * 2^(max(e,1)-134)
    beta::add_shifted(limbs, (uint32_t)units, 95);                                   // 2^-38 = 2^95 * 2^-133
    beta::add_shifted(limbs, units >> 32, 95 + 32);
    b = beta::round_quotient(limbs, count);
  }
  beta[g] = b;
}

__global__ __launch_bounds__(kAbsThreads) void group_final_kernel(const u32x4* w, int64_t n_out, int64_t k,
                                                                  int64_t rpg, int64_t cpg, GroupPlan plan,
                                                                  uint64_t* ws, float* beta) {
  const int64_t g = blockIdx.x;
  const int64_t r0 = g / plan.gk * rpg;
  const int64_t rows = n_out - r0 < rpg ? n_out - r0 : rpg;
  QDesc d = {};
  d.w = w;
  d.nvec = rows * cpg / 8;
  d.count = rows * cpg;
  d.nb = plan.nb;
  d.vpt = plan.vpt;
  d.ws = ws + g * plan.region;
  d.beta = beta + g;
  (void)beta::workgroup_beta(d, true);
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

// Products with activation groups: workgroups of kKgRows waves, one output
// row per wave, of one token (fewer, larger workgroups than one wave each:
// a launch over a whole matrix has tens of thousands of rows).  A pass covers
// 16 k-blocks (4 panels): lanes 4c .. 4c+3 take k-block c, 16 consecutive
// weights each, and the 4 lanes' int32 sums make that k-block's exact
// product, kept in the wave's LDS slice.  Then lane j adds up the k-blocks
// of feature block j (an exact int32 sum) and rescales it with beta of the
// row's group and gamma[t][j] (the two roundings of the per-matrix
// epilogue), and the blocks' fp32 results are added in ascending j.
//
// Weights go in as u = c + 1 in {0, 1, 2} (pruned positions u = 1), so that
// sum c x = sum u x - sum x, both as v_dot4_i32_i8 over bytes.
constexpr int kKgPasses = 2;       // passes whose loads are issued together
constexpr int kKgRows = 4;         // waves (rows) per workgroup

struct KgLoad {
  u32x4 x;           // the 16 int8 activations
  uint32_t w;        // DENSE2: the word of the 16 fields; N:M: code bytes 4q .. 4q+3 of the block
  uint64_t keep;     // N:M: the block's keep bitmap
};

// Every load is independent of the others (no address depends on loaded data).
__device__ __forceinline__ KgLoad kg_issue(const uint8_t* packed, const uint8_t* meta, const int8_t* xr,
                                           int64_t n_out, int nkb, int fmt, int n, int m, int64_t row, int kb, int q,
                                           int kb_end) {
  KgLoad L = {u32x4{0u, 0u, 0u, 0u}, 0u, 0ull};
  if (kb < kb_end) {
    L.x = *reinterpret_cast<const u32x4*>(xr + 64 * (int64_t)kb + 16 * q);
    if (fmt == 0) {
      L.w = *reinterpret_cast<const uint32_t*>(packed + panel_offset(n_out, nkb, 16, row, kb) + 4 * q);
    } else {
      const uint2 mv = *reinterpret_cast<const uint2*>(meta + panel_offset(n_out, nkb, 8, row, kb));
      L.keep = (uint64_t)mv.x | ((uint64_t)mv.y << 32);
      const int bb = 16 * n / m;                          // code bytes of a block
      const uint8_t* cp = packed + panel_offset(n_out, nkb, bb, row, kb);
      if (bb % 4 == 0) {                                   // 6:8, 2:4, ...: block offsets are dword-aligned
        if (4 * q < bb) L.w = *reinterpret_cast<const uint32_t*>(cp + 4 * q);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * q + i < bb) L.w |= (uint32_t)cp[4 * q + i] << (8 * i);
      }
    }
  }
  return L;
}

// The 16 weights' u as bytes.  N:M: m divides 16, so the lane's weights hold
// exactly 16 n / m kept codes, stored from code index 16 q n / m on; their
// 32 n / m bits come from the block's 4 lanes (cross-lane reads, uniform in
// the wave: every lane takes part).
__device__ __forceinline__ void kg_decode(const KgLoad& L, int fmt, int n, int m, int lane, uint32_t (&u)[4]) {
  const int q = lane & 3;
  if (fmt == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (L.w >> (2 * j)) & 0x03030303u;   // element 4j + b at bits 8b + 2j
    return;
  }
  const int bit0 = q * 32 * n / m;                        // first field's bit in the block's codes
  const int d0 = bit0 >> 5, base = lane & ~3;
  const int d1 = d0 + 1 <= 3 ? d0 + 1 : 3;               // d0 = 3 only when n = m (shift 0)
  const uint32_t lo = (uint32_t)__shfl((int)L.w, base + d0, 64), hi = (uint32_t)__shfl((int)L.w, base + d1, 64);
  uint32_t f = (uint32_t)((((uint64_t)hi << 32) | lo) >> (bit0 & 31));
  const uint32_t kp = (uint32_t)(L.keep >> (16 * q)) & 0xFFFFu;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool kept = (kp >> (4 * j + b)) & 1u;
      v |= (kept ? (f & 3u) : 1u) << (8 * b);
      f = kept ? f >> 2 : f;
    }
    u[j] = v;
  }
}

__global__ __launch_bounds__(64 * kKgRows) void linear_kgrouped_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ meta, int fmt, int n, int m,
    const float* __restrict__ beta, int64_t rpg, int per_block, const int8_t* __restrict__ xq,
    const float* __restrict__ gamma, int64_t kg, int64_t n_out, int64_t k, float* __restrict__ y) {
  extern __shared__ int32_t kg_lds[];                      // per wave: [nkb] k-block sums, then [groups] fp32 terms
  const int lane = threadIdx.x & 63, c = lane >> 2, q = lane & 3, wave = threadIdx.x >> 6;
  const int64_t row_w = (int64_t)blockIdx.x * kKgRows + wave, t = blockIdx.y;
  const int64_t row = row_w < n_out ? row_w : n_out - 1;   // a row past n_out repeats the last and stores nothing
  const int nkb = (int)(k / 64);
  const int groups = (int)(k / kg), bpg = (int)(kg / 64);
  int32_t* kbsum = kg_lds + wave * (nkb + groups);
  const int8_t* xr = xq + t * k;
  for (int kb0 = 0; kb0 < nkb; kb0 += 16 * kKgPasses) {
    KgLoad L[kKgPasses];
#pragma unroll
    for (int v = 0; v < kKgPasses; ++v)
      L[v] = kg_issue(packed, meta, xr, n_out, nkb, fmt, n, m, row, kb0 + 16 * v + c, q, nkb);
#pragma unroll
    for (int v = 0; v < kKgPasses; ++v) {
      const int kb = kb0 + 16 * v + c;
      uint32_t u[4];
      kg_decode(L[v], fmt, n, m, lane, u);
      int s = 0, sx = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = __builtin_amdgcn_sdot4((int)u[j], (int)L[v].x[j], s, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, (int)L[v].x[j], sx, false);
      }
      s -= sx;
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);                           // the k-block's 4 lanes
      if (q == 0 && kb < nkb) kbsum[kb] = s;
    }
  }
  __syncthreads();
  float* term = reinterpret_cast<float*>(kbsum + nkb);
  // beta of the row's group, or (block scales) of the row's group and feature block j
  const float* brow = per_block ? beta + row / rpg * groups : beta + row / rpg;
  float tj = 0.0f;
  for (int j = lane; j < groups; j += 64) {
    int s = 0;
    for (int i = 0; i < bpg; ++i) s += kbsum[j * bpg + i];
    const float b = fmaxf(brow[per_block ? j : 0], 1e-5f);
    const float sc = (b * fmaxf(gamma[t * groups + j], 1e-5f)) * (1.0f / 128.0f);
    tj = (float)s * sc;
    term[j] = tj;
  }
  float yacc = 0.0f;
  if (groups <= 64) {                                      // the terms sit in lanes 0 .. groups-1
    for (int j = 0; j < groups; ++j)
      yacc = yacc + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tj), j));
  } else {
    __syncthreads();
    for (int j = 0; j < groups; ++j) yacc = yacc + term[j];
  }
  if (lane == 0 && row_w < n_out) y[t * n_out + row_w] = yacc;
}

}  // namespace

hipError_t launch_quant_acts_kgrouped(const float* x, int64_t m_tok, int64_t k, int64_t kg, int8_t* xq, float* gamma,
                                      hipStream_t s) {
  hipLaunchKernelGGL(quant_acts_kgrouped_kernel, dim3((unsigned)(k / kg), (unsigned)m_tok), dim3(256), 0, s, x, k, kg,
                     xq, gamma);
  return hipGetLastError();
}

hipError_t launch_linear_kgrouped(const uint8_t* packed, const uint8_t* meta, int fmt, int n, int m, const float* beta,
                                  int64_t rows_per_group, bool beta_per_block, const int8_t* xq, const float* gamma,
                                  int64_t kg, int64_t m_tok, int64_t n_out, int64_t k, float* y, hipStream_t s) {
  // LDS per wave: k/64 int32 block sums and k/kg fp32 terms (at most 2 * 2048 words)
  const size_t lds = (size_t)kKgRows * (k / 64 + k / kg) * 4;
  hipLaunchKernelGGL(linear_kgrouped_kernel, dim3((unsigned)((n_out + kKgRows - 1) / kKgRows), (unsigned)m_tok),
                     dim3(64 * kKgRows), lds, s, packed, meta, fmt, n, m, beta, rows_per_group, beta_per_block ? 1 : 0,
                     xq, gamma, kg, n_out, k, y);
  return hipGetLastError();
}

hipError_t launch_grouped_beta(const uint16_t* w, int64_t n_out, int64_t k, int64_t rows_per_group,
                               int64_t cols_per_group, float* beta, uint64_t* ws, hipStream_t s) {
  const GroupPlan plan = group_plan(n_out, k, rows_per_group, cols_per_group);
  const int64_t rpg = rows_per_group < n_out ? rows_per_group : n_out;
  const u32x4* wv = reinterpret_cast<const u32x4*>(w);
  if ((rpg * cols_per_group) / 8 <= kWaveGroupVecs) {     // small groups: one wave each, one launch
    hipLaunchKernelGGL(group_wave_kernel, dim3((unsigned)((plan.groups + kWaveGroups - 1) / kWaveGroups)),
                       dim3(64 * kWaveGroups), 0, s, wv, n_out, k, rpg, cols_per_group, plan, beta);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(group_partial_kernel, dim3((unsigned)plan.nb, (unsigned)plan.gr, (unsigned)plan.gk),
                     dim3(kAbsThreads), 0, s, wv, n_out, k, rpg, cols_per_group, plan, ws);
  hipLaunchKernelGGL(group_final_kernel, dim3((unsigned)plan.groups), dim3(kAbsThreads), 0, s, wv, n_out, k, rpg,
                     cols_per_group, plan, ws, beta);
  return hipGetLastError();
}

}  // namespace sbl
