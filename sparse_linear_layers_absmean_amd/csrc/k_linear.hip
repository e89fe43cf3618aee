// Ternary x int8 product with fp32 rescale (BitLinear operation, bitnet.cpp
// article "Fundamento matematico" item 3: y = W~ x~ beta gamma / Qb; no bias
// per the BitNet spec), decode-sized token counts (m_tok <= 16).
//
// int8 MFMA formulation (gfx950 v_mfma_i32_16x16x64_i8): weights are the A
// operand (16 output rows x 64 k), activations the B operand (64 k x 16
// tokens).  A lane holds 16 consecutive k of one row (A) or one token (B).
//  * DENSE2: one 16-weight word decodes with 7 VALU ops into four dwords of
//    u = c + 1 bytes in natural k order; then sum_k u q = sum_k c q + sum_k q,
//    so acc = MFMA result - sum_k q, with sum_k q from v_dot4 against 0x01010101.
//  * N:M 6:8 and 2:4: per group, a 256-entry LDS table spreads the 2-bit kept
//    codes into int8 c bytes, a second table (indexed by the metadata bitmap
//    byte) gives v_perm selectors that scatter them to their k positions and
//    zero the pruned ones: 2 table reads + 2 v_perm per 8 weights.
// Work split: a workgroup owns 32 output rows (two 16-row tiles per wave) and
// its 8 waves split k; a 64-lane load brings 16 rows x 64 weights per tile.
// Partial int32 tiles are summed through LDS, then rescaled.  Up to 8
// independent matrices share one launch (grouped GEMV).  Everything integer
// is exact: |acc| <= 127 k < 2^24.
#include "sbl_decode.h"

namespace sbl {

namespace {

using namespace dec;

constexpr int kTW = 2;                 // 16-row tiles per wave
constexpr int kKS = 8;                 // waves per workgroup (k split)
constexpr int kGemvThreads = 64 * kKS;

template <int KIND>
struct Frag {
  u32x4 b[4];
  ARaw<KIND> a[kTW];
};

template <int KIND>
__device__ __forceinline__ void load_frag(Frag<KIND>& f, const LinDesc& d, int64_t row0, int r, int t,
                                          int sb, int nkb) {
  const int g = (threadIdx.x & 63) >> 4;
  const int kb = 4 * sb + g;
  const bool kok = kb < nkb;
  if (kok && t < d.m_tok) {
    const int8_t* xp = d.xq + (int64_t)t * d.k + (int64_t)kb * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.b[i] = ld16(xp + 16 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.b[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int ti = 0; ti < kTW; ++ti) {
    const int64_t row = row0 + 16 * ti + r;
    load_a<KIND>(f.a[ti], d, row, kb, kok && row < d.n_out);
  }
}

template <int KIND>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const LinBatch batch) {
  __shared__ NmLut lut;
  __shared__ int32_t red[kKS][kTW * 4][64];
  __shared__ int32_t redq[kKS][64];
  if (KIND != kDense2) build_lut<KIND>(lut);
  int di = 0;
  for (int i = 1; i < batch.count; ++i)
    if ((int)blockIdx.x >= batch.start[i]) di = i;
  const LinDesc& d = batch.d[di];
  const int64_t row0 = (int64_t)((int)blockIdx.x - batch.start[di]) * (16 * kTW);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nkb = d.k / 64;
  const int nsb = (nkb + 3) / 4;
  const int sb0 = wave * nsb / kKS, sb1 = (wave + 1) * nsb / kKS;
  if (KIND != kDense2) __syncthreads();

  v4i c[kTW];
#pragma unroll
  for (int ti = 0; ti < kTW; ++ti) c[ti] = v4i{0, 0, 0, 0};
  int qs = 0;
  if (sb0 < sb1) {
    Frag<KIND> cur;
    load_frag<KIND>(cur, d, row0, r, r, sb0, nkb);
    for (int sb = sb0; sb < sb1; ++sb) {
      Frag<KIND> nxt;
      const bool more = sb + 1 < sb1;
      if (more) load_frag<KIND>(nxt, d, row0, r, r, sb + 1, nkb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i b = {(int32_t)cur.b[i][0], (int32_t)cur.b[i][1], (int32_t)cur.b[i][2],
                       (int32_t)cur.b[i][3]};
#pragma unroll
        for (int ti = 0; ti < kTW; ++ti)
          c[ti] = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_a<KIND>(cur.a[ti], i, lut), b, c[ti], 0, 0, 0);
        if (KIND == kDense2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) qs = __builtin_amdgcn_sdot4(b[j], 0x01010101, qs, false);
        }
      }
      if (more) cur = nxt;
    }
  }
  if (KIND == kDense2) {
    qs += __shfl_xor(qs, 16, 64);
    qs += __shfl_xor(qs, 32, 64);                    // sum of q over this wave's k for token lane%16
  }
#pragma unroll
  for (int ti = 0; ti < kTW; ++ti)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][ti * 4 + v][lane] = c[ti][v];
  redq[wave][lane] = qs;
  __syncthreads();
  if (wave >= kTW) return;
  const int ti = wave;
  int32_t sum[4] = {0, 0, 0, 0};
  int32_t qsum = 0;
#pragma unroll
  for (int w = 0; w < kKS; ++w) {
#pragma unroll
    for (int v = 0; v < 4; ++v) sum[v] += red[w][ti * 4 + v][lane];
    qsum += redq[w][lane];
  }
  const int t = r;                                   // C[4*(lane/16)+v][lane%16]: column = token
  if (t >= d.m_tok) return;
  const float s = out_scale(d.beta, d.gamma, t);
  const int64_t rbase = row0 + 16 * ti + 4 * g;
  float* yrow = d.y + (int64_t)t * d.n_out;
  int32_t* arow = d.acc ? d.acc + (int64_t)t * d.n_out : nullptr;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = rbase + v;
    if (row < d.n_out) {
      const int32_t a = sum[v] - (KIND == kDense2 ? qsum : 0);
      yrow[row] = (float)a * s;
      if (arow) arow[row] = a;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic path: any token count, any n:m.  One wave = 16 rows x 16 tokens over
// the whole k; weights decoded to natural-order int8 bytes per 16 k.
// ---------------------------------------------------------------------------

template <int M>
__device__ v4i nm_bytes16(const uint8_t* __restrict__ codes_row, const uint8_t* __restrict__ meta_row,
                          int n, int64_t k0) {
  uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
  for (int gi = 0; gi < 16 / M; ++gi) {
    const int64_t kg = k0 + gi * M;
    uint32_t bits = meta_row[kg >> 3];
    if (M == 4) bits = (bits >> (kg & 4)) & 0xFu;
    int64_t pos = 2 * (kg / M) * n;
    int kept = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      uint32_t cb = 0;
      if (((bits >> j) & 1u) && kept < n) {
        const uint32_t u = (codes_row[pos >> 3] >> (pos & 7)) & 3u;
        cb = (u - 1u) & 0xFFu;
        pos += 2;
        ++kept;
      }
      const int p = gi * M + j;
      out[p >> 2] |= cb << (8 * (p & 3));
    }
  }
  return v4i{(int32_t)out[0], (int32_t)out[1], (int32_t)out[2], (int32_t)out[3]};
}

template <int FMT, int M>
__global__ __launch_bounds__(256) void linear_generic_kernel(const uint8_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ meta, int n,
                                                             const float* __restrict__ beta,
                                                             const int8_t* __restrict__ xq,
                                                             const float* __restrict__ gamma,
                                                             int64_t m_tok, int64_t n_out, int64_t k,
                                                             float* __restrict__ y,
                                                             int32_t* __restrict__ acc_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int64_t r = row0 + (lane & 15);
  const int64_t t = tok0 + (lane & 15);
  const int g = lane >> 4;
  const bool row_ok = r < n_out, tok_ok = t < m_tok;
  const int64_t row_bytes = FMT == 0 ? k / 4 : k * n / (4 * M);
  const uint8_t* wrow = packed + (row_ok ? r : 0) * row_bytes;
  const uint8_t* mrow = FMT == 0 ? nullptr : meta + (row_ok ? r : 0) * (k / 8);
  const int8_t* xrow = xq + (tok_ok ? t : 0) * k;
  v4i c = {0, 0, 0, 0};
  int qs = 0;
  for (int64_t kb = 0; kb < k; kb += 64) {
    const int64_t kk = kb + 16 * g;
    v4i a = {0, 0, 0, 0};
    if (FMT == 0) a = dense2_quad(row_ok ? reinterpret_cast<const uint32_t*>(wrow)[kk >> 4] : 0x55555555u);
    else if (row_ok) a = nm_bytes16<M>(wrow, mrow, n, kk);
    u32x4 nb = {0u, 0u, 0u, 0u};
    if (tok_ok) nb = ld16(xrow + kk);
    const v4i b = {(int32_t)nb[0], (int32_t)nb[1], (int32_t)nb[2], (int32_t)nb[3]};
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    if (FMT == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) qs = __builtin_amdgcn_sdot4(b[j], 0x01010101, qs, false);
    }
  }
  qs += __shfl_xor(qs, 16, 64);
  qs += __shfl_xor(qs, 32, 64);
  if (!tok_ok) return;
  const float s = out_scale(beta, gamma, t);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = row0 + 4 * g + v;            // C[4*(lane/16)+v][lane%16]
    if (row < n_out) {
      const int32_t a = c[v] - (FMT == 0 ? qs : 0);
      y[t * n_out + row] = (float)a * s;
      if (acc_out) acc_out[t * n_out + row] = a;
    }
  }
}

int kind_of(int fmt, int n, int m) {
  if (fmt == 0) return kDense2;
  if (m == 8 && n == 6) return kNm68;
  if (m == 4 && n == 2) return kNm24;
  return -1;
}

hipError_t launch_gemv_group(int kind, const LinDesc* items, int count, hipStream_t s) {
  LinBatch b = {};
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    b.d[i] = items[i];
    b.start[i] = blocks;
    blocks += (int)((items[i].n_out + 16 * kTW - 1) / (16 * kTW));
  }
  b.start[count] = blocks;
  b.count = count;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kGemvThreads);
  if (kind == kDense2) hipLaunchKernelGGL(gemv_kernel<kDense2>, grid, block, 0, s, b);
  else if (kind == kNm68) hipLaunchKernelGGL(gemv_kernel<kNm68>, grid, block, 0, s, b);
  else hipLaunchKernelGGL(gemv_kernel<kNm24>, grid, block, 0, s, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, int fmt, int n, int m, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_out + 63) / 64), (unsigned)((a.m_tok + 15) / 16)), block(256);
  if (fmt == 0)
    hipLaunchKernelGGL((linear_generic_kernel<0, 8>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc);
  else if (m == 8)
    hipLaunchKernelGGL((linear_generic_kernel<1, 8>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc);
  else
    hipLaunchKernelGGL((linear_generic_kernel<1, 4>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc);
  return hipGetLastError();
}

hipError_t launch_linear_batch(const LinearArgs* items, int count, int fmt, int n, int m,
                               hipStream_t s) {
  const int kind = kind_of(fmt, n, m);
  LinDesc gemv[kMaxDesc];
  LinearArgs gemm[kMaxDesc];
  int nv = 0, nm = 0;
  for (int i = 0; i < count; ++i) {
    const LinearArgs& a = items[i];
    if (a.m_tok == 0 || a.n_out == 0) continue;
    hipError_t e = hipSuccess;
    if (kind < 0 || (a.m_tok > kGemvMaxTokens && !gemm_fits(a, kind))) {
      e = launch_linear_generic(a, fmt, n, m, s);
    } else if (a.m_tok <= kGemvMaxTokens) {
      gemv[nv++] = to_desc(a);
      if (nv == kMaxDesc) {
        e = launch_gemv_group(kind, gemv, nv, s);
        nv = 0;
      }
    } else {
      gemm[nm++] = a;
      if (nm == kMaxDesc) {
        e = launch_gemm_group(gemm, nm, kind, s);
        nm = 0;
      }
    }
    if (e != hipSuccess) return e;
  }
  if (nv) {
    const hipError_t e = launch_gemv_group(kind, gemv, nv, s);
    if (e != hipSuccess) return e;
  }
  if (nm) return launch_gemm_group(gemm, nm, kind, s);
  return hipSuccess;
}

}  // namespace sbl
