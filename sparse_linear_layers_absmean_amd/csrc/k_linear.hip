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
// Work split: a workgroup owns TB 16-row tiles of one matrix and TB*ks waves;
// the ks waves of a tile split k.  ks and TB are chosen per launch so that the
// grid is about one round of resident waves (a partial second round would run
// at a fraction of the bandwidth).  When the token rows fit (m_tok*k <= 32 KB)
// the workgroup stages them in LDS once and reads MFMA B operands from there,
// with sum_k q computed once per token; otherwise B comes from global memory.
// Each wave keeps kDepth weight loads in flight.  All global loads are buffer
// loads: rows, k-blocks and tokens out of range read zeros, so there is no
// branch around a load.  Partial int32 tiles of the ks waves are summed
// through LDS, then rescaled.  Up to 8 independent matrices share one launch
// (grouped GEMV).  Everything integer is exact: |acc| <= 127 k < 2^24.
#include "sbl_decode.h"

namespace sbl {

namespace {

using namespace dec;

constexpr int kMaxWaves = 16;          // waves per workgroup, at most
constexpr int kResidentWaves = 4096;   // one round: 4 waves per SIMD on 1024 SIMDs
constexpr int kXLdsMax = 32 * 1024;    // token rows staged in LDS up to this many bytes
constexpr uint32_t kFar = 0x80000000u; // a buffer offset beyond every buffer: reads zeros

struct GemvLaunch {
  LinBatch b;
  int32_t ks, tb;                      // waves per tile (k split), tiles per workgroup
};

// Raw weight words of one lane for one 64-weight k-block.  DENSE2: 4 words;
// 6:8: 3 code words + 2 meta words; 2:4: 2 code words + 2 meta words.
struct WStage {
  uint32_t a[5];
};

struct Rsrc {
  __amdgpu_buffer_rsrc_t w, m, x;
};

template <int KIND>
__device__ __forceinline__ void load_w(WStage& s, const Rsrc& rs, uint32_t ow, uint32_t om, int kb, bool kok) {
  if constexpr (KIND == kDense2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs.w, kok ? ow + (uint32_t)kb * 16u : kFar, 0, 0);
    s.a[0] = v[0]; s.a[1] = v[1]; s.a[2] = v[2]; s.a[3] = v[3];
  } else if constexpr (KIND == kNm68) {
    const auto c = __builtin_amdgcn_raw_buffer_load_b96(rs.w, kok ? ow + (uint32_t)kb * 12u : kFar, 0, 0);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rs.m, kok ? om + (uint32_t)kb * 8u : kFar, 0, 0);
    s.a[0] = c[0]; s.a[1] = c[1]; s.a[2] = c[2]; s.a[3] = m[0]; s.a[4] = m[1];
  } else {
    const auto c = __builtin_amdgcn_raw_buffer_load_b64(rs.w, kok ? ow + (uint32_t)kb * 8u : kFar, 0, 0);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rs.m, kok ? om + (uint32_t)kb * 8u : kFar, 0, 0);
    s.a[0] = c[0]; s.a[1] = c[1]; s.a[2] = m[0]; s.a[3] = m[1];
  }
}

// 64 activation bytes of token lane%16 for k-block kb: LDS (XL) or global memory
template <bool XL>
__device__ __forceinline__ void load_x(u32x4 (&b)[4], const Rsrc& rs, const uint8_t* xs, uint32_t ox,
                                       uint32_t zero_off, int kb, bool ok) {
  if constexpr (XL) {
    const uint8_t* p = xs + (ok ? ox + (uint32_t)kb * 64u : zero_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
  } else {
    const uint32_t xo = ok ? ox + (uint32_t)kb * 64u : kFar;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.x, xo, 16 * i, 0));
  }
}

// 2-bit fields -> bytes: 4 fields (8 bits) -> 4 bytes, by shifts and masks
__device__ __forceinline__ uint32_t fields4_to_bytes(uint32_t x) {
  const uint32_t y = (x | (x << 12)) & 0x000F000Fu;
  return (y | (y << 6)) & 0x03030303u;
}

// N:M: 16 weights (operand i of the k-block) as u = c + 1 bytes at the kept
// positions and 0 at the pruned ones, plus the keep mask as 0/1 bytes; the
// product is then MFMA(u) - MFMA(keep).  One table read per 8 weights (the
// v_perm selectors of the bitmap byte); the codes spread arithmetically.
template <int KIND>
__device__ __forceinline__ void nm_operands(const WStage& s, int i, const NmLut& L, v4i& u, v4i& km) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t plo, phi, mb;
    if constexpr (KIND == kNm68) {
      const int G = 2 * i + h;                         // group of 8 within the k-block
      const uint64_t lo64 = (uint64_t)s.a[0] | ((uint64_t)s.a[1] << 32);
      const uint64_t hi64 = (uint64_t)s.a[1] | ((uint64_t)s.a[2] << 32);
      const uint32_t c12 = (12 * G + 12 <= 64) ? (uint32_t)(lo64 >> (12 * G)) : (uint32_t)(hi64 >> (12 * G - 32));
      plo = fields4_to_bytes(c12 & 0xFFu);
      const uint32_t h4 = (c12 >> 8) & 0xFu;
      phi = (h4 | (h4 << 6)) & 0x0303u;
      mb = (s.a[3 + (G >> 2)] >> (8 * (G & 3))) & 0xFFu;
    } else {
      const int P = 2 * i + h;                         // code byte = two groups of 4
      plo = fields4_to_bytes((s.a[P >> 2] >> (8 * (P & 3))) & 0xFFu);
      phi = 0u;
      mb = (s.a[2 + (P >> 2)] >> (8 * (P & 3))) & 0xFFu;
    }
    const uint32_t s0 = L.sel[mb][0], s1 = L.sel[mb][1];
    u[2 * h] = (int32_t)__builtin_amdgcn_perm(phi, plo, s0);
    u[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(phi, plo, s1);
    km[2 * h] = (int32_t)__builtin_amdgcn_perm(0x01010101u, 0x01010101u, s0);
    km[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(0x01010101u, 0x01010101u, s1);
  }
}

// One k-block: c += sum u q, ck += sum keep q (DENSE2: keep = every weight,
// u from the 2-bit word decode), so that acc = c - ck.
template <int KIND>
__device__ __forceinline__ void mac(const WStage& s, const u32x4 (&bq)[4], v4i& c, v4i& ck, const NmLut& L) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4i b = {(int32_t)bq[i][0], (int32_t)bq[i][1], (int32_t)bq[i][2], (int32_t)bq[i][3]};
    if constexpr (KIND == kDense2) {
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(dense2_quad(s.a[i]), b, c, 0, 0, 0);
      const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
      ck = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, ck, 0, 0, 0);
    } else {
      v4i u, km;
      nm_operands<KIND>(s, i, L, u, km);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(u, b, c, 0, 0, 0);
      ck = __builtin_amdgcn_mfma_i32_16x16x64_i8(km, b, ck, 0, 0, 0);
    }
  }
}

// k-block kb = 4*sb + lane/16: super-block sb covers 256 weights of every row
template <int KIND, bool XL>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(const GemvLaunch L) {
  constexpr int D = XL ? 8 : 4;                      // weight loads in flight per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ NmLut lut;
  const LinBatch& batch = L.b;
  const int ks = L.ks;
  if (KIND != kDense2) build_lut<KIND>(lut);
  int di = 0;
  for (int i = 1; i < batch.count; ++i)
    if ((int)blockIdx.x >= batch.start[i]) di = i;
  const LinDesc& d = batch.d[di];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tw = wave / ks, slice = wave - tw * ks;   // tile of the workgroup, k slice
  const int64_t row0 = ((int64_t)((int)blockIdx.x - batch.start[di]) * L.tb + tw) * 16;
  const int r = lane & 15, g = lane >> 4;
  const int nkb = d.k / 64;
  const int nsb = (nkb + 3) / 4;
  const int sb0 = slice * nsb / ks, sb1 = (slice + 1) * nsb / ks;
  const int nit = row0 < d.n_out ? sb1 - sb0 : 0;   // tiles past the matrix: no work
  // buffers over this tile's rows (rows past n_out are outside them) and the activations
  const int64_t rows = d.n_out - row0 < 16 ? (d.n_out - row0 > 0 ? d.n_out - row0 : 0) : 16;
  const int64_t wbytes = KIND == kDense2 ? d.k / 4 : (KIND == kNm68 ? 3 * (int64_t)d.k / 16 : d.k / 8);
  Rsrc rs;
  rs.w = make_rsrc(d.packed + (rows ? row0 * wbytes : 0), rows * wbytes);
  rs.m = make_rsrc(KIND == kDense2 ? d.packed : d.meta + (rows ? row0 * (d.k / 8) : 0),
                   KIND == kDense2 ? 0 : rows * (d.k / 8));
  rs.x = make_rsrc(d.xq, (int64_t)d.m_tok * d.k);
  const uint32_t ow = (uint32_t)(r * wbytes), om = (uint32_t)(r * (d.k / 8));
  // LDS: [token rows m_tok*k (XL)][64 zero bytes][reduction ks*tb*4*64 ints]
  const uint32_t xbytes = XL ? (uint32_t)(d.m_tok * d.k) : 0u;
  const uint32_t zero_off = xbytes;
  int32_t* red = reinterpret_cast<int32_t*>(smem + xbytes + 64);
  const bool r_ok = r < d.m_tok;
  const uint32_t ox = r_ok ? (uint32_t)(r * d.k) : (XL ? zero_off : kFar);

  WStage wa[D];
  u32x4 bring[XL ? 1 : D][4];
  // weight loads of the first stages go out before the activations are staged
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int kb = 4 * (sb0 + j) + g;
    const bool ok = j < nit && kb < nkb;
    load_w<KIND>(wa[j], rs, ow, om, kb, ok);
    if constexpr (!XL) load_x<false>(bring[j], rs, smem, ox, zero_off, kb, ok && r_ok);
  }
  if constexpr (XL) {
    for (uint32_t o = threadIdx.x * 16u; o < xbytes; o += blockDim.x * 16u)
      *reinterpret_cast<u32x4*>(smem + o) =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.x, o, 0, 0));
    if (threadIdx.x < 4) *reinterpret_cast<u32x4*>(smem + zero_off + 16 * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();                               // activations (and the N:M tables)
  } else if (KIND != kDense2) {
    __syncthreads();                               // the N:M tables
  }

  v4i c = {0, 0, 0, 0}, ck = {0, 0, 0, 0};
  // Ring of D stages.  The main loop loads unconditionally (stages past the
  // wave's range read zeros), so the number of loads in flight is static and
  // each step waits only for its own stage.
  int it = 0;
  for (; it + D <= nit; it += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int kb = 4 * (sb0 + it + j) + g;
      u32x4 b[4];
      if constexpr (XL) load_x<true>(b, rs, smem, ox, zero_off, kb, kb < nkb && r_ok);
      else {
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = bring[j][q];
      }
      mac<KIND>(wa[j], b, c, ck, lut);
      const int sb = sb0 + it + j + D;
      const int kb2 = 4 * sb + g;
      const bool ok = sb < sb1 && kb2 < nkb;
      load_w<KIND>(wa[j], rs, ow, om, kb2, ok);
      if constexpr (!XL) load_x<false>(bring[j], rs, smem, ox, zero_off, kb2, ok && r_ok);
      __builtin_amdgcn_sched_barrier(0);            // keep each refill next to its use
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (it + j < nit) {
      const int kb = 4 * (sb0 + it + j) + g;
      u32x4 b[4];
      if constexpr (XL) load_x<true>(b, rs, smem, ox, zero_off, kb, kb < nkb && r_ok);
      else {
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = bring[j][q];
      }
      mac<KIND>(wa[j], b, c, ck, lut);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) c[v] -= ck[v];
  if (ks > 1) {
    int32_t* rw = red + (tw * ks) * 4 * 64;
#pragma unroll
    for (int v = 0; v < 4; ++v) rw[(slice * 4 + v) * 64 + lane] = c[v];
    __syncthreads();
    if (slice != 0) return;
    for (int w = 1; w < ks; ++w) {
#pragma unroll
      for (int v = 0; v < 4; ++v) c[v] += rw[(w * 4 + v) * 64 + lane];
    }
  }
  const int t = r;                                   // C[4*(lane/16)+v][lane%16]: column = token
  if (t >= d.m_tok || row0 >= d.n_out) return;
  const float s = out_scale(d.beta, d.gamma, t);
  const int64_t rbase = row0 + 4 * g;
  float* yrow = d.y + (int64_t)t * d.n_out;
  int32_t* arow = d.acc ? d.acc + (int64_t)t * d.n_out : nullptr;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = rbase + v;
    if (row < d.n_out) {
      yrow[row] = (float)c[v] * s;
      if (arow) arow[row] = c[v];
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

template <int KIND>
void launch_gemv(const GemvLaunch& L, bool xl, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  if (xl) hipLaunchKernelGGL((gemv_kernel<KIND, true>), grid, block, lds, s, L);
  else hipLaunchKernelGGL((gemv_kernel<KIND, false>), grid, block, lds, s, L);
}

hipError_t launch_gemv_group(int kind, const LinDesc* items, int count, hipStream_t s) {
  GemvLaunch L = {};
  int tiles = 0, max_nsb = 1;
  int64_t max_x = 0;
  for (int i = 0; i < count; ++i) {
    tiles += (int)((items[i].n_out + 15) / 16);
    const int nsb = (items[i].k / 64 + 3) / 4;
    max_nsb = nsb > max_nsb ? nsb : max_nsb;
    const int64_t xb = (int64_t)items[i].m_tok * items[i].k;
    max_x = xb > max_x ? xb : max_x;
  }
  if (tiles == 0) return hipSuccess;
  // k split: about one round of resident waves; tiles per workgroup: up to 8 waves
  int ks = kResidentWaves / tiles;
  ks = ks < 1 ? 1 : (ks > kMaxWaves ? kMaxWaves : ks);
  ks = ks > max_nsb ? max_nsb : ks;
  int tb = 8 / ks;
  tb = tb < 1 ? 1 : tb;
  L.ks = ks;
  L.tb = tb;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    L.b.d[i] = items[i];
    L.b.start[i] = blocks;
    const int t = (int)((items[i].n_out + 15) / 16);
    blocks += (t + tb - 1) / tb;
  }
  L.b.start[count] = blocks;
  L.b.count = count;
  const bool xl = max_x <= kXLdsMax;
  const size_t lds = (xl ? (size_t)max_x : 0) + 64 + (ks > 1 ? (size_t)ks * tb * 4 * 64 * sizeof(int32_t) : 0);
  const dim3 grid((unsigned)blocks), block(64 * ks * tb);
  if (kind == kDense2) launch_gemv<kDense2>(L, xl, grid, block, lds, s);
  else if (kind == kNm68) launch_gemv<kNm68>(L, xl, grid, block, lds, s);
  else launch_gemv<kNm24>(L, xl, grid, block, lds, s);
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
