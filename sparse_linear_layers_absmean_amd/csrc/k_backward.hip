// Backward of the Sparse-BitLinear layer under the dual straight-through
// estimator (Sparse-BitNet summaries: Spanish section 2, "Estrategia de
// Entrenamiento", Dual STE; Arabic section 2, item 3): the quantizers pass
// the gradient as the identity inside their clipping range, and the mask
// passes it densely to every master weight, the pruned ones included.  The
// scales beta and gamma are constants; dY is BF16; results are fp32.
//
//   dX[t, k] = RN(beta_eff * sum_n dY[t, n] C[n, k])   where the activation
//              clamp did not act (|rint(128 x / gamma_eff)| <= 127), else 0
//   dW[n, k] = sum_t dY[t, n] x_hat[t, k],  x_hat = RN_fp32(gamma_eff q) 2^-7,
//              for every (n, k)
//
// Both are contractions on the BF16 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation) with exact products: C is {-1, 0, 1}, and x_hat (24
// significant bits) is split exactly into three BF16 parts, so dW takes
// three MFMA per step.  Output tiles of 128 x 128 per 4 waves (each wave
// 64 x 64: 2 x 2 MFMA tiles), 64 of the contracted index per LDS stage; the
// stage's global loads are issued one stage ahead into registers, and the LDS
// hand-offs use barriers that leave them in flight.
//   dX: i = token, j = feature, l = output channel; A = dY rows, B = C decoded
//       from the packed weights (DENSE2 or N:M + bitmap, panel-major).
//   dW: i = output channel, j = feature, l = token; A = dY^T, B = x_hat.
#include "sbl_internal.h"


namespace sbl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBT = 256;          // threads
constexpr int kTile = 128;        // output tile edge
constexpr int kStep = 64;         // contracted indices per LDS stage
constexpr int kRow = kStep + 8;   // LDS row length in bf16 (144 bytes: 16-byte aligned, bank-spread)

constexpr uint16_t kOne = 0x3F80u;   // BF16 1.0 (-1.0 is kOne with the sign bit)
// token tiles per dX workgroup and channel tiles per dW workgroup (measured on
// the 3B-class block at 2048 tokens: dX 2.11 / 1.78 / 2.93 ms for 1 / 2 / 4;
// dW 2.77 / 3.11 ms for 1 / 2: the larger LDS footprint halves the resident
// workgroups)
constexpr int kDxTW = 2, kDwNW = 1;

__device__ __forceinline__ bf16x8 lds_vec(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// the 2 x 2 MFMA tiles of this wave for one LDS stage (16-deep sub-steps);
// A_s: [kTile][kRow] by i, B_s: [kTile][kRow] by j, both l-contiguous
__device__ __forceinline__ void mma_stage(const uint16_t* A_s, const uint16_t* B_s, f32x16 (&acc)[2][2], int wi,
                                          int wj, int li, int g) {
#pragma unroll
  for (int s = 0; s < kStep / 16; ++s) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      a[t] = lds_vec(A_s + (64 * wi + 32 * t + li) * kRow + 16 * s + 8 * g);
      b[t] = lds_vec(B_s + (64 * wj + 32 * t + li) * kRow + 16 * s + 8 * g);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
  }
}

// dW's stage: the same A operands against the three parts of x_hat (A read
// once per sub-step)
__device__ __forceinline__ void mma_stage3(const uint16_t* A_s, const uint16_t (*B_s)[kTile * kRow],
                                           f32x16 (&acc)[2][2], int wi, int wj, int li, int g) {
#pragma unroll
  for (int s = 0; s < kStep / 16; ++s) {
    bf16x8 a[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) a[t] = lds_vec(A_s + (64 * wi + 32 * t + li) * kRow + 16 * s + 8 * g);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      bf16x8 b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) b[t] = lds_vec(B_s[p] + (64 * wj + 32 * t + li) * kRow + 16 * s + 8 * g);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
    }
  }
}

// the packed weights of the product (either format, panel-major)
struct PackedW {
  const uint8_t* packed;
  const uint8_t* meta;
  int64_t n_out;
  int32_t nkb, fmt, n, m;
};

// Raw words of one (row, quarter): loaded a stage ahead, decoded when the
// stage is staged (quarter_load / quarter_fields), so that no load result is
// consumed in the stage that issues it.
struct QRaw {
  uint32_t w;              // DENSE2: the quarter's word
  uint32_t m0, m1;         // N:M: the block's bitmap
  uint32_t h[3];           // N:M: three code halfwords from the quarter's first code on
};

// a quarter outside the matrix: u = 1 (code 0) everywhere, in both formats
__device__ __forceinline__ QRaw quarter_zero() { return QRaw{0x55555555u, 0u, 0u, {0u, 0u, 0u}}; }

__device__ __forceinline__ QRaw quarter_load(const PackedW& W, int64_t row, int kb, int qq) {
  QRaw r = quarter_zero();
  if (W.fmt == 0) {
    r.w = *reinterpret_cast<const uint32_t*>(W.packed + panel_offset(W.n_out, W.nkb, 16, row, kb) + 4 * qq);
    return r;
  }
  // N:M: the kept weights of the block, in ascending order, hold consecutive
  // 2-bit codes; exactly n per group of m, so the quarter's first kept weight
  // is number 16 qq n / m, and its codes take at most 32 bits from bit
  // s = 32 qq n / m on: three halfwords (those inside the block) hold them
  const int bb = 16 * W.n / W.m;                           // code bytes per block (even)
  const uint16_t* cp = reinterpret_cast<const uint16_t*>(W.packed + panel_offset(W.n_out, W.nkb, bb, row, kb));
  const uint2 mv = *reinterpret_cast<const uint2*>(W.meta + panel_offset(W.n_out, W.nkb, 8, row, kb));
  r.m0 = mv.x;
  r.m1 = mv.y;
  const int h0 = (32 * qq * W.n / W.m) >> 4;
#pragma unroll
  for (int j = 0; j < 3; ++j) r.h[j] = h0 + j < bb / 2 ? cp[h0 + j] : 0u;
  return r;
}

// 16 ternary codes of the quarter (weights 16 qq .. 16 qq + 15 of its
// 64-weight block) as u = c + 1 in 2-bit fields (field e = weight 16 qq + e)
__device__ __forceinline__ uint32_t quarter_fields(const PackedW& W, const QRaw& r, int qq) {
  if (W.fmt == 0) {
    // DENSE2 block word qq holds weights 16 qq .. +15: weight 16 qq + e at bit 8 (e % 4) + 2 (e / 4)
    uint32_t f = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) f |= ((r.w >> (8 * (e & 3) + 2 * (e >> 2))) & 3u) << (2 * e);
    return f;
  }
  const uint32_t keep = (uint32_t)(((uint64_t)r.m0 | ((uint64_t)r.m1 << 32)) >> (16 * qq)) & 0xFFFFu;
  const int s0 = 32 * qq * W.n / W.m;
  uint64_t win = (uint64_t)r.h[0] | ((uint64_t)r.h[1] << 16) | ((uint64_t)r.h[2] << 32);
  win >>= s0 & 15;                                         // bit 0: the quarter's first code
  uint32_t f = 0;
  int idx = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    uint32_t u = 1u;                                       // pruned: code 0
    if ((keep >> e) & 1u) {
      u = (uint32_t)(win >> (2 * idx)) & 3u;
      ++idx;
    }
    f |= u << (2 * e);
  }
  return f;
}

// Workgroup barrier for the LDS hand-offs.  Unlike __syncthreads() it does
// not wait for outstanding global loads (vmcnt), so the next stage's
// prefetch stays in flight across it; the "memory" clobber keeps LDS
// accesses on their side.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// BF16 bits of the code c = u - 1 for a 2-bit field u: 1.0, 0 or -1.0
__device__ __forceinline__ uint32_t code_bf16(uint32_t u) {
  return u == 1u ? 0u : (uint32_t)kOne | (u == 0u ? 0x8000u : 0u);
}

// two 16-bit elements, element j of a and of b, as one dword (a's low)
__device__ __forceinline__ uint32_t pair16(uint32_t a, uint32_t b, int j) {
  return __builtin_amdgcn_perm(b, a, (j & 1) ? 0x07060302u : 0x05040100u);
}

// dX tile: 128 TW tokens x 128 features per workgroup of 4 TW waves (each
// 64 x 64).  The transposed ternary B tile of a stage is decoded once per
// workgroup and feeds all TW token tiles: the decode, not the MFMAs, is the
// VALU-heavy part (with 128 tokens: 36 VALU instructions per MFMA).
template <int TW>
__global__ __launch_bounds__(kBT * TW) void backward_dx_kernel(const uint16_t* __restrict__ dy, int64_t m_tok,
                                                               int64_t n_out, int64_t k, PackedW W,
                                                               const float* __restrict__ beta,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ gamma,
                                                               float* __restrict__ dx) {
  constexpr int kThr = kBT * TW, kTT = kTile * TW;
  constexpr int kItems = (kTile / 16 * kStep + kThr - 1) / kThr;   // (channel, quarter) items per thread
  constexpr int kVecs = kTile / 16 * 8 * 16 / kThr;                // B vectors written per thread
  __shared__ __attribute__((aligned(16))) uint16_t A_s[kTT * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t B_s[kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint32_t F_s[kTile / 16][kStep];   // 2-bit fields per (quarter, channel)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * kTT, k0 = (int64_t)blockIdx.x * kTile;
  f32x16 acc[2][2] = {};
  // A: dY[t0 + r][n0 .. n0 + 63], four 16-byte pieces per thread (n_out % 8 == 0);
  // B: (channel, quarter) items tid, tid + kThr, ...  Each stage's global
  // loads are issued one stage ahead, into registers.
  const int ar = tid >> 1, ah = tid & 1;
  u32x4 ra[4];
  QRaw rb[kItems];
  auto load_stage = [&](int64_t n0) {
    const int64_t t = t0 + ar;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t nn = n0 + 32 * ah + 8 * v;
      ra[v] = u32x4{0u, 0u, 0u, 0u};
      if (t < m_tok && nn < n_out) ra[v] = *reinterpret_cast<const u32x4*>(dy + t * n_out + nn);
    }
#pragma unroll
    for (int h = 0; h < kItems; ++h) {
      const int idx = tid + kThr * h, nl = idx & 63, q = idx >> 6;   // q: features k0 + 16 q .. +15
      const int64_t row = n0 + nl;
      const int kb = (int)(k0 / 64) + (q >> 2);
      rb[h] = idx < kTile / 16 * kStep && row < n_out && kb < W.nkb ? quarter_load(W, row, kb, q & 3)
                                                                     : quarter_zero();
    }
  };
  load_stage(0);
  for (int64_t n0 = 0; n0 < n_out; n0 += kStep) {
    lds_barrier();                                         // the previous stage has been read
#pragma unroll
    for (int v = 0; v < 4; ++v) *reinterpret_cast<u32x4*>(A_s + ar * kRow + 32 * ah + 8 * v) = ra[v];
    // B: C[n0 + nl][k0 + 16 q + e] -> B_s[16 q + e][nl], in two passes so
    // that every LDS write is a whole 16-byte vector: first the 2-bit fields
    // of each (output channel, 16-feature quarter) go to F_s, then each
    // vector (8 channels rg of one feature e) is gathered from F_s.  (One
    // 2-byte write per value put a wave's 64 writes on 4 banks.)
#pragma unroll
    for (int h = 0; h < kItems; ++h) {
      const int idx = tid + kThr * h, nl = idx & 63, q = idx >> 6;
      if (idx < kTile / 16 * kStep) F_s[q][nl] = quarter_fields(W, rb[h], q & 3);
    }
    if (n0 + kStep < n_out) load_stage(n0 + kStep);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int w = tid + kThr * i, rg = w & 7, e = (w >> 3) & 15, q = w >> 7;
      const u32x4 f0 = *reinterpret_cast<const u32x4*>(&F_s[q][8 * rg]);
      const u32x4 f1 = *reinterpret_cast<const u32x4*>(&F_s[q][8 * rg + 4]);
      const uint32_t fw[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
      u32x4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        d[j] = code_bf16((fw[2 * j] >> (2 * e)) & 3u) | (code_bf16((fw[2 * j + 1] >> (2 * e)) & 3u) << 16);
      *reinterpret_cast<u32x4*>(B_s + (16 * q + e) * kRow + 8 * rg) = d;
    }
    lds_barrier();
    mma_stage(A_s, B_s, acc, wi, wj, li, g);
  }
  // epilogue: lane (li, g) holds D[8 (v / 4) + 4 g + v % 4][li] of each 32 x 32 tile
  const float b = fmaxf(beta[0], 1e-5f);
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + 64 * wi + 32 * ti + 8 * (v >> 2) + 4 * g + (v & 3);
        const int64_t kk = k0 + 64 * wj + 32 * tj + li;
        if (t < m_tok && kk < k) {
          const float s = fmaxf(gamma[t], 1e-5f) * (1.0f / 128.0f);   // exact power-of-two scaling
          const float r = rintf(x[t * k + kk] / s);                 // the forward's fp32 quotient
          dx[t * k + kk] = fabsf(r) <= 127.0f ? b * acc[ti][tj][v] : 0.0f;
        }
      }
}

// x_hat = RN(gamma_eff q) 2^-7 split exactly into three BF16 parts (24
// significant bits, 8 per part: truncations and exact differences)
__device__ __forceinline__ void split3(float xh, uint16_t& h1, uint16_t& h2, uint16_t& h3) {
  const uint32_t b1 = __float_as_uint(xh) & 0xFFFF0000u;
  const float r1 = xh - __uint_as_float(b1);
  const uint32_t b2 = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(b2);
  h1 = (uint16_t)(b1 >> 16);
  h2 = (uint16_t)(b2 >> 16);
  h3 = (uint16_t)(__float_as_uint(r2) >> 16);
}

// dW tile: 128 NW output channels x 128 features per workgroup of 4 NW waves
// (each 64 x 64).  The three BF16 parts of a stage's x_hat tile are computed
// once per workgroup and feed all NW channel tiles (the split, repeated for
// every channel tile, is the VALU-heavy part).
template <int NW>
__global__ __launch_bounds__(kBT * NW) void backward_dw_kernel(const uint16_t* __restrict__ dy, int64_t m_tok,
                                                               int64_t n_out, int64_t k,
                                                               const int8_t* __restrict__ xq,
                                                               const float* __restrict__ gamma,
                                                               float* __restrict__ dw) {
  constexpr int kTN = kTile * NW;
  constexpr int kJ = 8 / NW;                               // x_hat columns per thread
  __shared__ __attribute__((aligned(16))) uint16_t A_s[kTN * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t B_s[3][kTile * kRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kTN, k0 = (int64_t)blockIdx.x * kTile;
  f32x16 acc[2][2] = {};
  // staging (both operands transposed: the stage's 64 tokens are the MFMA's
  // contracted index): thread = tokens t0 + 4 tq .. +3 x 8 columns, transposed
  // in registers and written as 8-byte vectors (4 tokens of one column), so
  // that 16 lanes fill 128 contiguous bytes of one LDS row.  (One 2-byte write
  // per value put a wave's writes on a few banks.)  x_hat: thread = 4 tokens x
  // kJ columns (8 cb + kJ jh ..).
  const int tq = tid & 15, cb = tid >> 4;                  // token quad, 8-column block of dY
  const int xb = (tid >> 4) & 15, jh = tid >> 8;           // x_hat: 8-column block, its part jh
  // each stage's global loads are issued one stage ahead, into registers
  u32x4 va[4];                                             // dY[t0 + 4 tq + tt][n0 + 8 cb .. +7]
  uint32_t qv[4][kJ / 4];                                  // xq[t0 + 4 tq + tt][k0 + 8 xb + kJ jh .. +kJ-1]
  float ge[4];                                             // gamma_eff of those tokens
  auto load_stage = [&](int64_t t0) {
    const int64_t nn = n0 + 8 * cb;
    const int64_t kk = k0 + 8 * xb + kJ * jh;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int64_t t = t0 + 4 * tq + tt;
      va[tt] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < kJ / 4; ++w) qv[tt][w] = 0u;
      ge[tt] = 0.0f;
      if (t < m_tok && nn < n_out) va[tt] = *reinterpret_cast<const u32x4*>(dy + t * n_out + nn);
      if (t < m_tok && kk < k) {
#pragma unroll
        for (int w = 0; w < kJ / 4; ++w) qv[tt][w] = reinterpret_cast<const uint32_t*>(xq + t * k + kk)[w];
        ge[tt] = fmaxf(gamma[t], 1e-5f);
      }
    }
  };
  load_stage(0);
  for (int64_t t0 = 0; t0 < m_tok; t0 += kStep) {
    lds_barrier();
    // A: dY[t0 + 4 tq + tt][n0 + 8 cb + j] -> A_s[8 cb + j][4 tq + tt]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint2 d = make_uint2(pair16(va[0][j >> 1], va[1][j >> 1], j), pair16(va[2][j >> 1], va[3][j >> 1], j));
      *reinterpret_cast<uint2*>(A_s + (8 * cb + j) * kRow + 4 * tq) = d;
    }
    // B: x_hat[t0 + 4 tq + tt][k0 + c] in three parts -> B_s[p][c][4 tq + tt], c = 8 xb + kJ jh + j
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      uint16_t h[3][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int qe = (int)(int8_t)(qv[tt][j >> 2] >> (8 * (j & 3)));
        const float xh = (ge[tt] * (float)qe) * (1.0f / 128.0f);
        split3(xh, h[0][tt], h[1][tt], h[2][tt]);
      }
      const int c = 8 * xb + kJ * jh + j;
#pragma unroll
      for (int p = 0; p < 3; ++p)
        *reinterpret_cast<uint2*>(B_s[p] + c * kRow + 4 * tq) =
            make_uint2((uint32_t)h[p][0] | ((uint32_t)h[p][1] << 16), (uint32_t)h[p][2] | ((uint32_t)h[p][3] << 16));
    }
    if (t0 + kStep < m_tok) load_stage(t0 + kStep);
    lds_barrier();
    mma_stage3(A_s, B_s, acc, wi, wj, li, g);
  }
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t nn = n0 + 64 * wi + 32 * ti + 8 * (v >> 2) + 4 * g + (v & 3);
        const int64_t kk = k0 + 64 * wj + 32 * tj + li;
        if (nn < n_out && kk < k) dw[nn * k + kk] = acc[ti][tj][v];
      }
}

// ---------------------------------------------------------------------------
// Workspace path.  The kernels above decode the ternary codes (dX) and
// transpose and split the operands (dW) again for every output tile.  With a
// caller workspace this is done once per call:
//   ct  [k][np]     the codes C^T as BF16 (np = n_out rounded up to 64; zeros
//                   past n_out)
//   dyt [np][mp]    dY^T (mp = m_tok rounded up to 64; zeros past both ends)
//   xt  [3][k][mp]  the three BF16 parts of x_hat, transposed (zeros past m_tok)
// and the two gradients become plain BF16 contractions whose operands both
// have the contracted index contiguous:
//   dX[t][kk] = sum_n dy[t][n] ct[kk][n]               (A = dY, B = ct)
//   dW[n][kk] = sum_p sum_t dyt[n][t] xt[p][kk][t]      (A = dyt, B = xt)
// ---------------------------------------------------------------------------

// C^T of one tile of 64 output channels x one 64-weight block (grid: np / 64,
// k / 64).  Rows past n_out decode as code 0.
__global__ __launch_bounds__(256) void bwd_codes_t_kernel(PackedW W, int64_t np, uint16_t* __restrict__ ct) {
  __shared__ uint32_t F[4][64];                            // 2-bit fields of (quarter, channel)
  const int tid = threadIdx.x, nl = tid & 63, q = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64, row = n0 + nl;
  const int kb = (int)blockIdx.y;
  F[q][nl] = quarter_fields(W, row < W.n_out ? quarter_load(W, row, kb, q) : quarter_zero(), q);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int w = tid + 256 * i, e = w >> 3, rg = w & 7;  // feature 64 kb + e, channels n0 + 8 rg .. +7
    const int qq = e >> 4, sh = 2 * (e & 15);
    u32x4 d;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      d[j] = code_bf16((F[qq][8 * rg + 2 * j] >> sh) & 3u) | (code_bf16((F[qq][8 * rg + 2 * j + 1] >> sh) & 3u) << 16);
    *reinterpret_cast<u32x4*>(ct + ((int64_t)kb * 64 + e) * np + n0 + 8 * rg) = d;
  }
}

// dY^T of one 64-channel x 64-token tile (grid: np / 64, mp / 64)
__global__ __launch_bounds__(256) void bwd_dy_t_kernel(const uint16_t* __restrict__ dy, int64_t m_tok, int64_t n_out,
                                                       int64_t mp, uint16_t* __restrict__ dyt) {
  __shared__ __attribute__((aligned(16))) uint16_t T[64][kRow];   // [token][channel]
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64, t0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int w = tid + 256 * i, t = w >> 3, c = w & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t0 + t < m_tok && n0 + 8 * c < n_out) v = *reinterpret_cast<const u32x4*>(dy + (t0 + t) * n_out + n0 + 8 * c);
    *reinterpret_cast<u32x4*>(&T[t][8 * c]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int w = tid + 256 * i, nl = w >> 3, c = w & 7;  // channel n0 + nl, tokens t0 + 8 c .. +7
    u32x4 d;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = (uint32_t)T[8 * c + 2 * j][nl] | ((uint32_t)T[8 * c + 2 * j + 1][nl] << 16);
    *reinterpret_cast<u32x4*>(dyt + (n0 + nl) * mp + t0 + 8 * c) = d;
  }
}

// the three BF16 parts of x_hat, transposed, for one 64-feature x 64-token
// tile (grid: k / 64, mp / 64)
__global__ __launch_bounds__(256) void bwd_xhat_t_kernel(const int8_t* __restrict__ xq, const float* __restrict__ gamma,
                                                         int64_t m_tok, int64_t k, int64_t mp,
                                                         uint16_t* __restrict__ xt) {
  __shared__ __attribute__((aligned(16))) uint32_t S[3][64][kStep / 2 + 4];   // [part][token][feature pair]
  const int tid = threadIdx.x, t = tid >> 2, c = tid & 3;  // token t0 + t, features k0 + 16 c .. +15
  const int64_t k0 = (int64_t)blockIdx.x * 64, t0 = (int64_t)blockIdx.y * 64;
  u32x4 qv = {0u, 0u, 0u, 0u};
  float ge = 0.0f;
  if (t0 + t < m_tok) {
    qv = *reinterpret_cast<const u32x4*>(xq + (t0 + t) * k + k0 + 16 * c);
    ge = fmaxf(gamma[t0 + t], 1e-5f);
  }
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    uint16_t h[2][3];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qe = (int)(int8_t)(qv[(e + u) >> 2] >> (8 * ((e + u) & 3)));
      split3((ge * (float)qe) * (1.0f / 128.0f), h[u][0], h[u][1], h[u][2]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) S[p][t][8 * c + e / 2] = (uint32_t)h[0][p] | ((uint32_t)h[1][p] << 16);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int w = tid + 256 * i, p = w >> 9, f = (w >> 3) & 63, c8 = w & 7;   // part p, feature k0 + f, tokens t0 + 8 c8 ..
    const int sh = 16 * (f & 1);
    u32x4 d;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      d[j] = ((S[p][8 * c8 + 2 * j][f >> 1] >> sh) & 0xFFFFu) | (((S[p][8 * c8 + 2 * j + 1][f >> 1] >> sh) & 0xFFFFu) << 16);
    *reinterpret_cast<u32x4*>(xt + (int64_t)p * k * mp + (k0 + f) * mp + t0 + 8 * c8) = d;
  }
}

constexpr uint32_t kFarOff = 0x80000000u;   // a buffer offset past every buffer of this path: reads zeros

// One LDS stage of a WTI x WTJ block of 32 x 32 MFMA tiles per wave, against
// P parts of B (plane stride ps elements) that share each A operand.
template <int WTI, int WTJ, int P>
__device__ __forceinline__ void mma_block(const uint16_t* A_s, const uint16_t* B_s, int ps, f32x16 (&acc)[WTI][WTJ],
                                          int i_off, int j_off, int li, int g) {
#pragma unroll
  for (int s = 0; s < kStep / 16; ++s) {
    bf16x8 a[WTI];
#pragma unroll
    for (int t = 0; t < WTI; ++t) a[t] = lds_vec(A_s + (i_off + 32 * t + li) * kRow + 16 * s + 8 * g);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      bf16x8 b[WTJ];
#pragma unroll
      for (int t = 0; t < WTJ; ++t) b[t] = lds_vec(B_s + p * ps + (j_off + 32 * t + li) * kRow + 16 * s + 8 * g);
#pragma unroll
      for (int ti = 0; ti < WTI; ++ti)
#pragma unroll
        for (int tj = 0; tj < WTJ; ++tj)
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
    }
  }
}

// Operands of a contraction D[i][j] = sum_p sum_l A[i][l] B[p][j][l]: rows of
// A are i < ni (pitch lda; l < la_valid, a multiple of 8, else zero), rows of
// B are j < nj (pitch ldb, parts plane elements apart); the contracted length
// L is a multiple of 64 and B holds zeros wherever A's l is invalid.
struct BwdGemm {
  const uint16_t* a;
  int64_t ni, lda, la_valid;
  const uint16_t* b;
  int64_t nj, ldb, plane;
  int64_t L;
  // epilogue: dX (EPI 0) or dW (EPI 1)
  const float* beta;
  const float* x;
  const float* gamma;
  float* out;
  int64_t m_tok, k;
};

// 64 TI WTI x 64 WTJ output tiles per workgroup of 4 TI waves (2 TI along i x
// 2 along j, each a WTI x WTJ block of 32 x 32 MFMA tiles), 64 of the
// contracted index per LDS stage, the global loads of
// the next D stages in flight in registers.  NB = 2 LDS buffers: a stage's
// operands are written to one while the MFMAs read the other (one barrier per
// stage); NB = 1: one buffer, refilled between two barriers, which halves the
// LDS and lets two workgroups share a CU.  P parts of B share each A operand.
// Tile order: the grid is 1-D over gx x gy tiles (gx along j).  Workgroup b
// runs on XCD b % 8, and each XCD takes a contiguous run of tile numbers;
// tile numbers walk groups of gm rows of tiles column by column, so that the
// workgroups an XCD runs at once share both A and B tiles in its L2.
template <int P, int TI, int EPI, int D, int NB, int WTI, int WTJ>
__global__ __launch_bounds__(kBT * TI) void bwd_gemm_kernel(const BwdGemm o, int gx, int gy, int gm) {
  constexpr int kThr = kBT * TI, kTI = 64 * TI * WTI, kTJ = 64 * WTJ;
  constexpr int kAPer = kTI * 8 / kThr;                    // A pieces per thread
  constexpr int kBPer = kTJ * 8 / kThr;                    // B pieces per thread and part
  __shared__ __attribute__((aligned(16))) uint16_t A_s[NB][kTI * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t B_s[NB][P][kTJ * kRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int wi = wave >> 1, wj = wave & 1;
  const int nwg = (int)gridDim.x, xcd = (int)blockIdx.x & 7, per = nwg >> 3, rem = nwg & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + ((int)blockIdx.x >> 3);
  const int grp = t / (gm * gx), rr = t - grp * gm * gx;
  const int rows = gy - grp * gm < gm ? gy - grp * gm : gm;
  const int64_t i0 = (int64_t)(grp * gm + rr % rows) * kTI, j0 = (int64_t)(rr / rows) * kTJ;
  f32x16 acc[WTI][WTJ] = {};
  // Buffer loads without branches (a load under a branch makes the compiler
  // drain every load in flight before using any of them, which serialised
  // the stages): resources over this tile's rows, so that rows past the end
  // read zeros; pieces past A's valid l take an offset past every buffer.
  // piece w of a tile (A or B) = row w / 8, l = 8 (w % 8) .. +7 of the stage;
  // thread t holds pieces t, t + kThr, ...
  const int64_t a_rows = o.ni - i0 < kTI ? o.ni - i0 : kTI;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(o.a + i0 * o.lda, a_rows * o.lda * 2);
  uint32_t voa[kAPer];
#pragma unroll
  for (int h = 0; h < kAPer; ++h) {
    const int w = tid + kThr * h;
    voa[h] = (uint32_t)((w >> 3) * o.lda + 8 * (w & 7)) * 2u;
  }
  const int64_t b_rows = o.nj - j0 < kTJ ? o.nj - j0 : kTJ;
  __amdgpu_buffer_rsrc_t rsb[P];
#pragma unroll
  for (int p = 0; p < P; ++p) rsb[p] = make_rsrc(o.b + p * o.plane + j0 * o.ldb, b_rows * o.ldb * 2);
  uint32_t vob[kBPer];
#pragma unroll
  for (int h = 0; h < kBPer; ++h) {
    const int w = tid + kThr * h;
    vob[h] = (uint32_t)((w >> 3) * o.ldb + 8 * (w & 7)) * 2u;
  }
  u32x4 ra[D][kAPer], rb[D][P][kBPer];
  auto load_stage = [&](int64_t l0, int slot) {
#pragma unroll
    for (int h = 0; h < kAPer; ++h) {
      const bool ok = l0 + 8 * ((tid + kThr * h) & 7) < o.la_valid;
      ra[slot][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rsa, ok ? voa[h] + (uint32_t)l0 * 2u : kFarOff, 0, 0));
    }
#pragma unroll
    for (int h = 0; h < kBPer; ++h)
#pragma unroll
      for (int p = 0; p < P; ++p)
        rb[slot][p][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rsb[p], vob[h] + (uint32_t)l0 * 2u, 0, 0));
  };
  auto write_stage = [&](int buf, int slot) {
#pragma unroll
    for (int h = 0; h < kAPer; ++h) {
      const int w = tid + kThr * h;
      *reinterpret_cast<u32x4*>(A_s[buf] + (w >> 3) * kRow + 8 * (w & 7)) = ra[slot][h];
    }
#pragma unroll
    for (int h = 0; h < kBPer; ++h) {
      const int w = tid + kThr * h;
#pragma unroll
      for (int p = 0; p < P; ++p)
        *reinterpret_cast<u32x4*>(B_s[buf][p] + (w >> 3) * kRow + 8 * (w & 7)) = rb[slot][p][h];
    }
  };
  const int nst = (int)(o.L / kStep);
  // Stage s travels in register set s % D; stage 0 goes to LDS first.  Loads
  // of stages past the end read zeros or bytes nobody uses (buffer loads stay
  // in bounds), so the refills need no branch.
#pragma unroll
  for (int s = 0; s < D; ++s) load_stage((int64_t)s * kStep, s);
  write_stage(0, 0);
  load_stage((int64_t)D * kStep, 0);
  lds_barrier();
  // one stage: u = st mod D fixes the register set of stage st + 1
  auto step = [&](int st, int u, bool last) {
    const int buf = NB == 2 ? st & 1 : 0;
    if (NB == 2 && !last) {
      write_stage(buf ^ 1, (u + 1) % D);                   // stage st + 1; its buffer's readers passed the barrier
      load_stage((int64_t)(st + 1 + D) * kStep, (u + 1) % D);
    }
    mma_block<WTI, WTJ, P>(A_s[buf], B_s[buf][0], kTJ * kRow, acc, 32 * WTI * wi, 32 * WTJ * wj, li, g);
    lds_barrier();
    if (NB == 1 && !last) {                                // one buffer: refill it once every wave has read it
      write_stage(0, (u + 1) % D);
      load_stage((int64_t)(st + 1 + D) * kStep, (u + 1) % D);
      lds_barrier();
    }
  };
  // main loop: every stage has a successor; then the last ones
  int st0 = 0;
  for (; st0 + D < nst; st0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(st0 + u, u, false);
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (st0 + u < nst) step(st0 + u, u, st0 + u + 1 == nst);
  // lane (li, g) holds D[8 (v / 4) + 4 g + v % 4][li] of each 32 x 32 tile
  const float b = EPI == 0 ? fmaxf(o.beta[0], 1e-5f) : 0.0f;
#pragma unroll
  for (int ti = 0; ti < WTI; ++ti)
#pragma unroll
    for (int tj = 0; tj < WTJ; ++tj)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + 32 * WTI * wi + 32 * ti + 8 * (v >> 2) + 4 * g + (v & 3);
        const int64_t j = j0 + 32 * WTJ * wj + 32 * tj + li;
        if (i < o.ni && j < o.nj) {
          if constexpr (EPI == 0) {                        // i = token, j = feature
            const float s = fmaxf(o.gamma[i], 1e-5f) * (1.0f / 128.0f);   // exact power-of-two scaling
            const float r = rintf(o.x[i * o.k + j] / s);                 // the forward's fp32 quotient
            o.out[i * o.k + j] = fabsf(r) <= 127.0f ? b * acc[ti][tj][v] : 0.0f;
          } else {                                         // i = output channel, j = feature
            o.out[i * o.k + j] = acc[ti][tj][v];
          }
        }
      }
}

// Register stages of loads, LDS buffers, token tiles per dX workgroup, MFMA
// tiles per wave and row groups of the tile order.  Measured on the 3B-class
// gate and down matrices at 2048 tokens (and the 13B-class ones at 4096):
// what pays is two independent workgroups per CU, whose barrier phases
// interleave (dW 488-496 us with one buffer against 580-592 us with two, at
// one workgroup per CU); deeper register stages and the grouped tile order
// changed dX by less than 2%; 4 x 2 or 2 x 4 MFMA tiles per wave (over 256
// VGPRs: one workgroup per CU) were 10-50% slower.
constexpr int kDxStages = 2, kDwStages = 1, kDxGroup = 4, kDwGroup = 8, kDxBuffers = 1, kDwBuffers = 1, kDxTI = 1,
              kDwTI = 1, kDxWTI = 2, kDxWTJ = 2, kDwWTI = 2, kDwWTJ = 2;

__host__ __device__ constexpr int64_t round64(int64_t v) { return (v + 63) / 64 * 64; }
constexpr int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

}  // namespace

int64_t backward_ws_bytes(int64_t m_tok, int64_t n_out, int64_t k) {
  const int64_t np = round64(n_out), mp = round64(m_tok);
  return align256(k * np * 2) + align256(np * mp * 2) + align256(3 * k * mp * 2);
}

hipError_t launch_backward_ws(const BackwardArgs& a, void* ws, hipStream_t s) {
  const int64_t np = round64(a.n_out), mp = round64(a.m_tok);
  // the contraction's buffer resources span up to 256 rows of np or mp BF16
  // values (32-bit sizes); beyond that the tile kernels need no workspace
  if (256 * 2 * (np > mp ? np : mp) >= ((int64_t)1 << 31)) return launch_backward(a, s);
  uint8_t* p = static_cast<uint8_t*>(ws);
  uint16_t* ct = reinterpret_cast<uint16_t*>(p);
  uint16_t* dyt = reinterpret_cast<uint16_t*>(p + align256(a.k * np * 2));
  uint16_t* xt = reinterpret_cast<uint16_t*>(p + align256(a.k * np * 2) + align256(np * mp * 2));
  if (a.dx) {
    PackedW W{a.packed, a.meta, a.n_out, (int32_t)(a.k / 64), a.fmt, a.n, a.m};
    hipLaunchKernelGGL(bwd_codes_t_kernel, dim3((unsigned)(np / 64), (unsigned)(a.k / 64)), dim3(256), 0, s, W, np, ct);
    BwdGemm o = {};
    o.a = a.dy; o.ni = a.m_tok; o.lda = a.n_out; o.la_valid = a.n_out;
    o.b = ct; o.nj = a.k; o.ldb = np; o.plane = 0; o.L = np;
    o.beta = a.beta; o.x = a.x; o.gamma = a.gamma; o.out = a.dx; o.m_tok = a.m_tok; o.k = a.k;
    constexpr int kTI = kDxTI, kRi = 64 * kTI * kDxWTI, kRj = 64 * kDxWTJ;
    const int gx = (int)((a.k + kRj - 1) / kRj), gy = (int)((a.m_tok + kRi - 1) / kRi);
    if ((int64_t)gx * gy * kBT * kTI >= ((int64_t)1 << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_gemm_kernel<1, kTI, 0, kDxStages, kDxBuffers, kDxWTI, kDxWTJ>), dim3((unsigned)(gx * gy)),
                       dim3(kBT * kTI), 0, s, o, gx, gy, kDxGroup);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dw) {
    hipLaunchKernelGGL(bwd_dy_t_kernel, dim3((unsigned)(np / 64), (unsigned)(mp / 64)), dim3(256), 0, s, a.dy, a.m_tok,
                       a.n_out, mp, dyt);
    hipLaunchKernelGGL(bwd_xhat_t_kernel, dim3((unsigned)(a.k / 64), (unsigned)(mp / 64)), dim3(256), 0, s, a.xq,
                       a.gamma, a.m_tok, a.k, mp, xt);
    BwdGemm o = {};
    o.a = dyt; o.ni = a.n_out; o.lda = mp; o.la_valid = mp;
    o.b = xt; o.nj = a.k; o.ldb = mp; o.plane = a.k * mp; o.L = mp;
    o.out = a.dw; o.m_tok = a.m_tok; o.k = a.k;
    constexpr int kTI = kDwTI, kRi = 64 * kTI * kDwWTI, kRj = 64 * kDwWTJ;
    const int gx = (int)((a.k + kRj - 1) / kRj), gy = (int)((a.n_out + kRi - 1) / kRi);
    if ((int64_t)gx * gy * kBT * kTI >= ((int64_t)1 << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_gemm_kernel<3, kTI, 1, kDwStages, kDwBuffers, kDwWTI, kDwWTJ>), dim3((unsigned)(gx * gy)),
                       dim3(kBT * kTI), 0, s, o, gx, gy, kDwGroup);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.dx) {
    PackedW W{a.packed, a.meta, a.n_out, (int32_t)(a.k / 64), a.fmt, a.n, a.m};
    constexpr int kTW = kDxTW;
    const dim3 grid((unsigned)((a.k + kTile - 1) / kTile), (unsigned)((a.m_tok + kTile * kTW - 1) / (kTile * kTW)));
    hipLaunchKernelGGL((backward_dx_kernel<kTW>), grid, dim3(kBT * kTW), 0, s, a.dy, a.m_tok, a.n_out, a.k, W, a.beta,
                       a.x, a.gamma, a.dx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dw) {
    constexpr int kNW = kDwNW;
    const dim3 grid((unsigned)((a.k + kTile - 1) / kTile), (unsigned)((a.n_out + kTile * kNW - 1) / (kTile * kNW)));
    hipLaunchKernelGGL((backward_dw_kernel<kNW>), grid, dim3(kBT * kNW), 0, s, a.dy, a.m_tok, a.n_out, a.k, a.xq,
                       a.gamma, a.dw);
  }
  return hipGetLastError();
}

}  // namespace sbl
