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
// three MFMA per step.  One 128 x 128 output tile per workgroup of 4 waves
// (each 64 x 64: 2 x 2 MFMA tiles), 64 of the contracted index per LDS stage.
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

constexpr uint16_t kOne = 0x3F80u, kMinusOne = 0xBF80u;   // BF16 1.0, -1.0

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

// 16 ternary codes of row `row`, weights 16 qq .. 16 qq + 15 of 64-weight block kb,
// as u = c + 1 in 2-bit fields (field e = weight 16 qq + e)
struct PackedW {
  const uint8_t* packed;
  const uint8_t* meta;
  int64_t n_out;
  int32_t nkb, fmt, n, m;
};

__device__ __forceinline__ uint32_t quarter_fields(const PackedW& W, int64_t row, int kb, int qq) {
  if (W.fmt == 0) {
    // DENSE2 block word qq holds weights 16 qq .. +15: weight 16 qq + e at bit 8 (e % 4) + 2 (e / 4)
    const uint32_t w = *reinterpret_cast<const uint32_t*>(W.packed + panel_offset(W.n_out, W.nkb, 16, row, kb) + 4 * qq);
    uint32_t f = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) f |= ((w >> (8 * (e & 3) + 2 * (e >> 2))) & 3u) << (2 * e);
    return f;
  }
  // N:M: the kept weights of the block, in ascending order, hold consecutive
  // 2-bit codes; exactly n per group of m, so the quarter's first kept weight
  // is number 16 qq n / m, and its codes take at most 32 bits from bit
  // s = 32 qq n / m on: three halfwords (those inside the block) hold them
  const int bb = 16 * W.n / W.m;                           // code bytes per block (even)
  const uint16_t* cp = reinterpret_cast<const uint16_t*>(W.packed + panel_offset(W.n_out, W.nkb, bb, row, kb));
  const uint2 mv = *reinterpret_cast<const uint2*>(W.meta + panel_offset(W.n_out, W.nkb, 8, row, kb));
  const uint32_t keep = (uint32_t)(((uint64_t)mv.x | ((uint64_t)mv.y << 32)) >> (16 * qq)) & 0xFFFFu;
  const int s0 = 32 * qq * W.n / W.m, h0 = s0 >> 4;
  uint64_t win = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (h0 + j < bb / 2) win |= (uint64_t)cp[h0 + j] << (16 * j);
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

__global__ __launch_bounds__(kBT) void backward_dx_kernel(const uint16_t* __restrict__ dy, int64_t m_tok, int64_t n_out,
                                                          int64_t k, PackedW W, const float* __restrict__ beta,
                                                          const float* __restrict__ x, const float* __restrict__ gamma,
                                                          float* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) uint16_t A_s[kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t B_s[kTile * kRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * kTile, k0 = (int64_t)blockIdx.x * kTile;
  f32x16 acc[2][2] = {};
  for (int64_t n0 = 0; n0 < n_out; n0 += kStep) {
    __syncthreads();                                       // the previous stage has been read
    {  // A: dY[t0 + r][n0 .. n0 + 63], four 16-byte pieces per thread (n_out % 8 == 0)
      const int r = tid >> 1, h = tid & 1;
      const int64_t t = t0 + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t nn = n0 + 32 * h + 8 * v;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (t < m_tok && nn < n_out) val = *reinterpret_cast<const u32x4*>(dy + t * n_out + nn);
        *reinterpret_cast<u32x4*>(A_s + r * kRow + 32 * h + 8 * v) = val;
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // B: C[n0 + nl][k0 + 64 bb + 16 qq + e] -> B_s[64 bb + 16 qq + e][nl]
      const int nl = 32 * half + (tid >> 3), bb = (tid >> 2) & 1, qq = tid & 3;
      const int64_t row = n0 + nl;
      const int kb = (int)(k0 / 64) + bb;
      uint32_t f = 0x55555555u;                            // u = 1 everywhere: code 0
      if (row < n_out && kb < W.nkb) f = quarter_fields(W, row, kb, qq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t u = (f >> (2 * e)) & 3u;
        B_s[(64 * bb + 16 * qq + e) * kRow + nl] = u == 2u ? kOne : (u == 0u ? kMinusOne : (uint16_t)0);
      }
    }
    __syncthreads();
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

__global__ __launch_bounds__(kBT) void backward_dw_kernel(const uint16_t* __restrict__ dy, int64_t m_tok, int64_t n_out,
                                                          int64_t k, const int8_t* __restrict__ xq,
                                                          const float* __restrict__ gamma, float* __restrict__ dw) {
  __shared__ __attribute__((aligned(16))) uint16_t A_s[kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t B_s[3][kTile * kRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kTile, k0 = (int64_t)blockIdx.x * kTile;
  f32x16 acc[2][2] = {};
  const int r = tid >> 2, c32 = 32 * (tid & 3);            // staging: token row r of the stage, 32 columns
  for (int64_t t0 = 0; t0 < m_tok; t0 += kStep) {
    __syncthreads();
    const int64_t t = t0 + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {  // A: dY[t][n0 + c32 + 8v .. +7] -> A_s[c32 + 8v + e][r]
      const int64_t nn = n0 + c32 + 8 * v;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (t < m_tok && nn < n_out) val = *reinterpret_cast<const u32x4*>(dy + t * n_out + nn);
#pragma unroll
      for (int e = 0; e < 8; ++e) A_s[(c32 + 8 * v + e) * kRow + r] = (uint16_t)(val[e >> 1] >> (16 * (e & 1)));
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {  // B: x_hat[t][k0 + c32 + 16v .. +15] in three parts -> B_s[p][..][r]
      const int c = c32 + 16 * v;
      u32x4 qv = {0u, 0u, 0u, 0u};
      float ge = 0.0f;
      if (t < m_tok && k0 + c < k) {
        qv = *reinterpret_cast<const u32x4*>(xq + t * k + k0 + c);
        ge = fmaxf(gamma[t], 1e-5f);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qe = (int)(int8_t)(qv[e >> 2] >> (8 * (e & 3)));
        const float xh = (ge * (float)qe) * (1.0f / 128.0f);
        uint16_t h1, h2, h3;
        split3(xh, h1, h2, h3);
        B_s[0][(c + e) * kRow + r] = h1;
        B_s[1][(c + e) * kRow + r] = h2;
        B_s[2][(c + e) * kRow + r] = h3;
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 3; ++p) mma_stage(A_s, B_s[p], acc, wi, wj, li, g);
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

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const dim3 block(kBT);
  if (a.dx) {
    PackedW W{a.packed, a.meta, a.n_out, (int32_t)(a.k / 64), a.fmt, a.n, a.m};
    const dim3 grid((unsigned)((a.k + kTile - 1) / kTile), (unsigned)((a.m_tok + kTile - 1) / kTile));
    hipLaunchKernelGGL(backward_dx_kernel, grid, block, 0, s, a.dy, a.m_tok, a.n_out, a.k, W, a.beta, a.x, a.gamma,
                       a.dx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dw) {
    const dim3 grid((unsigned)((a.k + kTile - 1) / kTile), (unsigned)((a.n_out + kTile - 1) / kTile));
    hipLaunchKernelGGL(backward_dw_kernel, grid, block, 0, s, a.dy, a.m_tok, a.n_out, a.k, a.xq, a.gamma, a.dw);
  }
  return hipGetLastError();
}

}  // namespace sbl
