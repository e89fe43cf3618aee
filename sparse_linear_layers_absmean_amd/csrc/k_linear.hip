// Ternary x int8 product with fp32 rescale (BitLinear operation, bitnet.cpp
// article "Fundamento matematico" item 3: y = W~ x~ beta gamma / Qb; no bias
// per the BitNet spec).
//
// int8 MFMA formulation (gfx950 v_mfma_i32_16x16x64_i8): weights are the A
// operand (16 output rows x 64 k), activations the B operand (64 k x 16
// tokens).  A DENSE2 dword holds 16 weights as u = c + 1 in 2-bit fields;
// (dword >> 2s) & 0x03030303 yields four int8 lanes u(k0+4j+s), j = 0..3, so
// the 16 weights decode with 7 VALU ops into the A operand in a permuted
// k-order.  The activations are permuted the same way (a 4x4 byte transpose
// with v_perm), so the contraction over the 64 k-slots is unchanged:
//   sum_k u q = sum_k c q + sum_k q,   hence acc = MFMA result - sum_k q.
// The per-token sum of q comes from v_dot4 with 0x01010101 on the B operand.
// All integer steps are exact; int32 cannot overflow since |acc| <= 127 k < 2^24.
#include "sbl_internal.h"

namespace sbl {

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i transpose4x4(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3) {
  // out_s byte j = byte s of n_j
  const uint32_t x0 = __builtin_amdgcn_perm(n1, n0, 0x05010400u);
  const uint32_t x1 = __builtin_amdgcn_perm(n1, n0, 0x07030602u);
  const uint32_t y0 = __builtin_amdgcn_perm(n3, n2, 0x05010400u);
  const uint32_t y1 = __builtin_amdgcn_perm(n3, n2, 0x07030602u);
  v4i r;
  r[0] = (int32_t)__builtin_amdgcn_perm(y0, x0, 0x05040100u);
  r[1] = (int32_t)__builtin_amdgcn_perm(y0, x0, 0x07060302u);
  r[2] = (int32_t)__builtin_amdgcn_perm(y1, x1, 0x05040100u);
  r[3] = (int32_t)__builtin_amdgcn_perm(y1, x1, 0x07060302u);
  return r;
}

__device__ __forceinline__ v4i decode_dense2(uint32_t wd) {
  v4i a;
  a[0] = (int32_t)(wd & 0x03030303u);
  a[1] = (int32_t)((wd >> 2) & 0x03030303u);
  a[2] = (int32_t)((wd >> 4) & 0x03030303u);
  a[3] = (int32_t)((wd >> 6) & 0x03030303u);
  return a;
}

// 16 weights of row r at k0 .. k0+15 from the N:M format, as a DENSE2 dword
template <int M>
__device__ uint32_t nm_dword(const uint8_t* __restrict__ codes_row, const uint8_t* __restrict__ meta_row,
                             int n, int64_t k0) {
  uint32_t out = 0;
#pragma unroll
  for (int gi = 0; gi < 16 / M; ++gi) {
    const int64_t kg = k0 + gi * M;                 // first k of the group
    const int64_t G = kg / M;                       // group index within the row
    uint32_t bits = meta_row[kg >> 3];
    if (M == 4) bits = (bits >> (kg & 4)) & 0xFu;
    int64_t pos = 2 * G * n;                        // bit offset of the group's first code
    int kept = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      uint32_t u = 1u;
      if (((bits >> j) & 1u) && kept < n) {
        u = (codes_row[pos >> 3] >> (pos & 7)) & 3u;
        pos += 2;
        ++kept;
      }
      out |= u << (2 * (gi * M + j));
    }
  }
  return out;
}

template <int FMT, int M>
__global__ __launch_bounds__(256) void linear_mfma_kernel(const uint8_t* __restrict__ packed,
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
  const uint8_t* mrow = meta + (row_ok ? r : 0) * (k / 8);
  const int8_t* xrow = xq + (tok_ok ? t : 0) * k;
  v4i c = {0, 0, 0, 0};
  int qs = 0;
  for (int64_t kb = 0; kb < k; kb += 64) {
    const int64_t kk = kb + 16 * g;
    uint32_t wd = 0x55555555u;                      // u = 1 everywhere: code 0
    if (row_ok) {
      if (FMT == 0) wd = reinterpret_cast<const uint32_t*>(wrow)[kk >> 4];
      else wd = nm_dword<M>(wrow, mrow, n, kk);
    }
    uint4 nb = make_uint4(0, 0, 0, 0);
    if (tok_ok) nb = *reinterpret_cast<const uint4*>(xrow + kk);
    const v4i a = decode_dense2(wd);
    const v4i b = transpose4x4(nb.x, nb.y, nb.z, nb.w);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    qs = __builtin_amdgcn_sdot4(b[0], 0x01010101, qs, false);
    qs = __builtin_amdgcn_sdot4(b[1], 0x01010101, qs, false);
    qs = __builtin_amdgcn_sdot4(b[2], 0x01010101, qs, false);
    qs = __builtin_amdgcn_sdot4(b[3], 0x01010101, qs, false);
  }
  qs += __shfl_xor(qs, 16, 64);
  qs += __shfl_xor(qs, 32, 64);                     // sum of q over k for token t
  if (!tok_ok) return;
  const float bs = fmaxf(beta[0], 1e-5f);
  const float gs = fmaxf(gamma[t], 1e-5f);
  const float s = (bs * gs) * 0.0078125f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = row0 + 4 * g + v;            // C[4*(lane/16)+v][lane%16]
    if (row < n_out) {
      const int32_t a = c[v] - qs;
      y[t * n_out + row] = (float)a * s;
      if (acc_out) acc_out[t * n_out + row] = a;
    }
  }
}

}  // namespace

hipError_t launch_linear(const uint8_t* packed, const uint8_t* meta, int fmt, int n, int m,
                         const float* beta, const int8_t* xq, const float* gamma, int64_t m_tok,
                         int64_t n_out, int64_t k, float* y, int32_t* acc, hipStream_t s) {
  const dim3 grid((unsigned)((n_out + 63) / 64), (unsigned)((m_tok + 15) / 16)), block(256);
  if (fmt == 0)
    hipLaunchKernelGGL((linear_mfma_kernel<0, 8>), grid, block, 0, s, packed, meta, n, beta, xq, gamma, m_tok, n_out, k, y, acc);
  else if (m == 8)
    hipLaunchKernelGGL((linear_mfma_kernel<1, 8>), grid, block, 0, s, packed, meta, n, beta, xq, gamma, m_tok, n_out, k, y, acc);
  else
    hipLaunchKernelGGL((linear_mfma_kernel<1, 4>), grid, block, 0, s, packed, meta, n, beta, xq, gamma, m_tok, n_out, k, y, acc);
  return hipGetLastError();
}

}  // namespace sbl
