// Prefill / training-forward GEMM of the BitLinear product (bitnet.cpp article
// "Fundamento matematico" item 3, y = W~ x~ beta gamma / Qb) for token counts
// above the decode range: at thousands of tokens the ternary x int8 product
// is a dense contraction, so it runs on gfx950 int8 MFMA
// (v_mfma_i32_32x32x32_i8, 32 rows x 32 tokens x 32 k per instruction).
//
// Tiling: a workgroup (4 waves) owns 256 weight rows x 128 tokens; wave
// (wn, wt) owns rows 128*wn .. +128 (4 MFMA row tiles) x tokens 64*wt .. +64
// (2 column tiles).  Per 128-k step:
//  * activations: the workgroup stages a 128 token x 128 byte int8 tile in
//    LDS (double-buffered, rows padded to 144 bytes so the 16-byte operand
//    reads of 8 consecutive tokens hit distinct banks); each B operand read
//    feeds 4 MFMAs (one per row tile);
//  * weights: every lane loads its packed bytes straight from global memory
//    (16 bytes of DENSE2 = 64 weights per row tile) and decodes them into A
//    operands in registers (7 VALU ops per 16 weights; N:M via LDS tables +
//    v_perm), one k-step ahead of use.
// DENSE2 feeds u = c + 1 to the MFMA and subtracts sum_k q per token at the
// end (the sums come from v_dot4 on the B operands); N:M decodes to c.
// All integer work is exact; results are bit-identical to the GEMV path.
#include "sbl_decode.h"

namespace sbl {

namespace {

using namespace dec;

typedef int32_t v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;            // weight rows per workgroup
constexpr int kBN = 128;            // tokens per workgroup
constexpr int kBK = 128;            // k per step
constexpr int kStride = kBK + 16;   // LDS bytes per token row
constexpr int kThreads = 256;
constexpr int kRT = 4;              // 32-row tiles per wave
constexpr int kCT = 2;              // 32-token tiles per wave

__device__ __forceinline__ void lds_st16(uint8_t* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ v4i lds_ld16(const uint8_t* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return v4i{(int32_t)v[0], (int32_t)v[1], (int32_t)v[2], (int32_t)v[3]};
}

template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const LinBatch batch) {
  __shared__ NmLut lut;
  __shared__ __attribute__((aligned(16))) uint8_t btile[2][kBN * kStride];
  if (KIND != kDense2) build_lut<KIND>(lut);

  int di = 0;
  for (int i = 1; i < batch.count; ++i)
    if ((int)blockIdx.x >= batch.start[i]) di = i;
  const LinDesc& d = batch.d[di];
  const int lt = (int)blockIdx.x - batch.start[di];
  const int tile_n = lt % d.tiles_n, tile_t = lt / d.tiles_n;
  const int64_t n0 = (int64_t)tile_n * kBM;
  const int64_t t0 = (int64_t)tile_t * kBN;
  const int64_t K = d.k;
  const int nks = (int)((K + kBK - 1) / kBK);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave & 1, wt = wave >> 1;
  const int li = lane & 31, g = lane >> 5;

  // activation staging: thread -> token (tid >> 3) + 32p, 16-byte chunk tid & 7
  const int st_tok = tid >> 3, st_chunk = tid & 7;
  auto load_b = [&](int ks, u32x4* r) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t tok = t0 + st_tok + 32 * p;
      const int64_t kk = (int64_t)ks * kBK + 16 * st_chunk;
      r[p] = (tok < d.m_tok && kk < K) ? ld16(d.xq + tok * K + kk) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_b = [&](int buf, const u32x4* r) {
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_st16(&btile[buf][(st_tok + 32 * p) * kStride + 16 * st_chunk], r[p]);
  };
  // weights: lane (li, g) of row tile rt covers k = ks*128 + 64g .. +64 of row n0 + 128wn + 32rt + li
  auto load_w = [&](int ks, ARaw<KIND>* a) {
    const int kb = 2 * ks + g;                       // 64-weight block index within the row
    const bool kok = (int64_t)kb * 64 < K;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int64_t row = n0 + 128 * wn + 32 * rt + li;
      load_a<KIND>(a[rt], d, row, kb, kok && row < d.n_out);
    }
  };

  v16i acc[kRT][kCT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[rt][ct] = v16i{};
  int qs[kCT] = {0, 0};

  ARaw<KIND> wcur[kRT], wnxt[kRT];
  u32x4 bst[4];
  load_b(0, bst);
  load_w(0, wcur);
  store_b(0, bst);
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {
      load_b(ks + 1, bst);
      load_w(ks + 1, wnxt);
    }
    const uint8_t* bt = &btile[buf][0];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {               // 32-k MFMA sub-steps
      v4i b[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
        b[ct] = lds_ld16(bt + (64 * wt + 32 * ct + li) * kStride + 64 * g + 16 * kk);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const v4i a = decode_a<KIND>(wcur[rt], kk, lut);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[ct], acc[rt][ct], 0, 0, 0);
      }
      if (KIND == kDense2) {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) qs[ct] = __builtin_amdgcn_sdot4(b[ct][j], 0x01010101, qs[ct], false);
      }
    }
    if (more) {
      store_b(buf ^ 1, bst);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) wcur[rt] = wnxt[rt];
    }
    __syncthreads();
  }

  // epilogue: lane (li, g) holds C[8*(v/4) + 4g + v%4][li] of each 32x32 tile
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    if (KIND == kDense2) qs[ct] += __shfl_xor(qs[ct], 32, 64);
    const int64_t t = t0 + 64 * wt + 32 * ct + li;
    if (t >= d.m_tok) continue;
    const float s = out_scale(d.beta, d.gamma, t);
    float* yrow = d.y + t * d.n_out;
    int32_t* arow = d.acc ? d.acc + t * d.n_out : nullptr;
    const int32_t corr = KIND == kDense2 ? qs[ct] : 0;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = n0 + 128 * wn + 32 * rt + 8 * q + 4 * g;
        int32_t a4[4];
        float y4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a4[j] = acc[rt][ct][4 * q + j] - corr;
          y4[j] = (float)a4[j] * s;
        }
        if (row + 3 < d.n_out && ((t * d.n_out + row) & 3) == 0) {
          *reinterpret_cast<float4*>(yrow + row) = make_float4(y4[0], y4[1], y4[2], y4[3]);
          if (arow) *reinterpret_cast<int4*>(arow + row) = make_int4(a4[0], a4[1], a4[2], a4[3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (row + j < d.n_out) {
              yrow[row + j] = y4[j];
              if (arow) arow[row + j] = a4[j];
            }
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_group(const LinearArgs* items, int count, int kind, hipStream_t s) {
  LinBatch b = {};
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    b.d[i] = to_desc(items[i]);
    b.d[i].tiles_n = (int32_t)((items[i].n_out + kBM - 1) / kBM);
    b.start[i] = blocks;
    blocks += b.d[i].tiles_n * (int)((items[i].m_tok + kBN - 1) / kBN);
  }
  b.start[count] = blocks;
  b.count = count;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (kind == kDense2) hipLaunchKernelGGL(gemm_kernel<kDense2>, grid, block, 0, s, b);
  else if (kind == kNm68) hipLaunchKernelGGL(gemm_kernel<kNm68>, grid, block, 0, s, b);
  else hipLaunchKernelGGL(gemm_kernel<kNm24>, grid, block, 0, s, b);
  return hipGetLastError();
}

}  // namespace sbl
