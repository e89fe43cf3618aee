// Prefill GEMM of the BitLinear product (bitnet.cpp article "Fundamento
// matematico" item 3) for N:M 2:4 weights on gfx950's sparse MFMA,
// v_smfmac_i32_16x16x128_i8: the A operand holds only the two kept values of
// every group of four along k plus a 2-bit position for each, which is the
// 2:4 structure the Sparse-BitNet pages run on sparse tensor cores (method
// section 2, "N:M Sparsity"; section 4 on the measured speedups); here the
// matrix cores skip the pruned half of the weights.
//
// Operand layout of v_smfmac_i32_16x16x128_i8 (16 rows x 16 tokens x 128 k),
// established on the device with one-hot operands:
//  * A (4 VGPRs): lane l holds row l%16, k = 32*(l/16) .. +31; byte 2i+s is
//    the s-th kept value of the four-group k = 32*(l/16) + 4i .. +3.
//  * index (1 VGPR): nibble i = p0 | p1 << 2, the positions (0..3) inside
//    four-group i of the values in bytes 2i and 2i+1.
//  * B (8 VGPRs): lane l holds token l%16; bytes 0-15 are k = 16*(l/16) ..
//    +15, bytes 16-31 are k = 64 + 16*(l/16) .. +15.
//  * D (4 VGPRs): lane l holds rows 4*(l/16) .. +3 of token l%16.
// The N:M 2:4 storage (kept codes in k order, 2 bits each; BITMAP metadata)
// gives both directly: a lane's 32 k of one row are 16 kept codes (one code
// dword) and 32 bitmap bits (one metadata dword).
//
// Tiling: a workgroup of 4 waves owns 4*16*KRT weight rows x 16*KCT tokens;
// wave w owns KRT 16-row tiles x all KCT token tiles, so a decoded A operand
// feeds KCT sparse MFMAs and a B operand read from LDS feeds KRT.  The k loop
// advances 128 k per step (one sparse MFMA per tile pair); activations go
// straight from memory into a kNS-stage LDS ring (buffer_load ... lds), the
// weight words into registers kNS - 1 steps ahead, and each step decodes the
// next step's A operands between its own MFMAs.
// K need only be a multiple of 64: the second half of a last half step reads
// zero activations, which add nothing.
// All integer work is exact; results are bit-identical to the other paths.
#include "sbl_decode.h"

namespace sbl {

namespace {

using namespace dec;

typedef int32_t v8i __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBK = 128;                  // k per step
constexpr uint32_t kFar = 0x80000000u;    // a buffer offset beyond every buffer: reads zeros

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// byte offset of 16-byte chunk c (0..7) of token row r in an LDS activation
// tile of 128-byte rows, XOR-swizzled by (r/2) % 8: 16 consecutive rows
// reading one chunk hit 16 distinct 16-byte groups of gfx950's 64 banks
__device__ __forceinline__ int bt_off(int r, int c) { return r * kBK + 16 * (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ int32_t lds_ld4(const uint8_t* p, int i) {
  return reinterpret_cast<const int32_t*>(p)[i];
}

// Four 2-bit codes u (bits 2i, 2i+1 of x's low byte) -> four int8 c = u - 1
// bytes: two shift-or-mask rounds put code i in byte i, then v_perm maps u in
// {0, 1, 2} to {0xFF, 0x00, 0x01}.
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  x &= 0xFFu;
  const uint32_t y = (x | (x << 12)) & 0x000F000Fu;
  const uint32_t z = (y | (y << 6)) & 0x03030303u;
  return __builtin_amdgcn_perm(0u, 0x000100FFu, z);
}

// Sparse-MFMA index from 32 bitmap bits (eight four-groups with exactly two
// bits set each): nibble i = p0 | p1 << 2 with p0 the lowest and p1 the
// highest set position of group i.  Per group, from its bits b0..b3:
// p0 bit 0 = b1 & ~b0, p0 bit 1 = ~(b0 | b1), p1 bit 0 = b3 | (b1 & ~b2 & ~b3),
// p1 bit 1 = b2 | b3.
__device__ __forceinline__ int sparse_index(uint32_t x) {
  constexpr uint32_t M = 0x11111111u;
  const uint32_t b1 = x >> 1, b2 = x >> 2, b3 = x >> 3;
  const uint32_t i0 = b1 & ~x & M;
  const uint32_t i1 = ~(x | b1) & M;
  const uint32_t i2 = (b3 | (b1 & ~(b2 | b3))) & M;
  const uint32_t i3 = (b2 | b3) & M;
  return (int)(i0 | (i1 << 1) | (i2 << 2) | (i3 << 3));
}

// 4 waves along the rows; KRT 16-row tiles and KCT 16-token tiles per wave.
template <int KRT, int KCT, bool GRP = false>
__global__ __launch_bounds__(kThreads, 2) void gemm24_kernel(const LinBatch batch) {
  constexpr int kBM = 4 * 16 * KRT;                 // weight rows per workgroup
  constexpr int kBN = 16 * KCT;                     // tokens per workgroup (every wave sees all)
  constexpr int kStage = kBN * kBK;                 // bytes of one activation stage
  constexpr int kNS = 4;                            // activation stages in LDS
  constexpr int kDma = kStage / (1024 * 4);         // 1 KB LDS-direct loads per wave per step
  constexpr int kNA = 2 * KRT;                      // weight loads per wave per step
  static_assert(kDma >= 1 && kBN % 32 == 0 && KRT <= KCT && kNS % 2 == 0, "shape");
  __shared__ __attribute__((aligned(16))) uint8_t btile[kNS][kStage];

  int di = 0;
  for (int i = 1; i < batch.count; ++i)
    if ((int)blockIdx.x >= batch.start[i]) di = i;
  const LinDesc& d = batch.d[di];
  const int lt = (int)blockIdx.x - batch.start[di];
  const int tile_n = lt % d.tiles_n, tile_t = lt / d.tiles_n;
  const int64_t n0 = (int64_t)tile_n * kBM;
  const int64_t t0 = (int64_t)tile_t * kBN;
  const int64_t K = d.k;
  const int nks = (int)((K + kBK - 1) / kBK);      // steps; the last may be half (K % 128 == 64)
  const int nkb = (int)(K / 64);                    // 64-weight blocks per row

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, g = lane >> 4;

  // activations: instruction q (= wave + 4p) of a step fills LDS rows 8q ..
  // 8q+7 (1 KB); its lane l lands at row 8q + l/8, 16-byte slot l%8, and
  // fetches chunk (l%8) ^ ((row/2) % 8) of that token's 128 bytes (bt_off's
  // swizzle; (row/2) % 8 = 4 (q % 2) + l/16, and q % 2 = wave % 2)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(d.xq, (int64_t)d.m_tok * K);
  const int dchunk = (lane & 7) ^ (((wave & 1) << 2) | (lane >> 4));
  uint32_t voff_b[kDma];
#pragma unroll
  for (int p = 0; p < kDma; ++p)
    voff_b[p] = (uint32_t)((t0 + 8 * (wave + 4 * p) + (lane >> 3)) * K + 16 * dchunk);
  auto dma_b = [&](int ks, int stage) {
    const bool ok = kBK * ks + 16 * dchunk < K;    // false past the last (half) step
#pragma unroll
    for (int p = 0; p < kDma; ++p)
      dma16(rx, &btile[stage][1024 * (wave + 4 * p)], ok ? voff_b[p] + (uint32_t)(kBK * ks) : kFar);
  };
  // weights: row tile rt of this wave = rows n0 + 16*(KRT*wave + rt) + lr.  Lane
  // group g takes block 2*ks + g/2, half g%2 (its 4-byte code and bitmap
  // words); codes and bitmap are both 8 bytes per block, panel-major
  // (panel_offset), so one offset serves both.
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.packed, d.n_out * nkb * (int64_t)8);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(d.meta, d.n_out * nkb * (int64_t)8);
  const int nfull = nkb / 4;                        // full panels
  const uint32_t nbl = (uint32_t)(nkb - 4 * nfull); // blocks of a last partial panel
  const uint32_t pb = 32u * (uint32_t)d.n_out;      // bytes per panel
  const uint32_t row0 = (uint32_t)(n0 + 16 * KRT * wave + lr);
  const uint32_t full0 = row0 * 32u, last0 = row0 * nbl * 8u;
  uint32_t wcode[kNS][KRT], wmeta[kNS][KRT];
  auto load_wall = [&](int ks, uint32_t* wc, uint32_t* wm) {
    const int kb = 2 * ks + (g >> 1);
    const int p = kb >> 2;
    const bool full = p < nfull;
    const uint32_t base = (uint32_t)p * pb + (full ? full0 : last0) + (uint32_t)(kb & 3) * 8u + 4u * (g & 1);
    const uint32_t rstep = full ? 16u * 32u : 16u * nbl * 8u;   // next row tile: 16 rows on
#pragma unroll
    for (int rt = 0; rt < KRT; ++rt) {
      const uint32_t off = kb < nkb ? base + (uint32_t)rt * rstep : kFar;
      wc[rt] = __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0);
      wm[rt] = __builtin_amdgcn_raw_buffer_load_b32(rm, off, 0, 0);
    }
  };

  v4i acc[KRT][KCT];
#pragma unroll
  for (int rt = 0; rt < KRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < KCT; ++ct) acc[rt][ct] = v4i{0, 0, 0, 0};

  // decoded A operands and indices, double-buffered by step parity
  v4i a[2][KRT];
  int ix[2][KRT];
  auto decode = [&](uint32_t cw, uint32_t mw, v4i& av, int& iv) {
    av = v4i{(int32_t)spread4(cw), (int32_t)spread4(cw >> 8), (int32_t)spread4(cw >> 16),
             (int32_t)spread4(cw >> 24)};
    iv = sparse_index(mw);
  };

  // prologue: steps 0 .. kNS-2 in flight (activations into LDS, weights into
  // registers), step 0's operands decoded
#pragma unroll
  for (int s = 0; s < kNS - 1; ++s) {
    dma_b(s, s);
    load_wall(s, wcode[s], wmeta[s]);
    __builtin_amdgcn_sched_barrier(0);              // the loop's issue order, step by step
  }
#pragma unroll
  for (int rt = 0; rt < KRT; ++rt) decode(wcode[0][rt], wmeta[0][rt], a[0][rt], ix[0][rt]);

  // one 128-k step; u = ks mod kNS fixes the LDS stage and the register slot.
  // Loads are unconditional (steps past the end read zeros), so the wait is an
  // exact count: the stage of step ks was issued kNS-1 steps ago, followed by
  // its weight loads and (kNS-2) later steps (the compiler itself waits for
  // the weight registers).
  constexpr int kWait = kNA + (kNS - 2) * (kDma + kNA);
  static_assert(kWait < 64, "vmcnt field");
  auto step = [&](const int ks, const int u) {
    __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("s_barrier" ::: "memory");         // every wave's part of stage u is in LDS,
    __builtin_amdgcn_sched_barrier(0);              // and stage u-1 has been read by all
    dma_b(ks + kNS - 1, (u + kNS - 1) % kNS);
    load_wall(ks + kNS - 1, wcode[(u + kNS - 1) % kNS], wmeta[(u + kNS - 1) % kNS]);
    const uint8_t* bt = &btile[u][0];
    // sub-step ct: token tile ct against every row tile with the operands
    // decoded one step earlier, while row tile ct (ct < KRT) of the next step
    // is decoded (about 31 VALU beside KRT MFMAs)
    const int c = u & 1, n = c ^ 1;
#pragma unroll
    for (int ct = 0; ct < KCT; ++ct) {
      const uint8_t* r0 = bt + bt_off(16 * ct + lr, g);
      const uint8_t* r1 = bt + bt_off(16 * ct + lr, 4 + g);
      const v8i b = v8i{lds_ld4(r0, 0), lds_ld4(r0, 1), lds_ld4(r0, 2), lds_ld4(r0, 3),
                        lds_ld4(r1, 0), lds_ld4(r1, 1), lds_ld4(r1, 2), lds_ld4(r1, 3)};
#pragma unroll
      for (int rt = 0; rt < KRT; ++rt)
        acc[rt][ct] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[c][rt], b, acc[rt][ct], ix[c][rt], 0, 0);
      if (ct < KRT) decode(wcode[(u + 1) % kNS][ct], wmeta[(u + 1) % kNS][ct], a[n][ct], ix[n][ct]);
#pragma unroll
      for (int m = 0; m < KRT; ++m) {                 // interleave: one MFMA, then a share of the decode
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int ks0 = 0;
  for (; ks0 + kNS <= nks; ks0 += kNS) {
#pragma unroll
    for (int u = 0; u < kNS; ++u) step(ks0 + u, u);
  }
#pragma unroll
  for (int u = 0; u < kNS - 1; ++u)
    if (ks0 + u < nks) step(ks0 + u, u);
  // every LDS-direct load has landed before the workgroup can leave
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // epilogue: lane (lr, g) holds rows 4g .. 4g+3 of token lr of each tile
#pragma unroll
  for (int ct = 0; ct < KCT; ++ct) {
    const int64_t t = t0 + 16 * ct + lr;
    if (t >= d.m_tok) continue;
    const float s = out_scale(d.beta, d.gamma, t);
    float* yrow = d.y + t * d.n_out;
    int32_t* arow = d.acc ? d.acc + t * d.n_out : nullptr;
#pragma unroll
    for (int rt = 0; rt < KRT; ++rt) {
      const int64_t row = n0 + 16 * (KRT * wave + rt) + 4 * g;
      int32_t a4[4];
      float y4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a4[j] = acc[rt][ct][j];
        if constexpr (GRP) {   // group scales: beta of each row (rows past n_out take the last row's)
          const int64_t rj = row + j < d.n_out ? row + j : d.n_out - 1;
          y4[j] = (float)a4[j] * out_scale_g(row_beta(d.beta, d.beta_rows, rj), d.gamma[t]);
        } else {
          y4[j] = (float)a4[j] * s;
        }
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

template <int KRT, int KCT, bool GRP = false>
hipError_t launch24(const LinearArgs* items, int count, hipStream_t s) {
  constexpr int kBM = 4 * 16 * KRT, kBN = 16 * KCT;
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
  hipLaunchKernelGGL((gemm24_kernel<KRT, KCT, GRP>), dim3((unsigned)blocks), dim3(kThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm24_group(const LinearArgs* items, int count, hipStream_t s) {
  if (items[0].beta_rows > 0) return launch24<4, 8, true>(items, count, s);   // group scales
  return launch24<4, 8>(items, count, s);
}

}  // namespace sbl
