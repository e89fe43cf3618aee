// Ternary x int8 product with fp32 rescale (BitLinear operation, bitnet.cpp
// article "Fundamento matematico" item 3: y = W~ x~ beta gamma / Qb; no bias
// per the BitNet spec), decode-sized token counts (m_tok <= 16).
//
// int8 MFMA formulation (gfx950 v_mfma_i32_16x16x64_i8): weights are the A
// operand (16 output rows x 64 k), activations the B operand (64 k x 16
// tokens).  A lane holds 16 consecutive k of one row (A) or one token (B).
//  * Both formats feed the MFMA u = c + 1 bytes at every k position, so that
//    sum_k u q = sum_k c q + sum_k q: acc = MFMA(u, q) - MFMA(ones, q).  The
//    second MFMA runs on the matrix pipe, which the decode leaves mostly idle.
//  * DENSE2: one 16-weight word decodes with 7 VALU ops into four dwords of
//    u bytes (the word-transposed layout makes each dword one shift + mask).
//  * N:M 6:8 and 2:4: per 8 weights, the 2-bit kept codes spread into bytes
//    by shifts and masks, one LDS table read (indexed by the metadata bitmap
//    byte) gives two v_perm selectors, and two v_perm place the codes at
//    their k positions, with a pad byte u = 1 at the pruned ones.
// Work split: a workgroup owns TB 16-row tiles of one matrix and TB*ks waves;
// the ks waves of a tile split k.  ks and TB are chosen per launch so that the
// grid is about one round of resident waves (a partial second round would run
// at a fraction of the bandwidth).  When the token rows fit (m_tok*k <= 32 KB)
// the workgroup stages them in LDS once and reads MFMA B operands from there;
// otherwise B comes from global memory.
// Each wave keeps kDepth weight loads in flight.  All global loads are buffer
// loads: rows, k-blocks and tokens out of range read zeros, so there is no
// branch around a load.  Partial int32 tiles of the ks waves are summed
// through LDS, then rescaled.  Up to 8 independent matrices share one launch
// (grouped GEMV).  Everything integer is exact: |acc| <= 127 k < 2^24.
#include "sbl_actq.h"
#include "sbl_decode.h"

namespace sbl {

namespace {

using namespace dec;

constexpr int kMaxWaves = 16;          // waves per workgroup, at most
// waves per launch the k split aims for: 2 per SIMD on 1024 SIMDs.  Fewer,
// longer waves keep fewer requests in flight (the stream stays compact) and
// fewer workgroups repeat the per-workgroup set-up (token staging, fused
// quantization); measured against 1536-4096: best or within 2% everywhere,
// 70B block -4%, 3B block -13% to -18% with the quantization fused.
constexpr int kResidentWaves = 2048;
constexpr int kSmallLaunchWaves = 1536;
constexpr int kXLdsMax = 32 * 1024;    // token rows staged through registers into LDS up to this many bytes
constexpr int kXBigMax = 128 * 1024;   // ... and by LDS-direct loads up to this many (one workgroup per CU)
constexpr int kBigLdsAttr = 150 * 1024;  // dynamic LDS the LDS-direct mode may request
constexpr int64_t kXBigMinWeights = int64_t(128) << 20;   // weights per launch for the LDS-direct mode
constexpr int kXMinWaves = 4;          // XL launches have at least this many waves per workgroup
constexpr int kXFPer = 4;              // fused quantization: 16-value pieces of x per thread, at most

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

// Bytes of one 64-weight block in the packed stream of each kind
template <int KIND> constexpr uint32_t kBlockBytes = KIND == kDense2 ? 16u : (KIND == kNm68 ? 12u : 8u);

// Panel-major addressing of a lane's blocks (panel_offset): block 4p + g of
// row `row` sits at p * pb + row * (blocks in panel p) * b + g * b.  The lane
// keeps the row terms of full panels and of the last, partial one.
struct PanelLane {
  uint32_t pb_w, pb_m;          // bytes of one full panel: codes, metadata
  uint32_t full_w, full_m;      // row * 4 * b
  uint32_t last_w, last_m;      // row * (blocks in the last panel) * b
  int nfull;                    // full panels
};

// The weights are streamed once per call: nontemporal cache policy (bit "nt"
// of the buffer instruction).  Measured against the default policy on every
// block of the decode table: 0.7B 17.9 -> 15.8 us, 3B 23.7 -> 21.4 us, 70B
// 58.4 -> 55.4 us at one token (DENSE2), and 3-12% at 4-16 tokens and for N:M.
constexpr int kWNt = 2;

template <int KIND>
__device__ __forceinline__ void load_w(WStage& s, const Rsrc& rs, const PanelLane& pl, int p, int g, bool kok) {
  constexpr uint32_t bw = kBlockBytes<KIND>;
  const bool full = p < pl.nfull;
  const uint32_t ow = kok ? (uint32_t)p * pl.pb_w + (full ? pl.full_w : pl.last_w) + (uint32_t)g * bw : kFar;
  const uint32_t om = kok ? (uint32_t)p * pl.pb_m + (full ? pl.full_m : pl.last_m) + (uint32_t)g * 8u : kFar;
  if constexpr (KIND == kDense2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs.w, ow, 0, kWNt);
    s.a[0] = v[0]; s.a[1] = v[1]; s.a[2] = v[2]; s.a[3] = v[3];
  } else if constexpr (KIND == kNm68) {
    const auto c = __builtin_amdgcn_raw_buffer_load_b96(rs.w, ow, 0, kWNt);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rs.m, om, 0, kWNt);
    s.a[0] = c[0]; s.a[1] = c[1]; s.a[2] = c[2]; s.a[3] = m[0]; s.a[4] = m[1];
  } else {
    const auto c = __builtin_amdgcn_raw_buffer_load_b64(rs.w, ow, 0, kWNt);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rs.m, om, 0, kWNt);
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

// v_perm selectors of the N:M decode, per bitmap byte: output byte p takes
// the code byte of its rank among the kept positions, or a pad byte holding
// u = 1 (code 0) where p is pruned.  The code bytes sit in bytes 0..3 (and
// 4, 5 for 6:8) of the {hi, lo} source pair; the pad is byte 6 (6:8) or 4 (2:4).
template <int KIND>
__device__ void build_gemv_sel(uint32_t (*sel)[2]) {
  for (int x = threadIdx.x; x < 256; x += blockDim.x) {
    uint32_t s0 = 0, s1 = 0;
    int ra = 0, rb = 0;
    for (int p = 0; p < 8; ++p) {
      const bool kept = (x >> p) & 1;
      uint32_t v;
      if (KIND == kNm68) {
        v = 6u;
        if (kept && ra < 6) v = (uint32_t)ra++;
      } else {                                     // two 4-groups: codes 0,1 then 2,3
        v = 4u;
        if (p < 4) { if (kept && ra < 2) v = (uint32_t)ra++; }
        else { if (kept && rb < 2) v = (uint32_t)(2 + rb++); }
      }
      if (p < 4) s0 |= v << (8 * p);
      else s1 |= v << (8 * (p - 4));
    }
    sel[x][0] = s0;
    sel[x][1] = s1;
  }
}

// One k-block: c += sum u q over its 64 weights (and, if CK, ck += sum q), so
// that acc = c - sum_k q.  u = c + 1 everywhere: DENSE2 decodes it from the 2-bit
// words; N:M scatters the kept codes and pads the pruned positions with
// u = 1.  N:M: the selector reads of 8 (or, under register pressure, twice 4)
// groups go out first, the codes spread into bytes while they are in flight,
// then 2 v_perm per 8 weights.
template <int KIND, int HALVES, bool CK>
__device__ __forceinline__ void mac(const WStage& s, const u32x4 (&bq)[4], v4i& c, v4i& ck,
                                    const uint32_t (*sel)[2]) {
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  if constexpr (KIND == kDense2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i b = {(int32_t)bq[i][0], (int32_t)bq[i][1], (int32_t)bq[i][2], (int32_t)bq[i][3]};
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(dense2_quad(s.a[i]), b, c, 0, 0, 0);
      if constexpr (CK) ck = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, ck, 0, 0, 0);
    }
  } else {
    constexpr int MW = KIND == kNm68 ? 3 : 2;      // first metadata word in the stage
    constexpr int NB = 8 / HALVES;                 // groups of 8 weights per batch
#pragma unroll
    for (int hb = 0; hb < HALVES; ++hb) {
      uint32_t s0[NB], s1[NB], plo[NB], phi[NB];
#pragma unroll
      for (int gg = 0; gg < NB; ++gg) {
        const int G = hb * NB + gg;
        const uint32_t mb = (s.a[MW + (G >> 2)] >> (8 * (G & 3))) & 0xFFu;
        const uint2 v = *reinterpret_cast<const uint2*>(&sel[mb][0]);
        s0[gg] = v.x;
        s1[gg] = v.y;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gg = 0; gg < NB; ++gg) {
        const int G = hb * NB + gg;
        if constexpr (KIND == kNm68) {
          const uint64_t lo64 = (uint64_t)s.a[0] | ((uint64_t)s.a[1] << 32);
          const uint64_t hi64 = (uint64_t)s.a[1] | ((uint64_t)s.a[2] << 32);
          const uint32_t c12 = (12 * G + 12 <= 64) ? (uint32_t)(lo64 >> (12 * G)) : (uint32_t)(hi64 >> (12 * G - 32));
          plo[gg] = fields4_to_bytes(c12 & 0xFFu);
          const uint32_t h4 = (c12 >> 8) & 0xFu;
          phi[gg] = ((h4 | (h4 << 6)) & 0x0303u) | 0x00010000u;
        } else {
          plo[gg] = fields4_to_bytes((s.a[G >> 2] >> (8 * (G & 3))) & 0xFFu);
          phi[gg] = 0x01010101u;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ii = 0; ii < NB / 2; ++ii) {
        const int i = hb * (NB / 2) + ii;
        const v4i b = {(int32_t)bq[i][0], (int32_t)bq[i][1], (int32_t)bq[i][2], (int32_t)bq[i][3]};
        v4i u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gg = 2 * ii + h;
          u[2 * h] = (int32_t)__builtin_amdgcn_perm(phi[gg], plo[gg], s0[gg]);
          u[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(phi[gg], plo[gg], s1[gg]);
        }
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(u, b, c, 0, 0, 0);
        if constexpr (CK) ck = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, ck, 0, 0, 0);
      }
    }
  }
}

// LDS-direct load: lane l's 16 bytes at buffer offset voff land at lds + 16*l
// (zeros past the buffer); counted by vmcnt.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// k-block kb = 4*sb + lane/16: super-block sb covers 256 weights of every row.
// XLM: how the token rows reach LDS: 0 not at all (read from memory per
// k-block), 1 through registers, issued first (m_tok*k <= kXLdsMax), 2 by
// LDS-direct loads (m_tok*k <= kXBigMax, k a multiple of 1024).
template <int KIND, int XLM, int D, bool XF>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(const GemvLaunch L) {
  constexpr bool XL = XLM != 0;
  static_assert(!XF || XLM == 1, "the fused activation quantization stages through registers");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t sel[256][2];
  __shared__ int32_t qs[16];                          // XL: sum_k q per token
  __shared__ uint32_t gbits[16];                      // XF: gamma per token (fp32 bits)
  const LinBatch& batch = L.b;
  const int ks = L.ks;
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
  // buffers over the whole packed matrix (the host keeps them below 2^31 bytes)
  // and the activations.  Rows past n_out of a last tile read other rows'
  // bytes (or zeros past the end); their results are never stored.
  constexpr uint32_t bw = kBlockBytes<KIND>;
  Rsrc rs;
  rs.w = make_rsrc(d.packed, d.n_out * (int64_t)nkb * bw);
  rs.m = make_rsrc(KIND == kDense2 ? d.packed : d.meta, KIND == kDense2 ? 0 : d.n_out * (int64_t)nkb * 8);
  rs.x = make_rsrc(d.xq, (int64_t)d.m_tok * d.k);
  PanelLane pl;
  {
    const uint32_t row = (uint32_t)(row0 + r);
    const uint32_t nbl = (uint32_t)(nkb - 4 * (nkb / 4));          // blocks in a last partial panel
    pl.pb_w = 4u * bw * (uint32_t)d.n_out;
    pl.pb_m = 32u * (uint32_t)d.n_out;
    pl.full_w = row * 4u * bw;
    pl.full_m = row * 32u;
    pl.last_w = row * nbl * bw;
    pl.last_m = row * nbl * 8u;
    pl.nfull = nkb / 4;
  }
  // LDS: [token rows m_tok*k (XL)][64 zero bytes][reduction ks*tb*4*64 ints]
  // LDS token rows are padded by 16 bytes (row t at t*(k+16)): the 16 lanes
  // that read one k-block of 16 tokens then hit 16 distinct bank groups
  // (with rows k bytes apart, k a multiple of 256, they all hit the same
  // banks).  Byte o of the m_tok x k token rows sits at lds_x(o).
  const uint32_t xbytes = XL ? (uint32_t)(d.m_tok * d.k) : 0u;
  const uint32_t xpitch = (uint32_t)d.k + 16u;
  const uint32_t zero_off = XL ? (uint32_t)d.m_tok * xpitch : 0u;
  auto lds_x = [&](uint32_t o) { return o + 16u * (o / (uint32_t)d.k); };
  int32_t* red = reinterpret_cast<int32_t*>(smem + zero_off + 64);
  const bool r_ok = r < d.m_tok;
  const uint32_t ox = r_ok ? (XL ? (uint32_t)r * xpitch : (uint32_t)(r * d.k)) : (XL ? zero_off : kFar);

  // XL: the activation loads go out first, so that they return ahead of the
  // weight stages; each thread stages up to kXPer 16-byte pieces.
  // XF: the same pieces come as 16 fp32 values each (kXFPer per thread at most).
  constexpr int kXPer = XF ? kXFPer : kXLdsMax / (16 * 64 * kXMinWaves);
  u32x4 xv[XLM == 1 && !XF ? kXPer : 1];
  float4 xf4[XF ? kXPer : 1][4];
  const int nxl = XL ? (int)((xbytes + blockDim.x * 16u - 1) / (blockDim.x * 16u)) : 0;   // XLM 1: <= kXPer
  if constexpr (XF) {
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(d.x, (int64_t)xbytes * 4);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (i < nxl) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xf4[i][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rf, o < xbytes ? 4 * o + 16 * j : kFar, 0, 0));
      }
    }
    if (threadIdx.x < 16) { qs[threadIdx.x] = 0; gbits[threadIdx.x] = 0u; }
  } else if constexpr (XLM == 1) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (i < nxl)
        xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.x, o < xbytes ? o : kFar, 0, 0));
    }
    if (threadIdx.x < 16) qs[threadIdx.x] = 0;
  } else if constexpr (XLM == 2) {
    // piece i of thread t = bytes (t + i*blockDim)*16 .. +15; a wave's
    // instruction fills 1 KB of one token row in LDS (k is a multiple of 1024
    // in this mode)
    for (int i = 0; i < nxl; ++i) {
      const uint32_t blk = (uint32_t)(wave * 64 + i * (int)blockDim.x) * 16u;   // wave-uniform
      if (blk < xbytes) dma16(rs.x, smem + lds_x(blk), (threadIdx.x + i * blockDim.x) * 16u);
    }
    if (threadIdx.x < 16) qs[threadIdx.x] = 0;
  }
  WStage wa[D];
  u32x4 bring[XL ? 1 : D][4];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int kb = 4 * (sb0 + j) + g;
    const bool ok = j < nit && kb < nkb;
    load_w<KIND>(wa[j], rs, pl, sb0 + j, g, ok);
    if constexpr (!XL) load_x<false>(bring[j], rs, smem, ox, zero_off, kb, ok && r_ok);
  }
  if (KIND != kDense2) build_gemv_sel<KIND>(sel);
  if constexpr (XF) {
    // per-token absmax (bitnet.cpp article, "Fundamento matematico", item 2),
    // then the same quantization as the activation quantizer, staged into LDS
    if (threadIdx.x < 4) *reinterpret_cast<u32x4*>(smem + zero_off + 16 * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();                               // qs, gbits cleared
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (i < nxl && o < xbytes) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, actq::absmax4(xf4[i][j]));
        atomicMax(&gbits[o / (uint32_t)d.k], __float_as_uint(mx));   // order of non-negative floats = of their bits
      }
    }
    __syncthreads();                               // gamma per token
    const bool publish = blockIdx.x == 0 && d.xq_out != nullptr;
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (i < nxl && o < xbytes) {
        // the standalone quantizer's step (same bits)
        const actq::Step st = actq::make_step(__uint_as_float(gbits[o / (uint32_t)d.k]));
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = actq::q_word(xf4[i][j], st);
        *reinterpret_cast<u32x4*>(smem + lds_x(o)) = v;
        if (publish) *reinterpret_cast<u32x4*>(d.xq_out + o) = v;
        int q = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) q = __builtin_amdgcn_sdot4((int)v[w], 0x01010101, q, false);
        atomicAdd(&qs[o / (uint32_t)d.k], q);
      }
    }
    if (blockIdx.x == 0 && d.gamma_out != nullptr && threadIdx.x < (unsigned)d.m_tok)
      d.gamma_out[threadIdx.x] = __uint_as_float(gbits[threadIdx.x]);
    __syncthreads();                               // activations, sum q and the N:M tables
  } else if constexpr (XLM == 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this thread's LDS-direct pieces have landed
    if (threadIdx.x < 4) *reinterpret_cast<u32x4*>(smem + zero_off + 16 * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();                               // every piece, qs cleared
    for (int i = 0; i < nxl; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (o < xbytes) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + lds_x(o));
        int q = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) q = __builtin_amdgcn_sdot4((int)v[w], 0x01010101, q, false);
        atomicAdd(&qs[o / (uint32_t)d.k], q);
      }
    }
    __syncthreads();                               // sum q and the N:M tables
  } else if constexpr (XL) {
    if (threadIdx.x < 4) *reinterpret_cast<u32x4*>(smem + zero_off + 16 * threadIdx.x) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();                               // qs cleared
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const uint32_t o = (threadIdx.x + i * blockDim.x) * 16u;
      if (i < nxl && o < xbytes) {
        *reinterpret_cast<u32x4*>(smem + lds_x(o)) = xv[i];
        int q = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) q = __builtin_amdgcn_sdot4((int)xv[i][w], 0x01010101, q, false);
        atomicAdd(&qs[o / (uint32_t)d.k], q);
      }
    }
    __syncthreads();                               // activations, sum q and the N:M tables
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
      mac<KIND, XL ? 1 : 2, !XL>(wa[j], b, c, ck, sel);
      const int sb = sb0 + it + j + D;
      const int kb2 = 4 * sb + g;
      const bool ok = sb < sb1 && kb2 < nkb;
      load_w<KIND>(wa[j], rs, pl, sb, g, ok);
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
      mac<KIND, XL ? 1 : 2, !XL>(wa[j], b, c, ck, sel);
    }
  }
  if constexpr (!XL) {
#pragma unroll
    for (int v = 0; v < 4; ++v) c[v] -= ck[v];
  }
  // Partial tiles of the ks waves meet in LDS; wave s then finishes the output
  // rows 4*(lane/16) + v with v = s (mod ks): C[4*(lane/16)+v][lane%16], column = token.
  const int t = r;
  if (ks > 1) {
    int32_t* rw = red + (tw * ks) * 4 * 64;
#pragma unroll
    for (int v = 0; v < 4; ++v) rw[(slice * 4 + v) * 64 + lane] = c[v];
    __syncthreads();
    if (slice >= 4) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v % ks != slice) continue;
      int32_t part[kMaxWaves];
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w) part[w] = w < ks ? rw[(w * 4 + v) * 64 + lane] : 0;
      int32_t a = 0;
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w) a += part[w];
      c[v] = a;
    }
  }
  if (t >= d.m_tok || row0 >= d.n_out) return;
  const float gt = XF ? __uint_as_float(gbits[t]) : d.gamma[t];
  const float sc = out_scale_g(d.beta, gt);
  const int32_t qt = XL ? qs[t] : 0;
  const int64_t rbase = row0 + 4 * g;
  float* yrow = d.y + (int64_t)t * d.n_out;
  int32_t* arow = d.acc ? d.acc + (int64_t)t * d.n_out : nullptr;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = rbase + v;
    if ((ks == 1 || v % ks == slice) && row < d.n_out) {
      const int32_t a = c[v] - qt;
      const float sr = d.beta_rows > 0 ? out_scale_g(row_beta(d.beta, d.beta_rows, row), gt) : sc;
      yrow[row] = (float)a * sr;
      if (arow) arow[row] = a;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic path: any token count, any n:m.  One wave = 16 rows x 16 tokens over
// the whole k; weights decoded to natural-order int8 bytes per 16 k.
// ---------------------------------------------------------------------------

// 16 weights at offset k0 (a multiple of 16) of one 64-weight block, from the
// block's codes and bitmap bytes
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
                                                             int32_t* __restrict__ acc_out,
                                                             int32_t beta_rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int64_t tok0 = (int64_t)blockIdx.y * 16;
  const int64_t r = row0 + (lane & 15);
  const int64_t t = tok0 + (lane & 15);
  const int g = lane >> 4;
  const bool row_ok = r < n_out, tok_ok = t < m_tok;
  const int64_t nkb = k / 64, bw = FMT == 0 ? 16 : 16 * n / M;      // bytes per 64-weight block
  const int64_t rr = row_ok ? r : 0;
  const int8_t* xrow = xq + (tok_ok ? t : 0) * k;
  v4i c = {0, 0, 0, 0};
  int qs = 0;
  for (int64_t kb = 0; kb < k; kb += 64) {
    const int64_t kk = kb + 16 * g;
    const uint8_t* wblk = packed + panel_offset(n_out, nkb, bw, rr, kb / 64);     // panel-major blocks
    v4i a = {0, 0, 0, 0};
    if (FMT == 0) a = dense2_quad(row_ok ? reinterpret_cast<const uint32_t*>(wblk)[g] : 0x55555555u);
    else if (row_ok) a = nm_bytes16<M>(wblk, meta + panel_offset(n_out, nkb, 8, rr, kb / 64), n, 16 * g);
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
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = row0 + 4 * g + v;            // C[4*(lane/16)+v][lane%16]
    if (row < n_out) {
      const int32_t a = c[v] - (FMT == 0 ? qs : 0);
      y[t * n_out + row] = (float)a * out_scale_g(row_beta(beta, beta_rows, row), gamma[t]);
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

// D = weight stages in flight per wave: the wave's whole k range when it is
// short, else 4 (with the panel-major layout the waves of a launch sweep the
// matrix together, and a shallower ring keeps the sweep's front compact).
// DENSE2 launches of at least 2^26 weights (70B-class) take 6: with the
// nontemporal weight loads the deeper ring measured 1-2% faster there (and
// slower for N:M, whose decode holds more registers, and for smaller
// launches).
template <int KIND>
void launch_gemv(const GemvLaunch& L, int xlm, bool xf, int spw, bool deep, dim3 grid, dim3 block, size_t lds,
                 hipStream_t s) {
  if (xf) {
    if (spw <= 2) hipLaunchKernelGGL((gemv_kernel<KIND, 1, 2, true>), grid, block, lds, s, L);
    else if (KIND == kDense2 && deep) hipLaunchKernelGGL((gemv_kernel<kDense2, 1, 6, true>), grid, block, lds, s, L);
    else hipLaunchKernelGGL((gemv_kernel<KIND, 1, 4, true>), grid, block, lds, s, L);
  } else if (xlm == 1) {
    if (spw <= 2) hipLaunchKernelGGL((gemv_kernel<KIND, 1, 2, false>), grid, block, lds, s, L);
    else if (KIND == kDense2 && deep) hipLaunchKernelGGL((gemv_kernel<kDense2, 1, 6, false>), grid, block, lds, s, L);
    else hipLaunchKernelGGL((gemv_kernel<KIND, 1, 4, false>), grid, block, lds, s, L);
  } else if (xlm == 2) {
    // more dynamic LDS than the default limit: raised once per kernel
    static const bool raised = hipFuncSetAttribute((const void*)gemv_kernel<KIND, 2, 2, false>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, kBigLdsAttr) == hipSuccess &&
                               hipFuncSetAttribute((const void*)gemv_kernel<KIND, 2, 4, false>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, kBigLdsAttr) == hipSuccess;
    (void)raised;
    if (spw <= 2) hipLaunchKernelGGL((gemv_kernel<KIND, 2, 2, false>), grid, block, lds, s, L);
    else hipLaunchKernelGGL((gemv_kernel<KIND, 2, 4, false>), grid, block, lds, s, L);
  } else {
    if (spw <= 2) hipLaunchKernelGGL((gemv_kernel<KIND, 0, 2, false>), grid, block, lds, s, L);
    else hipLaunchKernelGGL((gemv_kernel<KIND, 0, 4, false>), grid, block, lds, s, L);
  }
}

// Launch shape of a grouped GEMV: k split (waves per tile) and tiles per
// workgroup, about one round of resident waves.
struct GemvShape {
  int ks, tb, spw;
  int xlm;    // token-row staging: 0 none, 1 registers, 2 LDS-direct (gemv_kernel's XLM)
  bool big;   // at least 2^26 weights in the launch
};
GemvShape gemv_shape(const LinDesc* items, int count) {
  int tiles = 0, max_nsb = 1;
  int64_t max_x = 0, weights = 0;
  bool k1024 = true;
  for (int i = 0; i < count; ++i) {
    k1024 = k1024 && items[i].k % 1024 == 0;
    tiles += (int)((items[i].n_out + 15) / 16);
    const int nsb = (items[i].k / 64 + 3) / 4;
    max_nsb = nsb > max_nsb ? nsb : max_nsb;
    const int64_t xb = (int64_t)items[i].m_tok * items[i].k;
    max_x = xb > max_x ? xb : max_x;
    weights += items[i].n_out * (int64_t)items[i].k;
  }
  GemvShape g;
  // LDS-direct staging pays for its full-size workgroups and its staging pass
  // only on long weight streams (70B-class widths: +23-30% at 8-16 tokens;
  // 3B-class launches: 6-10% slower)
  g.xlm = max_x <= kXLdsMax ? 1 : (max_x <= kXBigMax && weights >= kXBigMinWeights && k1024 ? 2 : 0);
  // the LDS-direct mode runs one 16-wave workgroup per CU; it keeps twice
  // the waves (measured: 5-9% faster than 2048 at 8 tokens, 70B widths)
  // launches streaming fewer than 2^26 weights (3B-class blocks) do better
  // with fewer waves still (measured: 3B block 21.4 -> 20.2 us at one token,
  // 24.0 -> 22.6 at 4, 27.6 -> 26.2 at 8; the 70B-class launches, all at
  // least 2^26 weights, were 2-5% slower with 1536)
  g.big = weights >= (int64_t(1) << 26);
  const int base = g.big ? kResidentWaves : kSmallLaunchWaves;
  const int target = g.xlm == 2 ? 2 * base : base;
  g.ks = tiles > 0 ? target / tiles : 1;
  g.ks = g.ks < 1 ? 1 : (g.ks > kMaxWaves ? kMaxWaves : g.ks);
  g.ks = g.ks > max_nsb ? max_nsb : g.ks;
  g.tb = 8 / g.ks;
  g.tb = g.tb < 1 ? 1 : g.tb;
  if (g.xlm == 1 && g.ks * g.tb < kXMinWaves) g.tb = (kXMinWaves + g.ks - 1) / g.ks;   // the staging needs the threads
  if (g.xlm == 2) g.tb = kMaxWaves / g.ks;                // one workgroup per CU (LDS): make it a full one
  g.spw = (max_nsb + g.ks - 1) / g.ks;            // stages per wave
  return g;
}

// whether the fused activation quantization covers m_tok x k activations at
// this shape, and pays: every workgroup reads and quantizes the whole input,
// so beyond kXFuseMax values per launch the standalone quantizer (one launch,
// ~3.5 us) costs less (measured, 70B-class widths: 8192 inputs fused +1-2 us
// per launch against +3.5 us; 28672 inputs fused +8 us against +5 us)
constexpr int64_t kXFuseMax = 16384;
bool gemv_fuses(const GemvShape& g, int64_t m_tok, int64_t k) {
  return g.xlm == 1 && m_tok * k <= kXFuseMax && m_tok * k <= (int64_t)16 * kXFPer * 64 * g.ks * g.tb;
}

// xf: fp32 activations shared by every item, quantized inside the launch
// (the caller has checked gemv_fuses); xq_out / gamma_out: where the launch
// publishes them (nullable).
hipError_t launch_gemv_group(int kind, const LinDesc* items, int count, hipStream_t s, const float* xf = nullptr,
                             int8_t* xq_out = nullptr, float* gamma_out = nullptr) {
  GemvLaunch L = {};
  int tiles = 0;
  int64_t max_xp = 0;                              // token rows in LDS, padded: m_tok * (k + 16)
  for (int i = 0; i < count; ++i) {
    tiles += (int)((items[i].n_out + 15) / 16);
    const int64_t xp = (int64_t)items[i].m_tok * (items[i].k + 16);
    max_xp = xp > max_xp ? xp : max_xp;
  }
  if (tiles == 0) return hipSuccess;
  const GemvShape g = gemv_shape(items, count);
  L.ks = g.ks;
  L.tb = g.tb;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    L.b.d[i] = items[i];
    L.b.d[i].x = xf;
    L.b.d[i].xq_out = xq_out;
    L.b.d[i].gamma_out = gamma_out;
    L.b.start[i] = blocks;
    const int t = (int)((items[i].n_out + 15) / 16);
    blocks += (t + g.tb - 1) / g.tb;
  }
  L.b.start[count] = blocks;
  L.b.count = count;
  const size_t xreg = g.xlm != 0 ? (size_t)max_xp : 0;
  const size_t lds = xreg + 64 + (g.ks > 1 ? (size_t)g.ks * g.tb * 4 * 64 * sizeof(int32_t) : 0);
  const dim3 grid((unsigned)blocks), block(64 * g.ks * g.tb);
  const bool xf_on = xf != nullptr;
  if (kind == kDense2) launch_gemv<kDense2>(L, g.xlm, xf_on, g.spw, g.big, grid, block, lds, s);
  else if (kind == kNm68) launch_gemv<kNm68>(L, g.xlm, xf_on, g.spw, g.big, grid, block, lds, s);
  else launch_gemv<kNm24>(L, g.xlm, xf_on, g.spw, g.big, grid, block, lds, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, int fmt, int n, int m, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_out + 63) / 64), (unsigned)((a.m_tok + 15) / 16)), block(256);
  if (fmt == 0)
    hipLaunchKernelGGL((linear_generic_kernel<0, 8>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc, (int32_t)a.beta_rows);
  else if (m == 8)
    hipLaunchKernelGGL((linear_generic_kernel<1, 8>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc, (int32_t)a.beta_rows);
  else
    hipLaunchKernelGGL((linear_generic_kernel<1, 4>), grid, block, 0, s, a.packed, a.meta, n, a.beta, a.xq, a.gamma, a.m_tok, a.n_out, a.k, a.y, a.acc, (int32_t)a.beta_rows);
  return hipGetLastError();
}

// whether the GEMV's 32-bit buffer offsets cover this product
bool gemv_fits(const LinearArgs& a, int kind) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t bw = kind == kDense2 ? 16 : (kind == kNm68 ? 12 : 8);
  return a.n_out * (a.k / 64) * bw < lim && a.n_out * (a.k / 8) < lim;
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
    if (kind < 0 || (a.m_tok > kGemvMaxTokens && !gemm_fits(a, kind)) ||
        (a.m_tok <= kGemvMaxTokens && !gemv_fits(a, kind))) {
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

hipError_t launch_linear_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                              const LinearArgs* items, int count, int fmt, int n, int m, hipStream_t s) {
  const int kind = kind_of(fmt, n, m);
  bool fuse = kind >= 0 && m_tok <= kGemvMaxTokens && count <= kMaxDesc;
  LinDesc ds[kMaxDesc];
  int nd = 0;
  for (int i = 0; fuse && i < count; ++i) {
    if (items[i].n_out == 0) continue;
    if (!gemv_fits(items[i], kind)) fuse = false;
    else ds[nd++] = to_desc(items[i]);
  }
  fuse = fuse && nd > 0 && gemv_fuses(gemv_shape(ds, nd), m_tok, k);
  if (fuse) return launch_gemv_group(kind, ds, nd, s, x, xq, gamma);
  const hipError_t e = launch_quant_acts(x, m_tok, k, xq, gamma, s);
  if (e != hipSuccess) return e;
  return launch_linear_batch(items, count, fmt, n, m, s);
}

}  // namespace sbl
