// Prefill / training-forward GEMM of the BitLinear product (bitnet.cpp article
// "Fundamento matematico" item 3, y = W~ x~ beta gamma / Qb) for token counts
// above the decode range: at thousands of tokens the ternary x int8 product
// is a dense contraction, so it runs on gfx950 int8 MFMA
// (v_mfma_i32_32x32x32_i8, 32 rows x 32 tokens x 32 k per instruction).
//
// Tiling: a workgroup of 4*WT waves owns 32*KRT*4 weight rows x 32*KCT*WT
// tokens; wave w owns KRT row tiles (32 rows each) x KCT token tiles, so every
// weight operand is decoded WT times per workgroup (once for N:M).  The k loop advances
// 128 k per step (four 32-k MFMA sub-steps); the MFMA's k order is free as
// long as A and B agree, so lane half g of a row takes the row's 64-weight
// block 2*step + g whole, with one load per row tile per step, and uses only
// the words it loaded (loads are the scarce resource here: the cost of a
// vector memory instruction grows with the cache lines it touches, not with
// its bytes).
//  * activations (the MFMA's A operand): each step's token x 128 byte tile is
//    fetched (eight tokens, whole 128-byte lines, per instruction) into
//    registers kDepth steps ahead, written to one of two LDS buffers one step
//    ahead of use and read back as operands; the 16-byte chunks of a token row
//    are XOR-swizzled by the token index so that consecutive tokens read
//    distinct banks.
//  * weights (the MFMA's B operand): fetched kDepth-1 steps ahead straight
//    into registers and decoded into operands (7 VALU ops per 16 weights;
//    N:M: codes spread arithmetically, one LDS selector read per 8 weights,
//    v_perm); each decoded weight operand feeds KCT MFMAs.
//  * with the activations as A, each lane's accumulators hold 16 tokens of
//    one weight row, so the epilogue writes whole 128-byte runs of a token's
//    output row.
//  * the per-step workgroup barrier waits only for LDS traffic, never for
//    the global loads in flight.
// K need only be a multiple of 64: in a last half step the second half reads
// zeros (weights and activations), which adds nothing.
// DENSE2 feeds u = c + 1 to the MFMA and subtracts sum_k q per token at the
// end; the threads that stage activations into LDS accumulate those sums
// with v_dot4 as they go (once per byte, not once per wave).  N:M decodes
// to c directly.
// All integer work is exact; results are bit-identical to the GEMV path.
#include "sbl_decode.h"

#include <type_traits>

namespace sbl {

namespace {

using namespace dec;

typedef int32_t v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;            // k per step
constexpr int kThreads = 256;
constexpr int kDepth = 2;           // steps of loads in flight (registers)
constexpr int kUnroll = 2;          // lcm(kDepth, 2 LDS buffers)
constexpr uint32_t kFar = 0x80000000u;   // a buffer offset beyond every buffer: reads zeros

// Raw weight bytes of one lane for one step of one row tile: the whole
// 64-weight block 2*step + g of the lane's row (g = lane half).  Raw data are
// kept untouched until decode so that no load result is consumed early
// (which would force a wait on the whole prefetch pipeline).
template <int KIND> struct WRaw;
template <> struct WRaw<kDense2> { uint32_t w[4]; };                 // 4 words of 16 weights
template <> struct WRaw<kNm68> { uint32_t c[3]; uint32_t m[2]; };    // 12 code bytes, 8 meta bytes
template <> struct WRaw<kNm24> { uint32_t c[2]; uint32_t m[2]; };    // 8 code bytes, 8 meta bytes

__device__ __forceinline__ v4i lds_ld16(const uint8_t* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return v4i{(int32_t)v[0], (int32_t)v[1], (int32_t)v[2], (int32_t)v[3]};
}

// byte offset of 16-byte chunk c (0..7) of token row r in an LDS activation
// tile of 128-byte rows.  gfx950's LDS serves a 16-byte read for 16 lanes per
// cycle from 64 banks (256 bytes): rows r and r+1 lie in the two halves of a
// bank row, and the chunk is XOR-swizzled by (r/2) % 8, so 16 consecutive
// rows reading the same chunk hit 16 distinct 16-byte bank groups.  (A swizzle
// by r % 8 leaves rows r and r+8 on the same banks: a 2-way conflict on every
// read.)
__device__ __forceinline__ int bt_off(int r, int c) { return r * kBK + 16 * (c ^ ((r >> 1) & 7)); }

// Buffer resources: loads past the end of a buffer return zeros, so tokens
// past m_tok need neither branches nor clamping.  Weights are stored
// panel-major (panel_offset); rows past n_out of a last tile read other rows'
// bytes or zeros, and their results are never stored.  32-bit offsets: the
// host keeps every buffer of this path below 2 GiB.  Past the row's last block
// the offset is kFar (zeros).
template <int KIND>
__device__ __forceinline__ void load_w(WRaw<KIND>& a, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rm,
                                       uint32_t ow, uint32_t om, bool ok) {
  if constexpr (KIND == kDense2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? ow : kFar, 0, 0);
    a.w[0] = v[0]; a.w[1] = v[1]; a.w[2] = v[2]; a.w[3] = v[3];
  } else if constexpr (KIND == kNm68) {
    const auto c = __builtin_amdgcn_raw_buffer_load_b96(rw, ok ? ow : kFar, 0, 0);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rm, ok ? om : kFar, 0, 0);
    a.c[0] = c[0]; a.c[1] = c[1]; a.c[2] = c[2];
    a.m[0] = m[0]; a.m[1] = m[1];
  } else {
    const auto c = __builtin_amdgcn_raw_buffer_load_b64(rw, ok ? ow : kFar, 0, 0);
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rm, ok ? om : kFar, 0, 0);
    a.c[0] = c[0]; a.c[1] = c[1];
    a.m[0] = m[0]; a.m[1] = m[1];
  }
}

// Workgroup barrier for LDS hand-off.  Unlike __syncthreads() it does not
// drain outstanding global loads (vmcnt), so the prefetch pipeline stays in
// flight across it; the "memory" clobber keeps LDS accesses on their side.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Four 2-bit codes u (bits 2i, 2i+1 of x's low byte) -> four int8
// c = u - 1 bytes, arithmetically: two shift-or-mask rounds put code i in
// byte i, then v_perm maps u in {0, 1, 2} to {0xFF, 0x00, 0x01}.  (A table in
// LDS would cost a lane-random LDS read instead, and those reads, not the
// MFMAs, bound the N:M decode.)
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  x &= 0xFFu;
  const uint32_t y = (x | (x << 12)) & 0x000F000Fu;   // codes 0,1 in bits 0-3, codes 2,3 in bits 16-19
  const uint32_t z = (y | (y << 6)) & 0x03030303u;    // code i in byte i
  return __builtin_amdgcn_perm(0u, 0x000100FFu, z);
}

// Weight operand (16 weights, k order) of sub-step j: word j of the lane's block.
template <int KIND>
__device__ __forceinline__ v4i decode_w(const WRaw<KIND>& a, int j, const NmLut& L) {
  if constexpr (KIND == kDense2) {
    return dense2_quad(a.w[j]);
  } else if constexpr (KIND == kNm68) {
    // word j: codes = bits 24j .. 24j+23 of the 96-bit block, meta = bytes 2j, 2j+1
    const uint32_t c24 = j == 0 ? a.c[0]
                       : j == 1 ? __builtin_amdgcn_alignbit(a.c[1], a.c[0], 24)
                       : j == 2 ? __builtin_amdgcn_alignbit(a.c[2], a.c[1], 16)
                                : (a.c[2] >> 8);
    const uint32_t m16 = (j & 1) ? (a.m[j >> 1] >> 16) : a.m[j >> 1];
    v4i r;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t c12 = (c24 >> (12 * q)) & 0xFFFu;
      const uint32_t mb = (m16 >> (8 * q)) & 0xFFu;
      const uint32_t lo = spread4(c12);
      const uint32_t hi = spread4(c12 >> 8);
      r[2 * q] = (int32_t)__builtin_amdgcn_perm(hi, lo, L.sel[mb][0]);
      r[2 * q + 1] = (int32_t)__builtin_amdgcn_perm(hi, lo, L.sel[mb][1]);
    }
    return r;
  } else {
    // word j: codes = bytes 2j, 2j+1, meta = bytes 2j, 2j+1
    const uint32_t c16 = (j & 1) ? (a.c[j >> 1] >> 16) : a.c[j >> 1];
    const uint32_t m16 = (j & 1) ? (a.m[j >> 1] >> 16) : a.m[j >> 1];
    v4i r;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t v = spread4(c16 >> (8 * q));
      const uint32_t mb = (m16 >> (8 * q)) & 0xFFu;
      r[2 * q] = (int32_t)__builtin_amdgcn_perm(v, v, L.sel[mb][0]);
      r[2 * q + 1] = (int32_t)__builtin_amdgcn_perm(v, v, L.sel[mb][1]);
    }
    return r;
  }
}

// KRT 32-row tiles and KCT 32-token tiles per wave; 4 waves along the rows
// and WT along the tokens (wave w: rows of w % 4, token tiles of w / 4).
// A wave with 16 accumulator tiles needs every register of a SIMD; the
// others are held to half of them, so that two waves share each SIMD and one's
// latencies hide behind the other's matrix work (256 x 128 tiles: +10% at
// 2048 tokens; 256 x 256 DENSE2 as 8 waves of 64 x 128: +2% at 2048 and +6%
// at 4096 tokens against 4 waves of 64 x 256).
template <int KIND, int KRT, int KCT, int WT, bool GRP = false>
__global__ __launch_bounds__(kThreads * WT, KRT * KCT * WT >= 16 ? 1 : 2) void gemm_kernel(const LinBatch batch) {
  constexpr int kRT = KRT, kCT = KCT;
  constexpr int kThr = kThreads * WT;               // 4 waves along the rows x WT along the tokens
  constexpr int kBM = 4 * 32 * kRT;                 // weight rows per workgroup
  constexpr int kBN = 32 * kCT * WT;                // tokens per workgroup
  constexpr int kTokPass = kThr / 8;                // tokens staged per pass (8 threads per token row)
  constexpr int kStPasses = kBN * kBK / (16 * kThr);   // 16-byte staging loads per thread
  __shared__ NmLut lut;
  __shared__ __attribute__((aligned(16))) uint8_t btile[2][kBN * kBK];
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
  const int nks = (int)((K + kBK - 1) / kBK);      // steps; the last may be half (K % 128 == 64)
  const int nkb = (int)(K / 64);                    // 64-weight blocks per row

  const int tid = threadIdx.x, wave = (tid >> 6) & 3, wt = tid >> 8, lane = tid & 63;
  const int li = lane & 31, g = lane >> 5;
  __shared__ __attribute__((aligned(16))) int32_t qsum_lds[kBN];
  __shared__ __attribute__((aligned(16))) float scale_lds[kBN];

  // activation staging: thread -> token (tid >> 3) + 32p, 16-byte chunk tid & 7
  // (eight tokens' whole 128-byte rows per load instruction)
  const int st_tok = tid >> 3, st_chunk = tid & 7;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(d.xq, (int64_t)d.m_tok * K);
  int voff_b[kStPasses];
#pragma unroll
  for (int p = 0; p < kStPasses; ++p) voff_b[p] = (int)((t0 + st_tok + kTokPass * p) * K + 16 * st_chunk);
  auto load_b = [&](int ks, u32x4* r) {
    const bool ok = kBK * ks + 16 * st_chunk < K;   // false: second half of a last half step
#pragma unroll
    for (int p = 0; p < kStPasses; ++p) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? voff_b[p] + kBK * ks : (int)kFar, 0, 0);
      r[p] = u32x4{v[0], v[1], v[2], v[3]};
    }
  };
  int qpart[kStPasses] = {};                         // DENSE2: per staged token, sum of its q bytes
  // `real`: the staged step exists (only those count towards the q sums)
  auto store_b = [&](int buf, const u32x4* r, bool real) {
#pragma unroll
    for (int p = 0; p < kStPasses; ++p) {
      *reinterpret_cast<u32x4*>(&btile[buf][bt_off(st_tok + kTokPass * p, st_chunk)]) = r[p];
      if (KIND == kDense2) {                        // branchless: a branch here costs the
        int q = 0;                                  // loop its exact load wait counts
#pragma unroll
        for (int j = 0; j < 4; ++j) q = __builtin_amdgcn_sdot4((int)r[p][j], 0x01010101, q, false);
        qpart[p] += real ? q : 0;
      }
    }
  };
  // weights: row tile rt of this wave = rows n0 + 32*kRT*wn + 32rt + li; the
  // lane's block 2*ks + g lies in panel ks/2 at block position 2*(ks&1) + g
  constexpr uint32_t bw = KIND == kDense2 ? 16u : (KIND == kNm68 ? 12u : 8u);   // bytes per block
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.packed, d.n_out * nkb * (int64_t)bw);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(KIND == kDense2 ? d.packed : d.meta, d.n_out * (K / 8));
  const int nfull = nkb / 4;                        // full panels
  const uint32_t nbl = (uint32_t)(nkb - 4 * nfull); // blocks of a last partial panel
  const uint32_t pb_w = 4u * bw * (uint32_t)d.n_out, pb_m = 32u * (uint32_t)d.n_out;
  uint32_t full_w[kRT], full_m[kRT], last_w[kRT], last_m[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const uint32_t row = (uint32_t)(n0 + 32 * kRT * wave + 32 * rt + li);
    full_w[rt] = row * 4u * bw;
    full_m[rt] = row * 32u;
    last_w[rt] = row * nbl * bw;
    last_m[rt] = row * nbl * 8u;
  }
  auto load_wall = [&](int ks, WRaw<KIND>* a) {
    const int p = ks >> 1;
    const bool full = p < nfull;
    const uint32_t bi = (uint32_t)(2 * (ks & 1) + g);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      load_w<KIND>(a[rt], rw, rm, (uint32_t)p * pb_w + (full ? full_w[rt] : last_w[rt]) + bi * bw,
                   (uint32_t)p * pb_m + (full ? full_m[rt] : last_m[rt]) + bi * 8u, 2 * ks + g < nkb);
  };

  v16i acc[kRT][kCT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[rt][ct] = v16i{};

  u32x4 bst[kDepth][kStPasses];
  WRaw<KIND> wr[kDepth][kRT];
  // prologue: steps 0 .. kDepth-1 in flight, step 0 in LDS
#pragma unroll
  for (int s = 0; s < kDepth; ++s) {
    if (s < nks) {
      load_b(s, bst[s]);
      load_wall(s, wr[s]);
    }
  }
  if (KIND != kDense2) __syncthreads();             // tables built
  store_b(0, bst[0], true);
  // Drain the prologue's loads once: the loop header's wait counts must hold
  // on the entry path too, and there the scheduler leaves step 0's weights as
  // the youngest loads, which would cost a full drain on every step.
  // (gfx9 s_waitcnt encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
  __builtin_amdgcn_s_waitcnt(0xF70);
  lds_barrier();

  // one 64-k step; u = ks mod kUnroll fixes the register slot and LDS buffer.
  // In the main loop (tail == false) the refills are unconditional: a refill
  // past the last step only fills a slot nobody reads (buffer loads stay in
  // bounds), and without branches around loads the compiler can wait for
  // exactly the stage it needs instead of draining every load in flight.
  auto step = [&](const int ks, const int u, const bool tail) {
    const int slot = u % kDepth;                    // == ks % kDepth (kUnroll is a multiple of kDepth)
    // activations of step ks + kDepth go to the slot step ks vacated (it is in LDS)
    if (!tail || ks + kDepth < nks) load_b(ks + kDepth, bst[slot]);
    const uint8_t* bt = &btile[u & 1][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {                   // 32-k MFMA sub-steps: lane half g takes
      v4i b[kCT];                                   // k = 128 ks + 64 g + 16 j .. +15
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) b[ct] = lds_ld16(bt + bt_off(32 * (wt * kCT + ct) + li, 4 * g + j));
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const v4i a = decode_w<KIND>(wr[slot][rt], j, lut);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[ct], a, acc[rt][ct], 0, 0, 0);
      }
    }
    // weights of step ks + kDepth reuse the slot just consumed
    if (!tail || ks + kDepth < nks) load_wall(ks + kDepth, wr[slot]);
    if (!tail || ks + 1 < nks) store_b((u + 1) & 1, bst[(u + 1) % kDepth], ks + 1 < nks);
    lds_barrier();
    // no decode of a later step's weights may be hoisted into this one: there
    // its loads are still the youngest in flight (a full drain)
    __builtin_amdgcn_sched_barrier(0);
  };
  // main loop without exits (keeps the accumulators resident in AGPRs) over
  // the steps whose refills are all real or harmless, then the last ones
  int ks0 = 0;
  for (; ks0 + kUnroll <= nks; ks0 += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) step(ks0 + u, u, false);
  }
#pragma unroll
  for (int u = 0; u < kUnroll - 1; ++u)
    if (ks0 + u < nks) step(ks0 + u, u, true);

  // per-token sums of q (DENSE2): the 8 threads staging a token hold its 8 chunks
  if (KIND == kDense2) {
#pragma unroll
    for (int p = 0; p < kStPasses; ++p) {
      int v = qpart[p];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (st_chunk == 0) qsum_lds[st_tok + kTokPass * p] = v;
    }
  }
  // output scale per token of the tile; with beta per row group (group
  // scales) the token's max(gamma, 1e-5), the scale being formed per row
  for (int i = tid; i < kBN; i += kThr)
    scale_lds[i] = t0 + i >= d.m_tok ? 0.0f : GRP ? fmaxf(d.gamma[t0 + i], 1e-5f) : out_scale(d.beta, d.gamma, t0 + i);
  __syncthreads();
  // epilogue: the MFMAs take the activations as A and the weights as B, so
  // lane (li, g) holds C[token 8*(v/4) + 4g + v%4][row li] of each 32 x 32
  // tile.  For each v the 32 lanes of a half write 32 consecutive rows of one
  // token's output: 128 contiguous bytes, whole cache lines.  (Rows as A put 4
  // rows of 32 tokens in each lane: every 16-byte store touched 32 lines.)
  // Buffer stores: the token offset is wave-uniform (scalar offset); rows past
  // n_out get an offset past the buffer and tokens past m_tok land past it, so
  // both are dropped without branches (the host keeps m_tok*n_out*4 + the last
  // tile's overhang below 2^31 bytes).
  const uint32_t tokb = (uint32_t)d.n_out * 4u;      // bytes per token row of y
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(d.y, d.m_tok * (int64_t)tokb);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(d.acc, d.acc ? d.m_tok * (int64_t)tokb : 0);
  const int wts = __builtin_amdgcn_readfirstlane(wt);
  uint32_t vo[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int64_t row = n0 + 32 * kRT * wave + 32 * rt + li;
    vo[rt] = row < d.n_out ? (uint32_t)row * 4u + (uint32_t)(4 * g) * tokb : kFar;
  }
  auto store_all = [&](auto with_acc) {
    // group scales: max(beta, 1e-5) of each row tile's row (rows past n_out take the last row's)
    float brow[kRT];
    if constexpr (GRP) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int64_t row = n0 + 32 * kRT * wave + 32 * rt + li;
        brow[rt] = fmaxf(*row_beta(d.beta, d.beta_rows, row < d.n_out ? row : d.n_out - 1), 1e-5f);
      }
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int tl4 = 32 * (wt * kCT + ct) + 8 * v4 + 4 * g;   // this lane's 4 tokens: tl4 .. tl4+3
        const float4 sc4 = *reinterpret_cast<const float4*>(&scale_lds[tl4]);
        int4 cq4 = make_int4(0, 0, 0, 0);
        if (KIND == kDense2) cq4 = *reinterpret_cast<const int4*>(&qsum_lds[tl4]);
        const float scj[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
        const int32_t cqj[4] = {cq4.x, cq4.y, cq4.z, cq4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * v4 + j;
          const uint32_t so = (uint32_t)(t0 + 32 * (wts * kCT + ct) + 8 * v4 + j) * tokb;   // wave-uniform
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            const int32_t a = acc[rt][ct][v] - cqj[j];
            float sc = scj[j];
            if constexpr (GRP) sc = (brow[rt] * scj[j]) * 0.0078125f;   // RN(RN(beta*gamma)*2^-7)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)a * sc), ry, vo[rt], so, 0);
            if constexpr (decltype(with_acc)::value) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)a, ra, vo[rt], so, 0);
          }
        }
      }
    }
  };
  if (d.acc) store_all(std::true_type{});
  else store_all(std::false_type{});
}

// Tile shapes (weight rows x tokens), workgroups that fit on one CU at once
// (occupancy of the kernel: 256 x 256 takes a whole CU), and the measured
// time of one full round of such workgroups per 128-k step, relative to a
// round of 256 x 256 tiles, for DENSE2 and for N:M 6:8 (fitted, as the median
// over the eight launches of the 3B-class block at 2048 tokens and the
// 13B-class block at 4096).  A launch costs whole rounds: small tiles fill the
// chip when a product has few large tiles (tile quantization), large tiles
// reuse operands.
struct TileShape { int rows, toks, slots; double cost[2]; };
constexpr TileShape kShapes[] = {{256, 256, 1, {1.0, 1.0}}, {256, 128, 2, {0.775, 0.947}},
                                 {128, 256, 2, {0.951, 0.829}}, {128, 128, 2, {0.526, 0.569}}};

int pick_shape(const LinearArgs* items, int count, int kind) {
  const int ci = kind == kDense2 ? 0 : 1;
  int best = 0;
  double best_t = 1e300;
  for (int si = 0; si < 4; ++si) {
    const TileShape& sh = kShapes[si];
    int64_t tiles = 0, ksteps = 0;
    for (int i = 0; i < count; ++i) {
      const int64_t t = ((items[i].n_out + sh.rows - 1) / sh.rows) * ((items[i].m_tok + sh.toks - 1) / sh.toks);
      tiles += t;
      ksteps += t * (items[i].k / kBK);
    }
    const int64_t per_round = 256 * (int64_t)sh.slots;
    const double rounds = (double)((tiles + per_round - 1) / per_round);
    const double t = rounds * sh.cost[ci] * ((double)ksteps / (double)tiles);
    if (t < best_t * 0.999) { best_t = t; best = si; }
  }
  return best;
}

}  // namespace

bool gemm_fits(const LinearArgs& a, int kind) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t row_bytes = kind == kDense2 ? a.k / 4 : (kind == kNm68 ? 3 * a.k / 16 : a.k / 8);
  return (a.m_tok + 256) * a.k < lim && (a.n_out + 256) * row_bytes < lim &&
         (a.n_out + 256) * (a.k / 8) < lim && (a.m_tok + 256) * a.n_out * 4 < lim;
}

namespace {

template <int KRT, int KCT, int WT = 1, bool GRP = false>
hipError_t launch_shape(const LinearArgs* items, int count, int kind, hipStream_t s) {
  constexpr int kBM = 4 * 32 * KRT, kBN = 32 * KCT * WT;
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
  const dim3 grid((unsigned)blocks), block(kThreads * WT);
  if (kind == kDense2) hipLaunchKernelGGL((gemm_kernel<kDense2, KRT, KCT, WT, GRP>), grid, block, 0, s, b);
  else hipLaunchKernelGGL((gemm_kernel<kNm68, KRT, KCT, WT, GRP>), grid, block, 0, s, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_group(const LinearArgs* items, int count, int kind, hipStream_t s) {
  if (kind == kNm24) return launch_gemm24_group(items, count, s);
  // group scales (beta per row block): one tile shape, with the epilogue that
  // reads beta per row
  if (items[0].beta_rows > 0) return launch_shape<1, 4, 1, true>(items, count, kind, s);
  switch (pick_shape(items, count, kind)) {
    // 256 x 256: DENSE2 as 8 waves (4 along the rows x 2 along the tokens,
    // 64 x 128 each, two waves per SIMD; each row's cheap decode done by two
    // waves), N:M as 4 waves of 64 x 256 (one per SIMD; its decode done once)
    case 0: return kind == kDense2 ? launch_shape<2, 4, 2>(items, count, kind, s)
                                   : launch_shape<2, 8, 1>(items, count, kind, s);
    case 1: return launch_shape<2, 4>(items, count, kind, s);
    case 2: return launch_shape<1, 8>(items, count, kind, s);
    default: return launch_shape<1, 4>(items, count, kind, s);
  }
}

}  // namespace sbl
