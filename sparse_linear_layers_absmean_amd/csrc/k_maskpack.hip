// Fused N:M mask + ternarization + packing of BF16 master weights, and the
// standalone packer for precomputed codes.
//
// Method (Sparse-BitNet, section 2): the N:M mask keeps, in every group of m
// consecutive weights along k, the n largest BF16 master magnitudes ("Mask
// Generation": from the full-precision masters, not the ternary codes);
// ties go to the lower index.  The ternary code is RoundClip(w/beta, -1, 1)
// with the absmean scale ("Ternary Quantization"), and the mask is applied
// to the codes ("Quant-Then-Mask Order"), so the packed N:M codes are the
// metadata-described discrete weights the kernel consumes.
//
// Exact integer formulation used here (no division):
//  * key_j = (|w_j| bits << log2 m) | (m-1-j) is unique inside a group and
//    orders first by magnitude, then by lower index; keep_j <=> fewer than n
//    keys exceed key_j.
//  * |w| > beta_eff/2  <=>  (|w| bf16 bits) > (fp32 bits of beta_eff/2) >> 16,
//    since fp32 order equals bit order for nonnegative values and a BF16
//    value is the top half of an fp32; RoundClip(w/beta) is nonzero exactly
//    then (a ratio of exactly 1/2 rounds to even, i.e. to 0).
//
// Patterns that drop at most two of a group (8:8, 7:8, 6:8, 4:4, 3:4, 2:4)
// take the packed path below: two BF16 magnitudes per 32-bit register and
// v_pk_{min,max,sub}_u16, so a group of 8 costs about 70 VALU operations
// (the per-key formulation needs about 180).  Other patterns use the
// per-key kernel.
//
// One thread handles one 64-weight chunk (128 bytes of BF16): groups never
// cross chunks (m divides 64) and chunks never cross rows (64 divides k), so
// the matrix is processed as a flat array.  Per chunk it writes 16 bytes of
// DENSE2, 8 bytes of bitmap, 64*n/m/4 bytes of N:M codes and 64 code bytes;
// the packed stream and the N:M metadata go to their panel-major places.
// DENSE2 word layout: see d2_shift.
// beta itself is finalized at the start of every workgroup from the absmean
// pass's partial sums (sbl_beta.h), while the first chunk loads are in flight.
#include "sbl_partial.h"
#include "sbl_select.h"

namespace sbl {

namespace {

constexpr int kThreads = 256;

// DENSE2 bit offset of weight p inside its 16-weight word: byte p%4, bit pair (p/4)%4,
// so (word >> 2s) & 0x03030303 holds weights 4s .. 4s+3 in byte order.
__device__ __forceinline__ int d2_shift(int p) { return 8 * (p & 3) + 2 * ((p >> 2) & 3); }

struct ChunkOut {
  uint32_t d2[4];        // DENSE2: word q holds weights 16q .. 16q+15
  uint64_t keep;         // bit j = weight j kept
  uint64_t nm_lo, nm_hi; // N:M compact codes, 2 bits per kept weight
  uint32_t cb[16];       // int8 codes, 4 per word
};

// threshold key: keep_j <=> key_j > thr (thr = -1 keeps all)
template <int M>
__device__ __forceinline__ int group_threshold(const int* key, int n) {
  const int drop = M - n;
  if (drop <= 0) return -1;
  if (drop == 1) {
    int mn = key[0];
#pragma unroll
    for (int j = 1; j < M; ++j) mn = min(mn, key[j]);
    return mn;
  }
  if (drop == 2) {
    // bottom-2 merge network: (lo, hi) = two smallest keys
    int lo = min(key[0], key[1]), hi = max(key[0], key[1]);
#pragma unroll
    for (int j = 2; j < M; j += 2) {
      const int a = min(key[j], key[j + 1]), b = max(key[j], key[j + 1]);
      const int nlo = min(lo, a);
      hi = min(max(lo, a), min(hi, b));
      lo = nlo;
    }
    return hi;
  }
  // general case: the drop-th smallest key is the one with exactly drop-1 smaller keys
  int thr = -1;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    int below = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) below += key[i] < key[j];
    thr = (below == drop - 1) ? key[j] : thr;
  }
  return thr;
}

__device__ __forceinline__ void nm_insert(ChunkOut& o, uint32_t u, int pos2) {
  const uint64_t v = (uint64_t)u;
  if (pos2 < 64) o.nm_lo |= v << pos2;
  else o.nm_hi |= v << (pos2 - 64);
}

// NT > 0: compile-time n (unrolled stores); NT == 0: runtime n
// Chunk c = block kb of row c / nkb: mask bits and codes go row-major, the
// packed stream and the N:M metadata panel-major (panel_offset).
template <int NT, int M>
__device__ __forceinline__ void store_outputs(const ChunkOut& o, int64_t c, int n_rt,
                                              uint8_t* mask, int8_t* codes, int fmt,
                                              uint8_t* packed, uint8_t* meta, int64_t n_out, int nkb) {
  const int n = NT > 0 ? NT : n_rt;
  constexpr int m = M;
  if (mask) reinterpret_cast<uint2*>(mask)[c] = make_uint2((uint32_t)o.keep, (uint32_t)(o.keep >> 32));
  if (codes) {
    uint4* cp = reinterpret_cast<uint4*>(codes) + c * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) cp[i] = make_uint4(o.cb[4 * i], o.cb[4 * i + 1], o.cb[4 * i + 2], o.cb[4 * i + 3]);
  }
  if (!packed) return;
  const uint32_t row = (uint32_t)c / (uint32_t)nkb, kb = (uint32_t)c - row * (uint32_t)nkb;   // c < 2^28
  if (fmt == 0) {
    *reinterpret_cast<uint4*>(packed + panel_offset(n_out, nkb, 16, row, kb)) =
        make_uint4(o.d2[0], o.d2[1], o.d2[2], o.d2[3]);
    return;
  }
  if (meta)
    *reinterpret_cast<uint2*>(meta + panel_offset(n_out, nkb, 8, row, kb)) =
        make_uint2((uint32_t)o.keep, (uint32_t)(o.keep >> 32));
  const int bytes = 16 * n / m;             // even; a multiple of 4 unless m == 8 and n is odd
  uint8_t* const dst = packed + panel_offset(n_out, nkb, bytes, row, kb);
  const uint32_t w[4] = {(uint32_t)o.nm_lo, (uint32_t)(o.nm_lo >> 32), (uint32_t)o.nm_hi,
                         (uint32_t)(o.nm_hi >> 32)};
  if ((bytes & 3) == 0) {
    uint32_t* p = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < bytes / 4) p[i] = w[i];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < bytes / 2) p[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
  }
}

// Loads are staged through LDS: the workgroup reads 256 consecutive chunks
// (32 KB) with lane-contiguous 16-byte loads, then each thread reads its own
// 128-byte chunk back (rows padded to 144 bytes: conflict-free).
constexpr int kPad = 144;

__device__ __forceinline__ int find_item(const QBatch& b) {
  int di = 0;
  for (int i = 1; i < b.count; ++i)
    if ((int64_t)blockIdx.x >= b.start[i]) di = i;
  return di;
}

// Words of chunk c0 + threadIdx.x (word i = weights 2i, 2i+1), for a workgroup
// whose chunks start at c0; `cnt` chunks exist from c0 on.
__device__ __forceinline__ void load_chunk(const u32x4* __restrict__ w, int64_t c0, int64_t cnt,
                                           uint8_t* stage, uint32_t (&dw)[32]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v16 = tid + kThreads * i;                    // 16-byte unit within the block
    if (v16 < cnt * 8) {
      const u32x4 v = ld_stream16(&w[c0 * 8 + v16]);
      *reinterpret_cast<u32x4*>(&stage[(v16 >> 3) * kPad + 16 * (v16 & 7)]) = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[tid * kPad + 16 * i]);
    dw[4 * i] = v[0]; dw[4 * i + 1] = v[1]; dw[4 * i + 2] = v[2]; dw[4 * i + 3] = v[3];
  }
}

constexpr int kCPT = 2;   // chunk groups per workgroup of the fused mask/pack kernel

// LDS-direct staging for the fused kernel: a group of kThreads chunks (32 KB)
// goes straight from memory into `stage` with buffer_load ... lds, no
// registers in between.  Wave w issues blocks q = 8w .. 8w+7 of 1 KB; lane l
// of block q fetches chunk 8q + l/8, 16-byte piece (l%8) ^ (l/8), which lands
// at byte 16*l of the block, so piece p of chunk row r sits at
// r*128 + 16*(p ^ (r%8)): the eight rows that eight consecutive threads read
// fall in distinct 16-byte bank groups.  Offsets past the resource (chunks
// beyond the matrix) read zeros.  The loads are counted by vmcnt; the data is
// visible to the workgroup after s_waitcnt vmcnt(0) and a barrier.  The
// masters are read once here: nontemporal cache policy (13B block: 112 µs
// instead of 141 µs with the default policy).
constexpr int kNt = 2;   // cache-policy bit "nt" of the buffer instruction
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, kNt);
}

__device__ __forceinline__ void dma_group(__amdgpu_buffer_rsrc_t rw, uint32_t chunk0, uint8_t* stage) {
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t piece = (lane & 7u) ^ (lane >> 3);
#pragma unroll
  for (uint32_t q = 0; q < 8; ++q) {
    const uint32_t blk = 8u * wave + q;
    dma16(rw, stage + 1024u * blk, (chunk0 + 8u * blk + (lane >> 3)) * 128u + 16u * piece);
  }
}

// this thread's chunk (row threadIdx.x of the staged group)
__device__ __forceinline__ void read_group(const uint8_t* stage, uint32_t (&dw)[32]) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (uint32_t i = 0; i < 8; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[t * 128u + 16u * (i ^ (t & 7u))]);
    dw[4 * i] = v[0]; dw[4 * i + 1] = v[1]; dw[4 * i + 2] = v[2]; dw[4 * i + 3] = v[3];
  }
}

constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0) (expcnt, lgkmcnt: no wait)

using namespace sel;

// four 2-bit values in bytes 0..3 -> bits 0..7
__device__ __forceinline__ uint32_t bytes_to_fields(uint32_t p) {
  const uint32_t t = p | (p >> 6);
  return (t | (t >> 12)) & 0xFFu;
}

// delete the 2-bit field number pos of x (higher fields move down)
__device__ __forceinline__ uint32_t remove_field(uint32_t x, uint32_t pos) {
  const uint32_t low = (1u << (2 * pos)) - 1u;
  return (x & low) | ((x >> 2) & ~low);
}

// FMT: format computed for `packed` (0 DENSE2, 1 N:M); CODES: int8 codes wanted;
// PRESEL: the keep bits are given (keep64, bit j = weight j of the chunk)
// instead of selected here.  get_words(g, W) supplies the M/2 words of group g.
template <int M, int DROP, int FMT, bool CODES, bool PRESEL, class GetWords>
__device__ __forceinline__ void mask_pack_chunk_from(GetWords get_words, int64_t c, const QDesc& d, uint32_t t2,
                                                     uint64_t keep64) {
  constexpr int N = M - DROP, WPG = M / 2;
  constexpr bool want_d2 = FMT == 0, want_nm = FMT == 1, want_codes = CODES;
  const uint32_t ones = opaque(kOnes);
  ChunkOut o = {};
  uint32_t nmw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < 64 / M; ++g) {
    uint32_t W[WPG];
    get_words(g, W);
    uint32_t A[WPG], F[WPG];
#pragma unroll
    for (int i = 0; i < WPG; ++i) A[i] = W[i] & 0x7FFF7FFFu;
    uint32_t keep;
    if constexpr (PRESEL) {
      keep = (uint32_t)(keep64 >> (g * M)) & ((1u << M) - 1u);
      scatter_bits<M>(keep, F);
    } else {
      keep = select_keep<M, DROP>(A, F, ones);
    }
    o.keep |= (uint64_t)keep << (g * M);
    // per half: index = G + 2*sign, G = (kept and mag > t); u = c + 1 = {1, 2, 1, 0}[index]
    uint32_t X[WPG];
#pragma unroll
    for (int i = 0; i < WPG; ++i) {
      const uint32_t G = pmin(psubsat(A[i], t2), F[i]);
      X[i] = ((W[i] >> 14) & 0x00020002u) | G;
    }
    uint32_t fields = 0;                               // u of the group, 2 bits each
#pragma unroll
    for (int q = 0; q < M / 4; ++q) {
      // bytes = index of weights 4q .. 4q+3, then u through the byte table
      const uint32_t idx = __builtin_amdgcn_perm(X[2 * q + 1], X[2 * q], 0x06040200u);
      const uint32_t P = __builtin_amdgcn_perm(0u, 0x00010201u, idx);
      const int p = g * M + 4 * q;                     // first weight of the quad
      if (want_d2) o.d2[p >> 4] |= P << (2 * ((p >> 2) & 3));
      if (want_codes) o.cb[p >> 2] = ((P | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
      if (want_nm) fields |= bytes_to_fields(P) << (8 * q);
    }
    if (want_nm) {
      const uint32_t dm = ~keep & ((1u << M) - 1u);    // dropped positions
      if constexpr (DROP == 2) fields = remove_field(fields, 31 - __builtin_clz(dm));
      if constexpr (DROP >= 1) fields = remove_field(fields, __builtin_ctz(dm));
      const int off = g * 2 * N, wi = off >> 5, sh = off & 31;
      nmw[wi] |= fields << sh;
      if (sh + 2 * N > 32) nmw[wi + 1] |= fields >> (32 - sh);
    }
  }
  o.nm_lo = (uint64_t)nmw[0] | ((uint64_t)nmw[1] << 32);
  o.nm_hi = (uint64_t)nmw[2] | ((uint64_t)nmw[3] << 32);
  store_outputs<N, M>(o, c, N, d.mask, d.codes, FMT, d.packed, d.meta, d.n_out, d.nkb);
}

// The same for a chunk held in registers (word i = weights 2i, 2i+1).
template <int M, int DROP, int FMT, bool CODES>
__device__ __forceinline__ void mask_pack_chunk(const uint32_t (&dw)[32], int64_t c, const QDesc& d, uint32_t t2) {
  mask_pack_chunk_from<M, DROP, FMT, CODES, false>(
      [&](int g, uint32_t* W) {
#pragma unroll
        for (int i = 0; i < M / 2; ++i) W[i] = dw[g * (M / 2) + i];
      },
      c, d, t2, 0);
}

// A workgroup takes kCPT consecutive groups of kThreads chunks; the next
// group's LDS-direct loads are in flight while the current one is computed.
// beta is finalized at the start, while the first group's loads are in flight.
template <int M, int DROP, int FMT, bool CODES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void mask_pack_fast_kernel(
    const QBatch batch) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads * 128];
  const int di = find_item(batch);
  const QDesc& d = batch.d[di];
  const int64_t nchunks = d.nvec / 8;
  const int64_t lwg = (int64_t)blockIdx.x - batch.start[di];
  const int64_t g0 = lwg * kThreads * kCPT;
  const int64_t span = nchunks - g0 < (int64_t)kThreads * kCPT ? nchunks - g0 : (int64_t)kThreads * kCPT;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.w + 8 * g0, span * 128);
  // beta's inputs are loaded first, so that it is computed while the chunk
  // loads are in flight (loads complete in issue order)
  beta::SlotLoads sl = {};
  if (!batch.beta_ready) sl = beta::load_slots(d);
  dma_group(rw, 0, stage);
  const float b = fmaxf(batch.beta_ready ? d.beta[0] : beta::finish_beta(d, sl, lwg == 0), 1e-5f);
  const uint32_t t2 = (__float_as_uint(b * 0.5f) >> 16) * kOnes;   // |w| > beta_eff/2 <=> mag > t
#pragma unroll
  for (int j = 0; j < kCPT; ++j) {
    const int64_t cg = g0 + (int64_t)j * kThreads;
    uint32_t dw[32];
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();                                  // group j is in LDS
    read_group(stage, dw);
    if (j + 1 < kCPT) {
      __syncthreads();                                // every thread has its chunk in registers
      dma_group(rw, (uint32_t)((j + 1) * kThreads), stage);
    }
    const int64_t c = cg + threadIdx.x;
    if (c < nchunks) {
      // group scales (beta complete before the launch): the beta of this chunk's group
      const uint32_t tc =
          d.beta_rows > 0 ? (__float_as_uint(fmaxf(d.beta[chunk_beta_index(d, c)], 1e-5f) * 0.5f) >> 16) * kOnes : t2;
      mask_pack_chunk<M, DROP, FMT, CODES>(dw, c, d, tc);
    }
  }
}

template <int M, int DROP, int FMT, bool CODES>
void launch_fast_kernel(const QBatch& b, hipStream_t s) {
  hipLaunchKernelGGL((mask_pack_fast_kernel<M, DROP, FMT, CODES>), dim3((unsigned)b.start[b.count]),
                     dim3(kThreads), 0, s, b);
}

template <int M, int DROP>
void launch_fast(const QBatch& b, hipStream_t s) {
  bool codes = false, nm = false;
  for (int i = 0; i < b.count; ++i) {
    codes = codes || b.d[i].codes != nullptr;
    nm = nm || (b.d[i].packed != nullptr && b.d[i].fmt == 1);
  }
  if (nm && codes) launch_fast_kernel<M, DROP, 1, true>(b, s);
  else if (nm) launch_fast_kernel<M, DROP, 1, false>(b, s);
  else if (codes) launch_fast_kernel<M, DROP, 0, true>(b, s);
  else launch_fast_kernel<M, DROP, 0, false>(b, s);
}

// ---------------------------------------------------------------- resident: one launch
// The whole weight preparation of a batch in one launch, for batches whose
// masters fit in the registers of one round of workgroups (the two-pass path
// reads them twice: beta must be complete before any code is known).
// Workgroup j of a matrix holds chunks [cpw j, cpw j + cpw) in registers
// (cpw = d.vpt <= 1024; thread t: 16-byte vectors t + 256u, u < 32, so each
// load instruction of a wave reads 1 KB contiguous), adds their magnitudes exactly, publishes its
// partial sum in slot j (sbl_partial.h) and then waits until every slot of
// its matrix is complete for this call.  The N:M selection does not depend on
// beta, so it is made in the first phase, vector by vector as the loads
// arrive (a 16-byte vector is one group of 8, or two of 4).  Then beta is
// finalized per wave (sbl_beta.h) and the chunks, with their keep bits, go
// through LDS (the same swizzled layout as the LDS-direct staging above) to
// the mask/pack code of the two-pass kernel, minus its selection.
//
// Completion of a slot for a call (no workspace initialization needed, and
// graph replays of one launch stay distinct):
//  * the workspace holds a generation word; a workgroup reads it at its start
//    and targets e = generation + 1;
//  * a slot is complete for target e when its tag equals tag(e, matrix, slot),
//    a bijection of e for a fixed slot (tags of earlier calls differ);
//  * every workspace word is stored and loaded as a relaxed agent-scope
//    atomic (coherent across the XCDs' L2 caches without cache-wide
//    writebacks or invalidates, which would serialize over hundreds of
//    workgroups); the slot's owner stores the sum and record, waits until
//    those stores are complete (s_waitcnt vmcnt(0)), then stores the tag, so
//    a waiter that has seen the tag reads the sum and record it tags;
//  * the wait is bounded in time: after max_ticks ticks of the chip's
//    constant real-time counter (s_memrealtime; 100 ticks per microsecond on
//    MI355X, the rate the host reads from the device) a workgroup computes the
//    missing partial sums itself from the masters, stores and tags them.  The
//    sums are exact, so every writer of a slot writes the same bits, and a
//    result never depends on who computed it.  (The host launches this
//    kernel only when the occupancy of the chip holds every workgroup at
//    once; the bound covers the case where other work delays some of them.)
//  * after its wait, workgroup 0 of the matrix, and every workgroup that
//    computed a missing sum, moves the generation from e - 1 to e (compare
//    and swap).  Every owner has read the generation before its tag exists,
//    so no workgroup that waits on its own reads it after the move; a late
//    one (started after the move) targets e + 1, completes every slot for it
//    (waiting or computing) and moves the generation on.  The next call thus
//    always targets a value above every tag written so far.
constexpr int kResR = kResChunksPerThread;        // chunks per thread held in registers
constexpr int kResChunks = kThreads * kResR;      // chunks per workgroup
static_assert(kResChunks == kResChunksPerWg, "resident partition");
constexpr int kResMaxSlots = beta::kWaveSlots;    // slots per matrix (the per-wave finalize)

// The mix is the published SplitMix64 output function (golden-ratio
// increment, then two xor-shift-multiply rounds with its constants): odd
// multipliers and xor-shifts, so bijective in e for a fixed slot.
__device__ __forceinline__ uint64_t res_tag(uint64_t e, const QDesc& d, int64_t slot) {
  uint64_t x = e + ((uint64_t)(uintptr_t)d.w ^ ((uint64_t)slot * 0x9E3779B97F4A7C15ull));
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tag store of a slot whose sum and record this thread has just stored:
// they are complete before the tag is written.
__device__ __forceinline__ void res_store_tag(uint64_t* p, uint64_t tag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  beta::ws_store<true>(p, tag);
}

// Slot j's partial sum straight from the masters (a workgroup that stopped
// waiting for it); stores and tags it like its owner.  All threads call it.
__device__ __forceinline__ void res_compute_slot(const QDesc& d, int64_t j, uint64_t tag, unsigned long long* bins) {
  const int64_t nchunks = d.nvec / 8, c0 = j * d.vpt;
  const int64_t span = nchunks - c0 < d.vpt ? nchunks - c0 : d.vpt;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.w + 8 * c0, span * 128);
  __syncthreads();                                   // earlier users of bins are done
  bins[threadIdx.x] = 0;
  __syncthreads();
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
#pragma unroll 1
  for (int u = 0; u < 8 * kResR; u += 4) {
    u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rw, (threadIdx.x + kThreads * (u + q)) * 16, 0, 0));
#pragma unroll
    for (int q = 0; q < 4; ++q) part::consume(v[q], acc0, acc1, bins, rare);
  }
  part::publish_partial<true>(d.ws, d.nb, j, acc0, acc1, rare, bins);
  if (threadIdx.x == 0) res_store_tag(d.ws + ws_res_gen(d.nb) + 1 + j, tag);
}

template <int M, int DROP, int FMT, bool CODES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void resident_kernel(
    const QBatch batch, uint32_t max_ticks) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads * 128];
  __shared__ __attribute__((aligned(8))) uint8_t kstage[kResR][kThreads * 8];   // keep bits, per chunk row
  __shared__ unsigned long long bins[256];
  __shared__ unsigned long long missing[kResMaxSlots / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int di = find_item(batch);
  const QDesc& d = batch.d[di];
  const int64_t slot = (int64_t)blockIdx.x - batch.start[di];
  const int64_t c0 = slot * d.vpt;
  const int64_t span = d.nvec / 8 - c0 < d.vpt ? d.nvec / 8 - c0 : d.vpt;
  const int64_t cend = c0 + span;                    // this workgroup's chunks: [c0, cend)
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.w + 8 * c0, span * 128);
  uint64_t* const gen = d.ws + ws_res_gen(d.nb);
  uint64_t* const tags = gen + 1;
  bins[tid] = 0;
  __syncthreads();
  const uint64_t e = load_agent(gen) + 1;            // this call's target
  u32x4 v[8 * kResR];
#pragma unroll
  for (int u = 0; u < 8 * kResR; ++u)
    v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (tid + kThreads * u) * 16, 0, kNt));
  // the magnitudes join the exact sum as the vectors arrive, and the sum is
  // published at once; the N:M selection (which beta does not affect) is made
  // after that, while the other workgroups' sums are still on their way (a
  // vector is one group of 8, or two groups of 4)
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
#pragma unroll
  for (int u = 0; u < 8 * kResR; ++u)
    if (u < 8 || 32 * u + (tid >> 3) < span) part::consume(v[u], acc0, acc1, bins, rare);
  part::publish_partial<true>(d.ws, d.nb, slot, acc0, acc1, rare, bins);
  if (tid == 0) res_store_tag(tags + slot, res_tag(e, d, slot));
  {
    // keep bits of vector u (chunk row r = 32 (u % 8) + tid / 8 of group u / 8,
    // piece tid % 8) go to LDS, read per chunk in the second phase
    const uint32_t ones = opaque(kOnes);
#pragma unroll
    for (int u = 0; u < 8 * kResR; ++u) {
      if (u >= 8 && 32 * u + (tid >> 3) >= span) continue;   // past this workgroup's chunks
      uint32_t A[4], F[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) A[i] = v[u][i] & 0x7FFF7FFFu;
      uint32_t keep;
      if constexpr (M == 8) keep = select_keep<8, DROP>(A, F, ones);
      else keep = select_keep<4, DROP>(A, F, ones) | (select_keep<4, DROP>(A + 2, F + 2, ones) << 4);
      kstage[u >> 3][(32u * (u & 7) + ((uint32_t)tid >> 3)) * 8u + ((uint32_t)tid & 7u)] = (uint8_t)keep;
    }
  }
  // wave 0 waits for the other slots (lane l: slots l + 64u).  A lane polls
  // only the tags it has not yet seen complete, and the wave backs off while
  // many are missing: every workgroup of a matrix polls the same few lines,
  // and early finishers would otherwise load them while the masters stream.
  if (tid < 64) {
    uint32_t lane_miss = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int u = 0; u < kResMaxSlots / 64; ++u)
      if (lane + 64 * u < d.nb) lane_miss |= 1u << u;
    for (;;) {
      uint64_t t[kResMaxSlots / 64];                 // the loads in flight together, then the compares
#pragma unroll
      for (int u = 0; u < kResMaxSlots / 64; ++u)
        t[u] = ((lane_miss >> u) & 1u) ? load_agent(tags + lane + 64 * u) : 0ull;
#pragma unroll
      for (int u = 0; u < kResMaxSlots / 64; ++u)
        if (((lane_miss >> u) & 1u) && t[u] == res_tag(e, d, lane + 64 * u)) lane_miss &= ~(1u << u);
      const unsigned long long waiting = __ballot(lane_miss != 0);
      if (waiting == 0 || __builtin_amdgcn_s_memrealtime() - t0 >= max_ticks) break;   // uniform in the wave
      if (__popcll(waiting) > 8) __builtin_amdgcn_s_sleep(32);   // ~2000 cycles
      else __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int u = 0; u < kResMaxSlots / 64; ++u) {
      const unsigned long long mu = __ballot((lane_miss >> u) & 1u);
      if (lane == 0) missing[u] = mu;
    }
  }
  __syncthreads();
  bool helped = false;
#pragma unroll 1
  for (int u = 0; u < kResMaxSlots / 64; ++u) {
    unsigned long long mu = missing[u];
    while (mu) {                                     // uniform: LDS value
      const int64_t j = 64 * u + __ffsll(mu) - 1;
      mu &= mu - 1;
      res_compute_slot(d, j, res_tag(e, d, j), bins);
      helped = true;
    }
  }
  __syncthreads();                                   // every slot is tagged for e (seen or computed)
  if (tid == 0 && (slot == 0 || helped)) {
    uint64_t expected = e - 1;
    __hip_atomic_compare_exchange_strong(gen, &expected, e, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  const float b = fmaxf(beta::finish_beta<true>(d, beta::load_slots<true>(d), slot == 0), 1e-5f);
  if (!d.mask && !d.codes && !d.packed) return;      // beta only (uniform)
  const uint32_t t2 = (__float_as_uint(b * 0.5f) >> 16) * kOnes;   // |w| > beta_eff/2 <=> mag > t
  const uint32_t sw = (uint32_t)(tid >> 3) & 7u;
#pragma unroll
  for (int g = 0; g < kResR; ++g) {
    if (c0 + (int64_t)g * kThreads >= cend) break;      // uniform
    if (g) __syncthreads();                           // the previous group has been read
#pragma unroll
    for (int q = 0; q < 8; ++q) {                     // vector tid + 256(8g + q): row 32q + tid/8, piece tid%8
      const int u = 8 * g + q;
      const uint32_t r = 32u * q + ((uint32_t)tid >> 3), pc = (uint32_t)tid & 7u;
      *reinterpret_cast<u32x4*>(&stage[r * 128u + 16u * (pc ^ sw)]) = v[u];
    }
    __syncthreads();
    const uint2 kk = *reinterpret_cast<const uint2*>(&kstage[g][tid * 8]);
    const int64_t c = c0 + (int64_t)g * kThreads + tid;
    // this thread's chunk is row tid of the stage (piece p at 16 (p ^ tid % 8));
    // group q of it is read when needed
    const uint8_t* row = stage + tid * 128u;
    if (c < cend)
      mask_pack_chunk_from<M, DROP, FMT, CODES, true>(
          [&](int q, uint32_t* W) {
            const uint32_t off = 16u * ((uint32_t)(q * M / 8) ^ ((uint32_t)tid & 7u)) + (M == 4 ? 8u * (q & 1) : 0u);
            if constexpr (M == 8) {
              const u32x4 x = *reinterpret_cast<const u32x4*>(row + off);
              W[0] = x[0]; W[1] = x[1]; W[2] = x[2]; W[3] = x[3];
            } else {
              const uint2 x = *reinterpret_cast<const uint2*>(row + off);
              W[0] = x.x; W[1] = x.y;
            }
          },
          c, d, t2, (uint64_t)kk.x | ((uint64_t)kk.y << 32));
  }
}

// Partition of a batch over `cap` co-resident workgroups: every matrix gets
// whole workgroups of cpw chunks, cpw the same for the batch and as small as
// the co-resident workgroups allow, so that every CU gets about the same
// share of the loads and of the selection work of the first phase (the
// slowest workgroup of a matrix holds up all the others); at most
// kResChunks (registers), and the slots must fit in the workspace.
bool res_partition(QBatch& b, int64_t cap) {
  int64_t total = 0;
  for (int i = 0; i < b.count; ++i) total += b.d[i].nvec / 8;
  if (cap <= b.count) return false;
  int64_t cpw = (total + (cap - b.count) - 1) / (cap - b.count);
  cpw = cpw < kThreads ? kThreads : (cpw + 7) / 8 * 8;
  if (cpw > kResChunks) return false;
  int64_t blocks = 0;
  for (int i = 0; i < b.count; ++i) {
    const int64_t nb = (b.d[i].nvec / 8 + cpw - 1) / cpw;
    if (nb > kResMaxSlots || ws_res_words(nb) > b.d[i].ws_words) return false;
    b.d[i].nb = nb;
    b.d[i].vpt = cpw;
    b.start[i] = blocks;
    blocks += nb;
  }
  b.start[b.count] = blocks;
  return blocks <= cap;
}

template <int M, int DROP, int FMT, bool CODES>
bool launch_resident_kernel(QBatch& b, uint32_t max_ticks, hipStream_t s, hipError_t* err) {
  static int capacity[64];                           // co-resident workgroups per device (0: unknown)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (capacity[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_kernel<M, DROP, FMT, CODES>, kThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return false;
    capacity[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
  }
  QBatch r = b;
  if (!res_partition(r, capacity[dev])) return false;
  hipLaunchKernelGGL((resident_kernel<M, DROP, FMT, CODES>), dim3((unsigned)r.start[r.count]), dim3(kThreads), 0,
                     s, r, max_ticks);
  *err = hipGetLastError();
  b = r;
  return true;
}

template <int M, int DROP>
bool launch_resident_m(QBatch& b, uint32_t max_ticks, hipStream_t s, hipError_t* err) {
  bool codes = false, nm = false;
  for (int i = 0; i < b.count; ++i) {
    codes = codes || b.d[i].codes != nullptr;
    nm = nm || (b.d[i].packed != nullptr && b.d[i].fmt == 1);
  }
  if (nm && codes) return launch_resident_kernel<M, DROP, 1, true>(b, max_ticks, s, err);
  if (nm) return launch_resident_kernel<M, DROP, 1, false>(b, max_ticks, s, err);
  if (codes) return launch_resident_kernel<M, DROP, 0, true>(b, max_ticks, s, err);
  return launch_resident_kernel<M, DROP, 0, false>(b, max_ticks, s, err);
}

// Any n (one thread per chunk, one sort key per weight).
// mfc: the keys rank |code| (nonzero or not) instead of |w| (the masks-from-
// quantized-weights ablation; ties still go to the lower index).
template <int M>
__global__ __launch_bounds__(kThreads) void mask_pack_kernel(const QBatch batch, int n, int mfc) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads * kPad];
  constexpr int SH = (M == 8) ? 3 : 2;
  const int di = find_item(batch);
  const QDesc& d = batch.d[di];
  const int64_t nchunks = d.nvec / 8;
  uint8_t* __restrict__ packed = d.packed;
  const int fmt = d.fmt;
  const int64_t lwg = (int64_t)blockIdx.x - batch.start[di];
  const float b = fmaxf(batch.beta_ready ? d.beta[0] : beta::workgroup_beta(d, lwg == 0), 1e-5f);
  int thr_mag = (int)(__float_as_uint(b * 0.5f) >> 16);
  const bool want_nm = packed && fmt == 1;
  {
    const int64_t c0 = lwg * kThreads;
    const int64_t cnt = nchunks - c0 < kThreads ? nchunks - c0 : kThreads;   // chunks in this block
    uint32_t dw[32];
    load_chunk(d.w, c0, cnt, stage, dw);
    const int64_t c = c0 + threadIdx.x;
    if (c >= nchunks) return;
    if (d.beta_rows > 0)                             // group scales: the beta of this chunk's group
      thr_mag = (int)(__float_as_uint(fmaxf(d.beta[chunk_beta_index(d, c)], 1e-5f) * 0.5f) >> 16);
    ChunkOut o = {};
#pragma unroll
    for (int g = 0; g < 64 / M; ++g) {
      int key[M];
      uint32_t sgn[M];
      bool nzc[M];                                   // code nonzero before the mask: |w| > beta_eff/2
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int idx = g * M + j;
        const uint32_t h = (idx & 1) ? (dw[idx >> 1] >> 16) : (dw[idx >> 1] & 0xFFFFu);
        nzc[j] = (int)(h & 0x7FFFu) > thr_mag;
        const uint32_t rank_mag = mfc ? (nzc[j] ? 1u : 0u) : (h & 0x7FFFu);
        key[j] = (int)((rank_mag << SH) | (uint32_t)(M - 1 - j));
        sgn[j] = h >> 15;
      }
      const int thr = group_threshold<M>(key, n);
      int kept = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int idx = g * M + j;
        const bool keep = key[j] > thr;
        const bool nz = keep && nzc[j];
        const uint32_t u = nz ? (sgn[j] ? 0u : 2u) : 1u;
        o.d2[idx >> 4] |= u << d2_shift(idx);
        o.keep |= (uint64_t)keep << idx;
        o.cb[idx >> 2] |= ((u - 1u) & 0xFFu) << (8 * (idx & 3));
        if (want_nm && keep) {
          nm_insert(o, u, 2 * (g * n + kept));
          ++kept;
        }
      }
    }
    store_outputs<0, M>(o, c, n, d.mask, d.codes, fmt, packed, d.meta, d.n_out, d.nkb);
  }
}

// Packing of caller-supplied codes (+ mask for N:M).
template <int M>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint4* __restrict__ codes, const uint2* __restrict__ maskv,
                                                        int64_t n_out, int nkb, int n, int fmt,
                                                        uint8_t* __restrict__ packed,
                                                        uint8_t* __restrict__ meta) {
  const int64_t nchunks = n_out * nkb;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    uint32_t cw[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = codes[c * 4 + i];
      cw[4 * i] = v.x; cw[4 * i + 1] = v.y; cw[4 * i + 2] = v.z; cw[4 * i + 3] = v.w;
    }
    uint64_t keep = 0;
    if (fmt == 1) {
      const uint2 mv = maskv[c];
      keep = (uint64_t)mv.x | ((uint64_t)mv.y << 32);
    }
    ChunkOut o = {};
    o.keep = keep;
#pragma unroll
    for (int g = 0; g < 64 / M; ++g) {
      int kept = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int idx = g * M + j;
        const uint32_t u = ((cw[idx >> 2] >> (8 * (idx & 3))) + 1u) & 3u;
        o.d2[idx >> 4] |= u << d2_shift(idx);
        if (fmt == 1 && ((keep >> idx) & 1) && kept < n) {
          nm_insert(o, u, 2 * (g * n + kept));
          ++kept;
        }
      }
      for (; fmt == 1 && kept < n; ++kept) nm_insert(o, 1u, 2 * (g * n + kept));
    }
    store_outputs<0, M>(o, c, n, nullptr, nullptr, fmt, packed, meta, n_out, nkb);
  }
}

int64_t grid_for(int64_t nchunks) {
  int64_t blocks = (nchunks + kThreads - 1) / kThreads;
  return blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks);
}

}  // namespace

hipError_t launch_mask_pack(QBatch& b, int n, int m, hipStream_t s, bool dry, int64_t* grid_out,
                            bool mask_from_codes) {
  const int drop = m - n;
  bool grouped = false;                              // group scales: beta per row group, complete beforehand
  for (int i = 0; i < b.count; ++i) grouped = grouped || b.d[i].beta_rows > 0;
  const bool fast = drop <= 2 && !mask_from_codes && (!grouped || b.beta_ready);
  const int64_t per_block = fast ? (int64_t)kThreads * kCPT : kThreads;   // chunks per workgroup
  int64_t blocks = 0;
  for (int i = 0; i < b.count; ++i) {
    b.start[i] = blocks;
    blocks += (b.d[i].nvec / 8 + per_block - 1) / per_block;
  }
  b.start[b.count] = blocks;
  if (grid_out) *grid_out = blocks;
  if (dry) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (!fast && m == 8) hipLaunchKernelGGL((mask_pack_kernel<8>), grid, block, 0, s, b, n, mask_from_codes ? 1 : 0);
  else if (!fast) hipLaunchKernelGGL((mask_pack_kernel<4>), grid, block, 0, s, b, n, mask_from_codes ? 1 : 0);
  else if (m == 8 && drop == 0) launch_fast<8, 0>(b, s);
  else if (m == 8 && drop == 1) launch_fast<8, 1>(b, s);
  else if (m == 8 && drop == 2) launch_fast<8, 2>(b, s);
  else if (m == 4 && drop == 0) launch_fast<4, 0>(b, s);
  else if (m == 4 && drop == 1) launch_fast<4, 1>(b, s);
  else if (m == 4 && drop == 2) launch_fast<4, 2>(b, s);
  return hipGetLastError();
}

bool launch_resident(QBatch& b, int n, int m, uint32_t max_ticks, hipStream_t s, hipError_t* err) {
  const int drop = m - n;
  if (m == 8 && drop == 0) return launch_resident_m<8, 0>(b, max_ticks, s, err);
  if (m == 8 && drop == 1) return launch_resident_m<8, 1>(b, max_ticks, s, err);
  if (m == 8 && drop == 2) return launch_resident_m<8, 2>(b, max_ticks, s, err);
  if (m == 4 && drop == 0) return launch_resident_m<4, 0>(b, max_ticks, s, err);
  if (m == 4 && drop == 1) return launch_resident_m<4, 1>(b, max_ticks, s, err);
  if (m == 4 && drop == 2) return launch_resident_m<4, 2>(b, max_ticks, s, err);
  return false;
}

hipError_t launch_pack(const int8_t* codes, const uint8_t* mask, int64_t n_out, int64_t k, int n, int m,
                       int fmt, uint8_t* packed, uint8_t* meta, hipStream_t s) {
  const int nkb = (int)(k / kChunk);
  const int64_t nchunks = n_out * nkb;
  const dim3 grid((unsigned)grid_for(nchunks)), block(kThreads);
  const uint4* cv = reinterpret_cast<const uint4*>(codes);
  const uint2* mv = reinterpret_cast<const uint2*>(mask);
  if (m == 8)
    hipLaunchKernelGGL((pack_kernel<8>), grid, block, 0, s, cv, mv, n_out, nkb, n, fmt, packed, meta);
  else
    hipLaunchKernelGGL((pack_kernel<4>), grid, block, 0, s, cv, mv, n_out, nkb, n, fmt, packed, meta);
  return hipGetLastError();
}

}  // namespace sbl
