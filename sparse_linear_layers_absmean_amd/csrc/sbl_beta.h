// Final step of the exact absmean scale: beta = RN_fp32(S / (n_out*k)) from
// the partial sums the absmean pass left in the workspace (layout in
// sbl_internal.h).  Every workgroup that needs beta computes it itself at its
// start (the sums are a few KB, read from L2), so no separate launch sits
// between the two passes; in the normal case each wave does it alone.
//  * No slot flagged (the normal case): the fast-window sums alone, added in
//    registers and rounded once.
//  * Otherwise the flagged slots' exact out-of-window sums join them: their
//    32-bit limbs are added column by column in LDS (a column sum stays below
//    2^44), and one thread carries the columns into a multi-word integer
//    (units of 2^-133).
// No atomics and nothing written to the workspace.
#pragma once

#include "sbl_internal.h"

namespace sbl {
namespace beta {

constexpr uint64_t kRareFlag = 1ull << 63;

// Workspace words are read and written plainly between launches.  Inside the
// one-launch kernel, where workgroups on different XCDs (each with its own L2)
// exchange them, they are accessed as relaxed agent-scope atomics instead:
// those loads and stores are coherent across the XCDs by themselves, with no
// cache-wide writeback or invalidate.
template <bool AGENT>
__device__ __forceinline__ uint64_t ws_load(const uint64_t* p) {
  if constexpr (AGENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool AGENT>
__device__ __forceinline__ void ws_store(uint64_t* p, uint64_t v) {
  if constexpr (AGENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// limbs: little-endian 32-bit words of a nonnegative integer (units of
// 2^-133); arrays hold kLimbs + 2 words, since add_shifted touches the two
// words above the one it starts in (the sum itself stays below 2^384)
constexpr int kLimbs = 12;

__device__ inline void add_shifted(uint32_t* L, uint64_t v, int s) {
  if (v == 0) return;
  const int li = s >> 5, sh = s & 31;
  const uint64_t lo = v << sh;
  const uint32_t hi = sh ? (uint32_t)(v >> (64 - sh)) : 0u;
  uint64_t t = (uint64_t)L[li] + (uint32_t)lo;
  L[li] = (uint32_t)t;
  t = (uint64_t)L[li + 1] + (uint32_t)(lo >> 32) + (t >> 32);
  L[li + 1] = (uint32_t)t;
  t = (uint64_t)L[li + 2] + hi + (t >> 32);
  L[li + 2] = (uint32_t)t;
  for (int i = li + 3; i < kLimbs && (t >> 32); ++i) {
    t = (uint64_t)L[i] + (t >> 32);
    L[i] = (uint32_t)t;
  }
}

// RN_fp32(D / n) for a dividend D = W * 2^e + r, 0 <= r < 2^e, with bit 63 of
// W set, r != 0 exactly when `sticky`, and 1 <= n <= 2^34.  floor(D / (n*2^e))
// = floor(W / n) = Q (since R + r/2^e < n), and Q >= 2^29 holds more than the
// 24 bits + guard that rounding needs; whatever is below is only a sticky
// flag (with n >= 1, Q < 2^64 as well).  Nearest, ties to even, subnormal
// results included.
__device__ inline float round_div(uint64_t W, int e, bool sticky, uint64_t n) {
  const uint64_t Q = W / n, R = W - Q * n;
  sticky = sticky || R != 0;
  const int qb = 64 - __clzll((long long)Q);        // 30 <= qb <= 64
  int lsb = qb - 24;                                // fp32 unit inside Q for a normal result
  if (e + lsb < -149) lsb = -149 - e;               // subnormal: the unit is 2^-149
  if (lsb > qb) return 0.0f;                        // below half the smallest subnormal
  const uint64_t mant = Q >> lsb;
  const uint64_t guard = (Q >> (lsb - 1)) & 1u;
  sticky = sticky || (Q & ((1ull << (lsb - 1)) - 1u)) != 0;
  const uint64_t m = mant + ((guard && (sticky || (mant & 1u))) ? 1u : 0u);
  return ldexpf((float)m, e + lsb);
}

// exact RN_fp32(S * 2^-133 / n) for the integer S held in limbs
__device__ inline float round_quotient(const uint32_t* L, uint64_t n) {
  int top = -1;
  for (int i = kLimbs - 1; i >= 0 && top < 0; --i)
    if (L[i]) top = i * 32 + 31 - __clz(L[i]);
  if (top < 0) return 0.0f;
  // 64-bit window of S whose bit 63 is S's bit `top`; lower bits: sticky
  const int lo = top - 63;
  uint64_t win;
  bool below = false;
  if (lo >= 0) {
    const int li = lo >> 5, sh = lo & 31;
    const uint64_t a = (uint64_t)L[li] | ((uint64_t)L[li + 1] << 32);
    const uint64_t c = (li + 2 < kLimbs) ? L[li + 2] : 0u;
    win = (a >> sh) | (sh ? (c << (64 - sh)) : 0u);
    for (int i = 0; i < li && !below; ++i) below = L[i] != 0;
    below = below || (L[li] & ((1u << sh) - 1u)) != 0;
  } else {
    win = ((uint64_t)L[0] | ((uint64_t)L[1] << 32)) << (-lo);
  }
  return round_div(win, lo - 133, below, n);
}

// The same for S = V * 2^95 (fast-window sums only), V = hi * 2^32 + lo with
// lo, hi < 2^62: registers only.
__device__ inline float round_quotient_fast(uint64_t lo, uint64_t hi, uint64_t n) {
  const uint64_t vlo = lo + (hi << 32);
  const uint64_t vhi = (hi >> 32) + (vlo < lo ? 1u : 0u);
  if (vlo == 0 && vhi == 0) return 0.0f;
  const int top = vhi ? 127 - __clzll((long long)vhi) : 63 - __clzll((long long)vlo);
  if (top <= 63) return round_div(vlo << (63 - top), top - 63 - 38, false, n);
  const int s = top - 63;                           // 1 .. 63
  const uint64_t W = (vlo >> s) | (vhi << (64 - s));
  return round_div(W, s - 38, (vlo << (64 - s)) != 0, n);
}

// Per-wave finalize (no barrier, no LDS): every wave of a workgroup loads all
// nb <= kWaveSlots partial sums itself, lane l taking slots l + 64u (u < 8),
// so the loads can be issued ahead of LDS-direct loads and beta computed while
// those are in flight (a workgroup barrier would first wait for them).
constexpr int kWaveSlots = 512;
struct SlotLoads {
  uint64_t v[kWaveSlots / 64];
};

template <bool AGENT = false>
__device__ __forceinline__ SlotLoads load_slots(const QDesc& d) {
  SlotLoads sl;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kWaveSlots / 64; ++u) {
    const int64_t i = lane + 64 * u;
    sl.v[u] = i < d.nb ? ws_load<AGENT>(d.ws + i) : 0ull;
  }
  return sl;
}

// Out-of-window path (some slot flagged; uniform across the workgroup):
// beta from the fast-window total V = lo + hi*2^32 (units of 2^-38) and the
// flagged slots' records, whose 32-bit limbs are added column by column in
// LDS (a column sum stays below 2^44); one thread carries the columns into a
// multi-word integer (units of 2^-133).  All threads call it.
template <bool AGENT = false>
__device__ inline float rare_beta(const QDesc& d, unsigned long long lo, unsigned long long hi, bool store) {
  constexpr int kCols = 2 * kWsLimbWords;
  static_assert(kCols == kLimbs, "one column per limb");
  __shared__ unsigned long long cols[kCols];
  __shared__ uint32_t limbs[kLimbs + 2];
  __shared__ float beta_s;
  const int tid = threadIdx.x;
  if (tid < kCols) cols[tid] = 0;
  __syncthreads();
  const uint64_t* recs = d.ws + ws_limb_base(d.nb);
  for (int64_t i = tid; i < d.nb; i += kAbsThreads) {
    if ((ws_load<AGENT>(d.ws + i) >> 63) == 0) continue;
#pragma unroll
    for (int j = 0; j < kWsLimbWords; ++j) {
      const uint64_t w = ws_load<AGENT>(recs + kWsLimbWords * i + j);
      atomicAdd(&cols[2 * j], (unsigned long long)(uint32_t)w);
      atomicAdd(&cols[2 * j + 1], (unsigned long long)(w >> 32));
    }
  }
  __syncthreads();
  if (tid == 0) {
    for (int i = 0; i < kLimbs + 2; ++i) limbs[i] = 0;
    for (int j = 0; j < kCols; ++j) add_shifted(limbs, cols[j], 32 * j);
    add_shifted(limbs, lo, 95);        // 2^-38 = 2^95 * 2^-133
    add_shifted(limbs, hi, 95 + 32);
    const float bt = round_quotient(limbs, (uint64_t)d.count);
    beta_s = bt;
    if (store) d.beta[0] = bt;
  }
  __syncthreads();
  return beta_s;
}

// beta of matrix d (unclamped) from slot values every wave loaded
// (load_slots, nb <= kWaveSlots), returned to every thread.  All threads of
// the workgroup call it; `store` makes this workgroup write d.beta.
template <bool AGENT = false>
__device__ inline float finish_beta(const QDesc& d, const SlotLoads& sl, bool store) {
  // sums split in 32-bit halves so that nothing overflows
  unsigned long long lo = 0, hi = 0;
  uint32_t flags = 0;
#pragma unroll
  for (int u = 0; u < kWaveSlots / 64; ++u) {
    flags |= (uint32_t)(sl.v[u] >> 63);
    lo += (uint32_t)sl.v[u];
    hi += (sl.v[u] & ~kRareFlag) >> 32;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo += __shfl_xor(lo, off, 64);
    hi += __shfl_xor(hi, off, 64);
  }
  if (__ballot(flags != 0) != 0) return rare_beta<AGENT>(d, lo, hi, store);   // uniform
  float b = 0.0f;
  if ((threadIdx.x & 63) == 0) b = round_quotient_fast(lo, hi, (uint64_t)d.count);
  b = __shfl(b, 0, 64);
  if (store && threadIdx.x == 0) d.beta[0] = b;
  return b;
}

// beta of matrix d for any nb <= 4096 (loads included); all threads call it.
__device__ inline float workgroup_beta(const QDesc& d, bool store) {
  if (d.nb <= kWaveSlots) return finish_beta(d, load_slots(d), store);
  __shared__ unsigned long long part[2][kAbsThreads / 64];
  __shared__ uint32_t rare_w[kAbsThreads / 64];
  const int tid = threadIdx.x, wave = tid >> 6;
  unsigned long long lo = 0, hi = 0;
  uint32_t flags = 0;
  for (int64_t i = tid; i < d.nb; i += kAbsThreads) {
    const uint64_t v = d.ws[i];
    flags |= (uint32_t)(v >> 63);
    lo += (uint32_t)v;
    hi += (v & ~kRareFlag) >> 32;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo += __shfl_xor(lo, off, 64);
    hi += __shfl_xor(hi, off, 64);
  }
  const bool any = __ballot(flags != 0) != 0;
  if ((tid & 63) == 0) {
    part[0][wave] = lo;
    part[1][wave] = hi;
    rare_w[wave] = any ? 1u : 0u;
  }
  __syncthreads();
  lo = hi = 0;
  uint32_t flagged = 0;
#pragma unroll
  for (int i = 0; i < kAbsThreads / 64; ++i) {
    lo += part[0][i];
    hi += part[1][i];
    flagged |= rare_w[i];
  }
  if (flagged) return rare_beta(d, lo, hi, store);
  __shared__ float beta_s;
  if (tid == 0) {
    const float b = round_quotient_fast(lo, hi, (uint64_t)d.count);
    beta_s = b;
    if (store) d.beta[0] = b;
  }
  __syncthreads();
  return beta_s;
}

}  // namespace beta
}  // namespace sbl
