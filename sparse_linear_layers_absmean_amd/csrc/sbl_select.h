// N:M keep selection on packed BF16 magnitudes (the fused mask/pack kernel).
//
// Method (Sparse-BitNet, section 2, "Mask Generation"): in every group of m
// consecutive weights along k the n largest BF16 master magnitudes are kept;
// equal magnitudes go to the lower index.  Patterns that drop at most two of
// a group (8:8, 7:8, 6:8, 4:4, 3:4, 2:4) use two magnitudes per 32-bit
// register and v_pk_{min,max,sub}_u16 networks (about 35 operations per group
// of 8); a rare path settles ties that straddle the cut.
#pragma once

#include "sbl_internal.h"

namespace sbl {
namespace sel {

// ---- packed 16-bit helpers: a 32-bit word holds weight 2i (low half) and 2i+1
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kOnes = 0x00010001u;

__device__ __forceinline__ u16x2 h2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t w32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t pmin(uint32_t a, uint32_t b) { return w32(__builtin_elementwise_min(h2(a), h2(b))); }
__device__ __forceinline__ uint32_t pmax(uint32_t a, uint32_t b) { return w32(__builtin_elementwise_max(h2(a), h2(b))); }
// per half: a > b ? a - b : 0
__device__ __forceinline__ uint32_t psubsat(uint32_t a, uint32_t b) { return w32(__builtin_elementwise_sub_sat(h2(a), h2(b))); }
__device__ __forceinline__ uint32_t swap16(uint32_t x) { return __builtin_amdgcn_alignbit(x, x, 16); }
// A register the optimizer cannot see through: min(sub_sat(a, b), 1) with a
// visible 1 is rewritten into per-half compares and selects (6 operations
// per word instead of 2).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// Both halves of the result = the DROP-th smallest magnitude of the group
// (a multiset order statistic), from min/max networks on packed halves.
template <int M, int DROP>
__device__ __forceinline__ uint32_t drop_threshold(const uint32_t* A) {
  uint32_t lo, hi;
  if constexpr (M == 8) {
    const uint32_t a = pmin(A[0], A[1]), b = pmax(A[0], A[1]);
    const uint32_t c = pmin(A[2], A[3]), d = pmax(A[2], A[3]);
    lo = pmin(a, c);                                   // per half: smallest of 4
    hi = pmin(pmax(a, c), pmin(b, d));                 // per half: second smallest of 4
  } else {
    lo = pmin(A[0], A[1]);
    hi = pmax(A[0], A[1]);
  }
  if constexpr (DROP == 1) return pmin(lo, swap16(lo));
  return pmin(pmax(lo, swap16(lo)), pmin(hi, swap16(hi)));
}

// per-half 0/1 flags of the M/2 words of a group -> M-bit mask (bit j = weight j)
template <int M>
__device__ __forceinline__ uint32_t gather_bits(const uint32_t* F) {
  uint32_t m = F[0];
#pragma unroll
  for (int i = 1; i < M / 2; ++i) m |= F[i] << (2 * i);
  return (m | (m >> 15)) & ((1u << M) - 1u);
}

template <int M>
__device__ __forceinline__ void scatter_bits(uint32_t keep, uint32_t* F) {
  const uint32_t x = keep | (keep << 15);
#pragma unroll
  for (int i = 0; i < M / 2; ++i) F[i] = (x >> (2 * i)) & kOnes;
}

// Keep bits (bit j = weight j) of one group from its M/2 words of magnitudes
// (sign bits cleared); F receives the same flags per half (0 or 1).
// `ones` is kOnes through opaque().
template <int M, int DROP>
__device__ __forceinline__ uint32_t select_keep(const uint32_t* A, uint32_t* F, uint32_t ones) {
  constexpr int N = M - DROP, WPG = M / 2;
  if constexpr (DROP == 0) {
#pragma unroll
    for (int i = 0; i < WPG; ++i) F[i] = kOnes;
    return (1u << M) - 1u;
  } else {
    const uint32_t S = drop_threshold<M, DROP>(A);
#pragma unroll
    for (int i = 0; i < WPG; ++i) F[i] = pmin(psubsat(A[i], S), ones);    // mag > S
    uint32_t keep = gather_bits<M>(F);
    if (__builtin_popcount(keep) != N) {
      // magnitudes equal to S straddle the cut: keep them, then drop the
      // highest-indexed ones until n remain (ties go to the lower index)
      uint32_t E[WPG];
#pragma unroll
      for (int i = 0; i < WPG; ++i) E[i] = (F[i] | pmin(psubsat(S, A[i]), ones)) ^ kOnes;
      uint32_t eq = gather_bits<M>(E);
      keep |= eq;
#pragma unroll
      for (int t = 0; t < DROP; ++t) {
        if (__builtin_popcount(keep) > N) {
          const uint32_t top = 1u << (31 - __builtin_clz(eq));
          keep &= ~top;
          eq &= ~top;
        }
      }
      scatter_bits<M>(keep, F);
    }
    return keep;
  }
}

// Keep bits of one group of M from its M/2 words of magnitudes (sign bits
// cleared) for any n, by the rank rule: key_j = mag_j << log2(M) | (M-1-j) is
// unique in the group and orders by magnitude, then lower index; the n largest
// keys are kept.  (About M*M compares: for the patterns and variants the
// packed networks above do not cover.)
template <int M>
__device__ __forceinline__ uint32_t keep_by_rank(const uint32_t* A, int n) {
  constexpr int SH = M == 8 ? 3 : 2;
  int key[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const uint32_t h = (j & 1) ? (A[j >> 1] >> 16) : (A[j >> 1] & 0xFFFFu);
    key[j] = (int)((h << SH) | (uint32_t)(M - 1 - j));
  }
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    int above = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) above += key[i] > key[j];
    keep |= (above < n ? 1u : 0u) << j;
  }
  return keep;
}

}  // namespace sel
}  // namespace sbl
