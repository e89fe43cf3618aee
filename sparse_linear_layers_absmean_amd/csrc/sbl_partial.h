// Partial sums of the exact absmean scale, shared by the streaming absmean
// pass and the resident weight-preparation kernel.
//
// A BF16 magnitude is an integer number of 2^-133 units, so the sum is exact
// and independent of the reduction order and of the launch shape:
//  * Fast path: values in [2^-31, 2) are multiples of 2^-38; a thread adds at
//    most 2^14 of them in fp64, whose partial sums stay below 2^15 and so are
//    exact; the per-thread total is an integer below 2^53 in 2^-38 units.
//  * Every other nonzero value (tiny, subnormal or >= 2) is rare in weights;
//    it adds its significand to a per-exponent 64-bit bin in LDS.  A
//    workgroup that used the bins turns them into one exact multi-word
//    integer, stores it beside its slot and flags the slot (bit 63).
// Workspace layout: sbl_internal.h.
#pragma once

#include "sbl_beta.h"

namespace sbl {
namespace part {

__device__ __forceinline__ void rare_add(unsigned long long* bins, uint32_t mag15, uint32_t& rare) {
  const uint32_t e = mag15 >> 7;
  const uint32_t sig = (mag15 & 0x7Fu) | (e ? 0x80u : 0u);
  atomicAdd(&bins[e], (unsigned long long)sig);
  rare = 1u;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_sub(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
}

// Adds the 8 BF16 magnitudes of one 16-byte vector.  One packed test per
// vector: every magnitude in the fast window [2^-31, 2) (bits 0x3000..0x3FFF)
// -> two fp64 sums; otherwise (zeros included) value by value, values
// outside the window to the per-exponent bins.
__device__ __forceinline__ void consume(const u32x4& v, double& acc0, double& acc1, unsigned long long* bins,
                                        uint32_t& rare) {
  uint32_t a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = v[j] & 0x7FFF7FFFu;
  const uint32_t t = pk_max(pk_max(pk_sub(a[0], 0x30003000u), pk_sub(a[1], 0x30003000u)),
                            pk_max(pk_sub(a[2], 0x30003000u), pk_sub(a[3], 0x30003000u)));
  if ((t & 0xF000F000u) == 0u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc0 += (double)__uint_as_float(a[j] << 16);
      acc1 += (double)__uint_as_float(a[j] & 0xFFFF0000u);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = a[j] & 0xFFFFu, hi = a[j] >> 16;
    if ((lo - 0x3000u) < 0x1000u) acc0 += (double)__uint_as_float(lo << 16);
    else if (lo) rare_add(bins, lo, rare);
    if ((hi - 0x3000u) < 0x1000u) acc1 += (double)__uint_as_float(hi << 16);
    else if (hi) rare_add(bins, hi, rare);
  }
}

// The same for the mask-then-quant variant: only the halves whose bit is set
// in `keep` (bit 2j: low half of word j, bit 2j+1: high half) are added.  The
// fast-window test still looks at every value (a dropped value outside the
// window only sends the vector to the per-value path).
__device__ __forceinline__ void consume_kept(const u32x4& v, uint32_t keep, double& acc0, double& acc1,
                                             unsigned long long* bins, uint32_t& rare) {
  uint32_t a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = v[j] & 0x7FFF7FFFu;
  const uint32_t t = pk_max(pk_max(pk_sub(a[0], 0x30003000u), pk_sub(a[1], 0x30003000u)),
                            pk_max(pk_sub(a[2], 0x30003000u), pk_sub(a[3], 0x30003000u)));
  if ((t & 0xF000F000u) == 0u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t mlo = ((keep >> (2 * j)) & 1u) ? 0xFFFFu : 0u;
      const uint32_t mhi = ((keep >> (2 * j + 1)) & 1u) ? 0xFFFF0000u : 0u;
      acc0 += (double)__uint_as_float((a[j] & mlo) << 16);
      acc1 += (double)__uint_as_float(a[j] & mhi);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = ((keep >> (2 * j)) & 1u) ? (a[j] & 0xFFFFu) : 0u;
    const uint32_t hi = ((keep >> (2 * j + 1)) & 1u) ? (a[j] >> 16) : 0u;
    if ((lo - 0x3000u) < 0x1000u) acc0 += (double)__uint_as_float(lo << 16);
    else if (lo) rare_add(bins, lo, rare);
    if ((hi - 0x3000u) < 0x1000u) acc1 += (double)__uint_as_float(hi << 16);
    else if (hi) rare_add(bins, hi, rare);
  }
}

// Workgroup reduction of the per-thread sums and the stores of slot `slot`
// of a matrix with nb slots: the fast-window total (bit 63 set when some
// thread met out-of-window values) and, for a flagged slot, the exact record
// of the bins.  Thread 0 does every store (AGENT: as agent-scope atomics,
// beta::ws_store).  All kAbsThreads threads call it; the bins are read after
// the barrier inside.
template <bool AGENT = false>
__device__ inline void publish_partial(uint64_t* ws, int64_t nb, int64_t slot, double acc0, double acc1,
                                       uint32_t rare, unsigned long long* bins) {
  // both partial sums are exact multiples of 2^-38 below 2^15
  unsigned long long units =
      (unsigned long long)(acc0 * 0x1p38) + (unsigned long long)(acc1 * 0x1p38);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) units += __shfl_xor(units, off, 64);
  const bool wave_rare = __ballot(rare != 0) != 0;
  __shared__ unsigned long long wave_sum[kAbsThreads / 64];
  __shared__ uint32_t wave_rare_s[kAbsThreads / 64];
  if ((threadIdx.x & 63) == 0) {
    wave_sum[threadIdx.x >> 6] = units;
    wave_rare_s[threadIdx.x >> 6] = wave_rare ? 1u : 0u;
  }
  __syncthreads();
  uint32_t flagged = 0;
#pragma unroll
  for (int i = 0; i < kAbsThreads / 64; ++i) flagged |= wave_rare_s[i];
  if (flagged) {                                     // uniform: the bins become one exact integer
    __shared__ unsigned long long nz_bins[kAbsThreads / 64];
    __shared__ uint32_t limbs[beta::kLimbs + 2];
    const unsigned long long nz = __ballot(bins[threadIdx.x] != 0);
    if ((threadIdx.x & 63) == 0) nz_bins[threadIdx.x >> 6] = nz;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int i = 0; i < beta::kLimbs + 2; ++i) limbs[i] = 0;
      for (int wv = 0; wv < kAbsThreads / 64; ++wv) {
        unsigned long long msk = nz_bins[wv];
        while (msk) {
          const int e = wv * 64 + __ffsll(msk) - 1;
          msk &= msk - 1;
          beta::add_shifted(limbs, bins[e], max(e, 1) - 1);   // significand * 2^(max(e,1)-134)
        }
      }
      uint64_t* rec = ws + ws_limb_base(nb) + kWsLimbWords * slot;
      for (int j = 0; j < kWsLimbWords; ++j)
        beta::ws_store<AGENT>(rec + j, (uint64_t)limbs[2 * j] | ((uint64_t)limbs[2 * j + 1] << 32));
    }
  }
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
#pragma unroll
    for (int i = 0; i < kAbsThreads / 64; ++i) t += wave_sum[i];   // < 2^62
    beta::ws_store<AGENT>(ws + slot, t | (flagged ? beta::kRareFlag : 0ull));
  }
}

}  // namespace part
}  // namespace sbl
