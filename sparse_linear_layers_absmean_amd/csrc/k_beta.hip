// Exact absmean scale of a BF16 weight matrix.
//
// beta = RN_fp32(mean |w|) over every value of the matrix: the ternary
// quantizer's scale comes from the mean absolute value of the weights
// (Sparse-BitNet method, "Ternary Quantization"; BitNet "Especificaciones
// Tecnicas": absmean quantization), taken before the N:M mask ("Quant-Then-
// Mask Order"), so pruned weights count too.
//
// The sum is exact, hence independent of the reduction order and of the
// launch shape: a BF16 magnitude is an integer number of 2^-133 units.
//  * Fast path: values in [2^-31, 2) are multiples of 2^-38; each thread adds
//    at most 2^14 of them in fp64, whose partial sums stay below 2^15 and so
//    are exact; the per-thread total is an integer below 2^53 in 2^-38 units.
//    Workgroup totals go to a 128-bit accumulator (64-bit atomic + carry count).
//  * Every other nonzero value (tiny, subnormal or >= 2) is rare in weights;
//    it adds its significand to a per-exponent 64-bit bin with an atomic.
//  * The last workgroup to finish rebuilds the exact sum as a multi-word
//    integer, divides it by n_out*k with a bit-serial long division and
//    rounds once to fp32 (nearest, ties to even), subnormals included.
//    It then zero-fills the accumulators, so the workspace is ready for the
//    next call (it must be zero-filled once before its first use).
#include "sbl_internal.h"

namespace sbl {

namespace {

constexpr int kBetaThreads = 256;
constexpr int64_t kMaxIterPerThread = 2048;   // 8 values each: <= 2^14 values per thread

__device__ __forceinline__ void rare_add(uint64_t* ws, uint32_t mag15) {
  const uint32_t e = mag15 >> 7;
  const uint32_t sig = (mag15 & 0x7Fu) | (e ? 0x80u : 0u);
  atomicAdd(reinterpret_cast<unsigned long long*>(&ws[kWsBins + e]), (unsigned long long)sig);
}

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// limbs: little-endian 32-bit words of a nonnegative integer (units of 2^-133)
constexpr int kLimbs = 12;

__device__ void add_shifted(uint32_t* L, uint64_t v, int s) {
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

// exact RN_fp32(S * 2^-133 / n) for the integer S held in limbs (shared memory)
__device__ float round_quotient(const uint32_t* L, uint64_t n) {
  int top = -1;
  for (int i = kLimbs - 1; i >= 0 && top < 0; --i)
    if (L[i]) top = i * 32 + 31 - __clz(L[i]);
  if (top < 0) return 0.0f;
  // 64-bit window of S whose bit 63 is S's bit `top`; bits of S below the
  // window only matter as a sticky flag.  The division below consumes at most
  // log2(n) + 26 <= 61 bits (n <= 2^34), so the window always suffices.
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
  uint64_t rem = 0, q = 0;
  bool found = false;
  int lsb = 0;
  for (int pos = top; pos >= -17; --pos) {
    rem = (rem << 1) | (win >> 63);
    win <<= 1;
    const uint32_t qb = rem >= n;
    if (qb) rem -= n;
    if (!found) {
      if (qb) {
        found = true;
        q = 1;
        lsb = max(pos - 23, -16);                   // 2^-149 is position -16 in 2^-133 units
      }
    } else {
      q = (q << 1) | qb;
    }
    if (found && pos == lsb - 1) break;             // guard bit collected
  }
  if (!found) return 0.0f;                          // below 2^-150: rounds to zero
  const bool sticky = rem != 0 || win != 0 || below;
  const uint64_t guard = q & 1u;
  uint64_t mant = q >> 1;
  if (guard && (sticky || (mant & 1u))) ++mant;
  return ldexpf((float)mant, lsb - 133);
}

__global__ __launch_bounds__(kBetaThreads) void beta_kernel(const u32x4* __restrict__ w, int64_t nvec,
                                                           uint64_t* __restrict__ ws,
                                                           float* __restrict__ beta_out,
                                                           uint64_t n_total) {
  double acc0 = 0.0, acc1 = 0.0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = ld_stream16(&w[i]);
    const uint32_t d[4] = {v[0], v[1], v[2], v[3]};
    bool rare = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (d[j] << 16) & 0x7FFFFFFFu;   // |w| of the low value as fp32 bits
      const uint32_t hi = d[j] & 0x7FFF0000u;           // |w| of the high value
      const bool in_lo = (lo - 0x30000000u) < 0x10000000u;   // [2^-31, 2)
      const bool in_hi = (hi - 0x30000000u) < 0x10000000u;
      acc0 += in_lo ? (double)__uint_as_float(lo) : 0.0;
      acc1 += in_hi ? (double)__uint_as_float(hi) : 0.0;
      rare |= (!in_lo && lo != 0u) || (!in_hi && hi != 0u);
    }
    if (rare) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = d[j] & 0x7FFFu, hi = (d[j] >> 16) & 0x7FFFu;
        if (lo && ((lo - 0x3000u) >= 0x1000u)) rare_add(ws, lo);
        if (hi && ((hi - 0x3000u) >= 0x1000u)) rare_add(ws, hi);
      }
    }
  }
  // both partial sums are exact multiples of 2^-38 below 2^15
  unsigned long long units =
      (unsigned long long)(acc0 * 0x1p38) + (unsigned long long)(acc1 * 0x1p38);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) units += __shfl_xor(units, off, 64);
  __shared__ unsigned long long wave_sum[kBetaThreads / 64];
  __shared__ unsigned long long nz_bins[kBetaThreads / 64];
  __shared__ uint64_t bins[256];
  __shared__ bool is_last;
  __shared__ uint32_t limbs[kLimbs];
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = units;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
    for (int i = 0; i < kBetaThreads / 64; ++i) s += wave_sum[i];
    unsigned long long* lo = reinterpret_cast<unsigned long long*>(&ws[kWsFastLo]);
    const unsigned long long old = atomicAdd(lo, s);
    if (old + s < old) atomicAdd(reinterpret_cast<unsigned long long*>(&ws[kWsFastHi]), 1ull);
    __threadfence();
    const unsigned long long ticket =
        atomicAdd(reinterpret_cast<unsigned long long*>(&ws[kWsCount]), 1ull);
    is_last = ticket == (unsigned long long)gridDim.x - 1;
  }
  __syncthreads();
  if (!is_last) return;
  // Last workgroup: every other one has finished its atomics.  Read the
  // per-exponent bins in parallel, then leave the workspace zero-filled for
  // the next call.
  __threadfence();
  const uint64_t b = ld_agent(&ws[kWsBins + threadIdx.x]);
  bins[threadIdx.x] = b;
  ws[kWsBins + threadIdx.x] = 0;
  const unsigned long long nz = __ballot(b != 0);
  if ((threadIdx.x & 63) == 0) nz_bins[threadIdx.x >> 6] = nz;
  __syncthreads();
  if (threadIdx.x != 0) return;
  const uint64_t fast_lo = ld_agent(&ws[kWsFastLo]);
  const uint64_t fast_hi = ld_agent(&ws[kWsFastHi]);
  ws[kWsFastLo] = 0;
  ws[kWsFastHi] = 0;
  ws[kWsCount] = 0;
  for (int i = 0; i < kLimbs; ++i) limbs[i] = 0;
  for (int wv = 0; wv < kBetaThreads / 64; ++wv) {
    unsigned long long m = nz_bins[wv];
    while (m) {
      const int e = wv * 64 + __ffsll(m) - 1;
      m &= m - 1;
      add_shifted(limbs, bins[e], max(e, 1) - 1);
    }
  }
  add_shifted(limbs, fast_lo, 95);        // 2^-38 = 2^95 * 2^-133
  add_shifted(limbs, fast_hi, 95 + 64);
  beta_out[0] = round_quotient(limbs, n_total);
}

__global__ void zero_ws_kernel(uint64_t* ws) {
  for (int i = threadIdx.x; i < kWsWords; i += blockDim.x) ws[i] = 0;
}

}  // namespace

hipError_t launch_workspace_init(uint64_t* ws, hipStream_t s) {
  hipLaunchKernelGGL(zero_ws_kernel, dim3(1), dim3(256), 0, s, ws);
  return hipGetLastError();
}

hipError_t launch_beta(const uint16_t* w, int64_t total, uint64_t* ws, float* beta,
                       hipStream_t s) {
  const int64_t nvec = total / 8;
  int64_t blocks = (nvec + kBetaThreads * 8 - 1) / (kBetaThreads * 8);
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  const int64_t min_blocks =
      (nvec + kBetaThreads * kMaxIterPerThread - 1) / (kBetaThreads * kMaxIterPerThread);
  if (blocks < min_blocks) blocks = min_blocks;
  hipLaunchKernelGGL(beta_kernel, dim3((unsigned)blocks), dim3(kBetaThreads), 0, s,
                     reinterpret_cast<const u32x4*>(w), nvec, ws, beta, (uint64_t)total);
  return hipGetLastError();
}

}  // namespace sbl
