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
//    Each workgroup stores its total in a slot of its own (no atomics: on this
//    chip same-address device atomics serialize at about 12 ns each).
//  * Every other nonzero value (tiny, subnormal or >= 2) is rare in weights;
//    it adds its significand to a per-exponent 64-bit bin with an atomic.
//  * A second, one-workgroup-per-matrix launch adds the slots and bins into a
//    multi-word integer, divides it by n_out*k with a bit-serial long division
//    and rounds once to fp32 (nearest, ties to even), subnormals included.
//    It then zero-fills the bins for the next call (they must be zero-filled
//    once before the first use); the slots are overwritten by every call.
// Several matrices share each launch (QBatch).
#include "sbl_internal.h"

namespace sbl {

namespace {

__device__ __forceinline__ void rare_add(uint64_t* ws, uint32_t mag15) {
  const uint32_t e = mag15 >> 7;
  const uint32_t sig = (mag15 & 0x7Fu) | (e ? 0x80u : 0u);
  atomicAdd(reinterpret_cast<unsigned long long*>(&ws[kWsBins + e]), (unsigned long long)sig);
}

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// RN_fp32(D / n) for a dividend D = W * 2^e + r, 0 <= r < 2^e, with bit 63 of
// W set, r != 0 exactly when `sticky`, and 64 <= n <= 2^34.  floor(D / (n*2^e))
// = floor(W / n) = Q (since R + r/2^e < n), and Q >= 2^29 holds more than the
// 24 bits + guard that rounding needs; whatever is below is only a sticky
// flag.  Nearest, ties to even, subnormal results included.
__device__ float round_div(uint64_t W, int e, bool sticky, uint64_t n) {
  const uint64_t Q = W / n, R = W - Q * n;
  sticky = sticky || R != 0;
  const int qb = 64 - __clzll((long long)Q);        // 30 <= qb <= 58
  int lsb = qb - 24;                                // fp32 unit inside Q for a normal result
  if (e + lsb < -149) lsb = -149 - e;               // subnormal: the unit is 2^-149
  if (lsb > qb) return 0.0f;                        // below half the smallest subnormal
  const uint64_t mant = Q >> lsb;
  const uint64_t guard = (Q >> (lsb - 1)) & 1u;
  sticky = sticky || (Q & ((1ull << (lsb - 1)) - 1u)) != 0;
  const uint64_t m = mant + ((guard && (sticky || (mant & 1u))) ? 1u : 0u);
  return ldexpf((float)m, e + lsb);
}

// exact RN_fp32(S * 2^-133 / n) for the integer S held in limbs (shared memory)
__device__ float round_quotient(const uint32_t* L, uint64_t n) {
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
__device__ float round_quotient_fast(uint64_t lo, uint64_t hi, uint64_t n) {
  const uint64_t vlo = lo + (hi << 32);
  const uint64_t vhi = (hi >> 32) + (vlo < lo ? 1u : 0u);
  if (vlo == 0 && vhi == 0) return 0.0f;
  const int top = vhi ? 127 - __clzll((long long)vhi) : 63 - __clzll((long long)vlo);
  if (top <= 63) return round_div(vlo << (63 - top), top - 63 - 38, false, n);
  const int s = top - 63;                           // 1 .. 63
  const uint64_t W = (vlo >> s) | (vhi << (64 - s));
  return round_div(W, s - 38, (vlo << (64 - s)) != 0, n);
}

__device__ __forceinline__ int find_item(const QBatch& b) {
  int di = 0;
  for (int i = 1; i < b.count; ++i)
    if ((int64_t)blockIdx.x >= b.start[i]) di = i;
  return di;
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
__device__ __forceinline__ void consume(const u32x4& v, double& acc0, double& acc1, uint64_t* ws) {
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
    else if (lo) rare_add(ws, lo);
    if ((hi - 0x3000u) < 0x1000u) acc1 += (double)__uint_as_float(hi << 16);
    else if (hi) rare_add(ws, hi);
  }
}

// Workgroup g of a matrix covers vectors [g*256*vpt, (g+1)*256*vpt) (vpt is a
// multiple of 8); thread t reads vectors t, t+256, ... of that range, so each
// load instruction of a wave reads 1 KB contiguous; eight loads in flight.
// Buffer loads past the matrix's end return zeros (which add nothing).
__global__ __launch_bounds__(kAbsThreads) void absmean_partial_kernel(const QBatch batch) {
  const int di = find_item(batch);
  const QDesc& d = batch.d[di];
  const int64_t wg = (int64_t)blockIdx.x - batch.start[di];
  const int vpt = (int)d.vpt;
  const int64_t first = wg * kAbsThreads * vpt;
  const int64_t span = d.nvec - first < (int64_t)kAbsThreads * vpt ? d.nvec - first
                                                                   : (int64_t)kAbsThreads * vpt;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.w + first, span * 16);
  uint64_t* ws = d.ws;
  double acc0 = 0.0, acc1 = 0.0;
  const int voff = threadIdx.x * 16;
  for (int j = 0; j < vpt; j += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rw, voff + (j + u) * kAbsThreads * 16, 0, 0));
#pragma unroll
    for (int u = 0; u < 8; ++u) consume(v[u], acc0, acc1, ws);
  }
  // both partial sums are exact multiples of 2^-38 below 2^15
  unsigned long long units =
      (unsigned long long)(acc0 * 0x1p38) + (unsigned long long)(acc1 * 0x1p38);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) units += __shfl_xor(units, off, 64);
  __shared__ unsigned long long wave_sum[kAbsThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = units;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
#pragma unroll
    for (int i = 0; i < kAbsThreads / 64; ++i) t += wave_sum[i];   // < 2^62
    ws[kWsSlots + wg] = t;
  }
}

// One workgroup per matrix, after the partial-sum launch has finished.
__global__ __launch_bounds__(kAbsThreads) void absmean_final_kernel(const QBatch batch) {
  const QDesc& d = batch.d[blockIdx.x];
  uint64_t* ws = d.ws;
  // slot sums split in 32-bit halves so that nothing overflows (nb <= 4096)
  unsigned long long s_lo = 0, s_hi = 0;
  for (int64_t i = threadIdx.x; i < d.nb; i += kAbsThreads) {
    const uint64_t v = ws[kWsSlots + i];
    s_lo += (uint32_t)v;
    s_hi += v >> 32;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    s_lo += __shfl_xor(s_lo, off, 64);
    s_hi += __shfl_xor(s_hi, off, 64);
  }
  __shared__ unsigned long long part[2][kAbsThreads / 64];
  __shared__ unsigned long long nz_bins[kAbsThreads / 64];
  __shared__ uint64_t bins[256];
  __shared__ uint32_t limbs[kLimbs];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[0][wave] = s_lo;
    part[1][wave] = s_hi;
  }
  const uint64_t b = ld_agent(&ws[kWsBins + threadIdx.x]);
  bins[threadIdx.x] = b;
  st_agent(&ws[kWsBins + threadIdx.x], 0);
  const unsigned long long nz = __ballot(b != 0);
  if ((threadIdx.x & 63) == 0) nz_bins[wave] = nz;
  __syncthreads();
  if (threadIdx.x != 0) return;
  unsigned long long lo = 0, hi = 0;
  for (int i = 0; i < kAbsThreads / 64; ++i) {
    lo += part[0][i];
    hi += part[1][i];
  }
  bool rare = false;
  for (int wv = 0; wv < kAbsThreads / 64; ++wv) rare = rare || nz_bins[wv] != 0;
  if (!rare) {
    d.beta[0] = round_quotient_fast(lo, hi, (uint64_t)d.nvec * 8u);
    return;
  }
  for (int i = 0; i < kLimbs; ++i) limbs[i] = 0;
  for (int wv = 0; wv < kAbsThreads / 64; ++wv) {
    unsigned long long msk = nz_bins[wv];
    while (msk) {
      const int e = wv * 64 + __ffsll(msk) - 1;
      msk &= msk - 1;
      add_shifted(limbs, bins[e], max(e, 1) - 1);
    }
  }
  add_shifted(limbs, lo, 95);        // 2^-38 = 2^95 * 2^-133
  add_shifted(limbs, hi, 95 + 32);
  d.beta[0] = round_quotient(limbs, (uint64_t)d.nvec * 8u);
}

__global__ void zero_ws_kernel(uint64_t* ws, int64_t words) {
  for (int64_t i = threadIdx.x; i < words; i += blockDim.x) ws[i] = 0;
}

}  // namespace

hipError_t launch_workspace_init(uint64_t* ws, int64_t words, hipStream_t s) {
  hipLaunchKernelGGL(zero_ws_kernel, dim3(1), dim3(256), 0, s, ws, words);
  return hipGetLastError();
}

hipError_t launch_absmean_partial(QBatch& b, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < b.count; ++i) {
    b.start[i] = blocks;
    blocks += b.d[i].nb;
  }
  b.start[b.count] = blocks;
  hipLaunchKernelGGL(absmean_partial_kernel, dim3((unsigned)blocks), dim3(kAbsThreads), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_absmean_final(QBatch& b, hipStream_t s) {
  hipLaunchKernelGGL(absmean_final_kernel, dim3((unsigned)b.count), dim3(kAbsThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace sbl
