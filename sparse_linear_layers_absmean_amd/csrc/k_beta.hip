// Exact absmean scale of a BF16 weight matrix: the streaming pass.
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
//    Each workgroup stores its total in a slot of its own (no atomics on
//    global memory: on this chip same-address device atomics serialize at
//    about 12 ns each).
//  * Every other nonzero value (tiny, subnormal or >= 2) is rare in weights;
//    it adds its significand to a per-exponent 64-bit bin in LDS.  A
//    workgroup that used the bins turns them into one exact multi-word
//    integer, stores it beside its slot and flags the slot (bit 63).
//  * The division and the single rounding happen where beta is needed, at the
//    start of the mask/pack kernels (sbl_beta.h); a one-workgroup-per-matrix
//    kernel does it when beta is the only output.
// Several matrices share each launch (QBatch).
#include "sbl_beta.h"
#include "sbl_select.h"

namespace sbl {

namespace {

__device__ __forceinline__ void rare_add(unsigned long long* bins, uint32_t mag15, uint32_t& rare) {
  const uint32_t e = mag15 >> 7;
  const uint32_t sig = (mag15 & 0x7Fu) | (e ? 0x80u : 0u);
  atomicAdd(&bins[e], (unsigned long long)sig);
  rare = 1u;
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

// Workgroup g of a matrix covers vectors [g*256*vpt, (g+1)*256*vpt) (vpt is a
// multiple of 8); thread t reads vectors t, t+256, ... of that range, so each
// load instruction of a wave reads 1 KB contiguous; 8 or 16 loads in flight.
// Buffer loads past the matrix's end return zeros (which add nothing).
// NT: nontemporal loads, for groups of matrices too large for the 256 MB
// Infinity Cache to hold until the mask/pack pass reads them again (13B
// block: 251 µs per call instead of 273 µs; 0.7B block: 39.4 instead of 38.4).
// KM > 0 (mask-then-quant): only the weights an n:KM mask keeps are summed
// (Sparse-BitNet summary, section 3 item 3, the ablated order); a 16-byte
// vector is one group of 8 or two groups of 4, selected by the rank rule.
template <bool NT, int KM>
__global__ __launch_bounds__(kAbsThreads) void absmean_partial_kernel(const QBatch batch, int n) {
  const int di = find_item(batch);
  const QDesc& d = batch.d[di];
  const int64_t wg = (int64_t)blockIdx.x - batch.start[di];
  const int vpt = (int)d.vpt;
  const int64_t first = wg * kAbsThreads * vpt;
  const int64_t span = d.nvec - first < (int64_t)kAbsThreads * vpt ? d.nvec - first
                                                                   : (int64_t)kAbsThreads * vpt;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(d.w + first, span * 16);
  uint64_t* ws = d.ws;
  __shared__ unsigned long long bins[256];          // per-exponent significand sums (rare values)
  bins[threadIdx.x] = 0;
  __syncthreads();
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t rare = 0;
  const int voff = threadIdx.x * 16;
  // batches of 8 vectors per thread, double-buffered: the next batch's loads
  // are issued before the current one is consumed
  auto load8 = [&](u32x4 (&v)[8], int j) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rw, voff + (j + u) * kAbsThreads * 16, 0, NT ? 2 : 0));
  };
  auto process8 = [&](const u32x4 (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (KM == 0) {
        consume(v[u], acc0, acc1, bins, rare);
      } else {
        uint32_t A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) A[j] = v[u][j] & 0x7FFF7FFFu;
        const uint32_t keep = KM == 8 ? sel::keep_by_rank<8>(A, n)
                                      : sel::keep_by_rank<4>(A, n) | (sel::keep_by_rank<4>(A + 2, n) << 4);
        consume_kept(v[u], keep, acc0, acc1, bins, rare);
      }
    }
  };
  u32x4 va[8], vb[8];
  load8(va, 0);
  for (int j = 0; j < vpt; j += 16) {
    if (j + 8 < vpt) load8(vb, j + 8);
    process8(va);
    if (j + 8 < vpt) {
      if (j + 16 < vpt) load8(va, j + 16);
      process8(vb);
    }
  }
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
      uint64_t* rec = ws + ws_limb_base(d.nb) + kWsLimbWords * wg;
      for (int j = 0; j < kWsLimbWords; ++j) rec[j] = (uint64_t)limbs[2 * j] | ((uint64_t)limbs[2 * j + 1] << 32);
    }
  }
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
#pragma unroll
    for (int i = 0; i < kAbsThreads / 64; ++i) t += wave_sum[i];   // < 2^62
    ws[wg] = t | (flagged ? beta::kRareFlag : 0ull);
  }
}

// beta alone (no mask, codes or packed output requested): one workgroup per matrix.
__global__ __launch_bounds__(kAbsThreads) void absmean_final_kernel(const QBatch batch) {
  (void)beta::workgroup_beta(batch.d[blockIdx.x], true);
}

__global__ void zero_ws_kernel(uint64_t* ws, int64_t words) {
  for (int64_t i = threadIdx.x; i < words; i += blockDim.x) ws[i] = 0;
}

constexpr int64_t kAbsStreamBytes = int64_t(128) << 20;   // masters per launch above which loads are nontemporal

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
  int64_t bytes = 0;
  for (int i = 0; i < b.count; ++i) bytes += b.d[i].nvec * 16;
  if (bytes > kAbsStreamBytes)
    hipLaunchKernelGGL((absmean_partial_kernel<true, 0>), dim3((unsigned)blocks), dim3(kAbsThreads), 0, s, b, 0);
  else
    hipLaunchKernelGGL((absmean_partial_kernel<false, 0>), dim3((unsigned)blocks), dim3(kAbsThreads), 0, s, b, 0);
  return hipGetLastError();
}

hipError_t launch_absmean_partial_kept(QBatch& b, int n, int m, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < b.count; ++i) {
    b.start[i] = blocks;
    blocks += b.d[i].nb;
  }
  b.start[b.count] = blocks;
  if (m == 8)
    hipLaunchKernelGGL((absmean_partial_kernel<false, 8>), dim3((unsigned)blocks), dim3(kAbsThreads), 0, s, b, n);
  else
    hipLaunchKernelGGL((absmean_partial_kernel<false, 4>), dim3((unsigned)blocks), dim3(kAbsThreads), 0, s, b, n);
  return hipGetLastError();
}

hipError_t launch_absmean_final(QBatch& b, hipStream_t s) {
  hipLaunchKernelGGL(absmean_final_kernel, dim3((unsigned)b.count), dim3(kAbsThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace sbl
