// Exact absmean scale of a BF16 weight matrix: the streaming pass.
//
// beta = RN_fp32(mean |w|) over every value of the matrix: the ternary
// quantizer's scale comes from the mean absolute value of the weights
// (Sparse-BitNet method, "Ternary Quantization"; BitNet "Especificaciones
// Tecnicas": absmean quantization), taken before the N:M mask ("Quant-Then-
// Mask Order"), so pruned weights count too.
//
// The sum is exact, hence independent of the reduction order and of the
// launch shape (sbl_partial.h).  Each workgroup stores its total in a slot of
// its own (no atomics on global memory: on this chip same-address device
// atomics serialize at about 12 ns each); the division and the single
// rounding happen where beta is needed, at the start of the mask/pack kernels
// (sbl_beta.h); a one-workgroup-per-matrix kernel does it when beta is the
// only output.  Batches small enough to stay on the chip skip this pass
// altogether (the resident kernel in k_maskpack.hip).
// Several matrices share each launch (QBatch).
#include "sbl_partial.h"
#include "sbl_select.h"

namespace sbl {

namespace {

using namespace part;

__device__ __forceinline__ int find_item(const QBatch& b) {
  int di = 0;
  for (int i = 1; i < b.count; ++i)
    if ((int64_t)blockIdx.x >= b.start[i]) di = i;
  return di;
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
  part::publish_partial(ws, d.nb, wg, acc0, acc1, rare, bins);
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
