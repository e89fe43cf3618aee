// Measured peaks of the chip, for the roofline figures: what a plain kernel
// reaches on a streaming HBM read and on back-to-back int8 MFMAs.  These are
// measurement aids, not part of the Sparse-BitLinear path (they live in their
// own library, libsbl_probe.so, which only the benchmark loads).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // 16-byte loads in flight per thread

// Grid-stride read of n16 16-byte vectors: each round, a thread issues
// kUnroll loads whose wave instructions each read 1 KB contiguous, then folds
// them into one word.  The sink is written only when the fold hits a value
// the buffer never produces (all-ones), so the loads cannot be dropped and
// nothing is written.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0xFFFFFFFFu) sink[0] = acc;
}

// Back-to-back independent v_mfma_i32_32x32x32_i8 (4 accumulators per wave),
// no memory traffic; one word per thread is stored at the end.
__global__ __launch_bounds__(kThreads) void mfma_i8_kernel(int32_t* __restrict__ sink, int iters) {
  v16i acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = v16i{};
  const v4i a = {(int32_t)threadIdx.x, 1, 2, 3}, b = {3, (int32_t)blockIdx.x, 1, 0};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at device pointer `buf` with
// `grid` workgroups of 256 threads; `sink` is one device word.  Returns a HIP
// error code (0 = launched).
int sbl_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

// `grid` workgroups of 256 threads, each wave issuing 4 * iters int8
// 32x32x32 MFMAs (65536 operations each); `sink` holds grid * 256 words.
int sbl_probe_mfma_i8(int32_t* sink, int grid, int iters, hipStream_t stream) {
  if (!sink || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_i8_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, sink, iters);
  return (int)hipGetLastError();
}

// The current device's peak engine clock (kHz), as the runtime reports it.
int sbl_probe_clock_khz(int* khz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeClockRate, dev);
  return (int)e;
}

}  // extern "C"
