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
// One thread handles one 64-weight chunk (128 bytes of BF16): groups never
// cross chunks (m divides 64) and chunks never cross rows (64 divides k), so
// the matrix is processed as a flat array.  Per chunk it writes 16 bytes of
// DENSE2, 8 bytes of bitmap, 64*n/m/4 bytes of N:M codes and 64 code bytes.
// DENSE2 word layout: see d2_shift.
#include "sbl_internal.h"

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

__device__ __forceinline__ void store_outputs(const ChunkOut& o, int64_t c, int n, int m,
                                              uint8_t* mask, int8_t* codes, int fmt,
                                              uint8_t* packed, uint8_t* meta) {
  if (mask) reinterpret_cast<uint2*>(mask)[c] = make_uint2((uint32_t)o.keep, (uint32_t)(o.keep >> 32));
  if (codes) {
    uint4* cp = reinterpret_cast<uint4*>(codes) + c * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) cp[i] = make_uint4(o.cb[4 * i], o.cb[4 * i + 1], o.cb[4 * i + 2], o.cb[4 * i + 3]);
  }
  if (!packed) return;
  if (fmt == 0) {
    reinterpret_cast<uint4*>(packed)[c] = make_uint4(o.d2[0], o.d2[1], o.d2[2], o.d2[3]);
    return;
  }
  if (meta) reinterpret_cast<uint2*>(meta)[c] = make_uint2((uint32_t)o.keep, (uint32_t)(o.keep >> 32));
  const int bytes = 16 * n / m;             // even; a multiple of 4 unless m == 8 and n is odd
  const uint32_t w[4] = {(uint32_t)o.nm_lo, (uint32_t)(o.nm_lo >> 32), (uint32_t)o.nm_hi,
                         (uint32_t)(o.nm_hi >> 32)};
  if ((bytes & 3) == 0) {
    uint32_t* p = reinterpret_cast<uint32_t*>(packed + c * bytes);
    for (int i = 0; i < bytes / 4; ++i) p[i] = w[i];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(packed + c * bytes);
    for (int i = 0; i < bytes / 2; ++i) p[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
  }
}

template <int M, int NT>   // NT > 0: compile-time n; NT == 0: runtime n
__global__ __launch_bounds__(kThreads) void mask_pack_kernel(const uint4* __restrict__ w, int64_t nchunks,
                                                             int n_rt, const float* __restrict__ beta,
                                                             uint8_t* __restrict__ mask,
                                                             int8_t* __restrict__ codes, int fmt,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ meta) {
  constexpr int SH = (M == 8) ? 3 : 2;
  const int n = NT > 0 ? NT : n_rt;
  const float b = fmaxf(beta[0], 1e-5f);
  const int thr_mag = (int)(__float_as_uint(b * 0.5f) >> 16);
  const int thr_nz = (thr_mag << SH) | (M - 1);      // key > thr_nz  <=>  |w| > beta_eff/2
  const bool want_nm = packed && fmt == 1;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    uint32_t dw[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = ld_stream16(&w[c * 8 + i]);
      dw[4 * i] = v[0]; dw[4 * i + 1] = v[1]; dw[4 * i + 2] = v[2]; dw[4 * i + 3] = v[3];
    }
    ChunkOut o = {};
#pragma unroll
    for (int g = 0; g < 64 / M; ++g) {
      int key[M];
      uint32_t sgn[M];
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int idx = g * M + j;
        const uint32_t h = (idx & 1) ? (dw[idx >> 1] >> 16) : (dw[idx >> 1] & 0xFFFFu);
        key[j] = (int)(((h & 0x7FFFu) << SH) | (uint32_t)(M - 1 - j));
        sgn[j] = h >> 15;
      }
      const int thr = group_threshold<M>(key, n);
      int kept = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int idx = g * M + j;
        const bool keep = key[j] > thr;
        const bool nz = keep && key[j] > thr_nz;
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
    store_outputs(o, c, n, M, mask, codes, fmt, packed, meta);
  }
}

// Packing of caller-supplied codes (+ mask for N:M).
template <int M>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint4* __restrict__ codes, const uint2* __restrict__ maskv,
                                                        int64_t nchunks, int n, int fmt,
                                                        uint8_t* __restrict__ packed,
                                                        uint8_t* __restrict__ meta) {
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
    store_outputs(o, c, n, M, nullptr, nullptr, fmt, packed, meta);
  }
}

int64_t grid_for(int64_t nchunks) {
  int64_t blocks = (nchunks + kThreads - 1) / kThreads;
  return blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks);
}

}  // namespace

hipError_t launch_mask_pack(const uint16_t* w, int64_t total, int n, int m, const float* beta,
                            uint8_t* mask, int8_t* codes, int fmt, uint8_t* packed,
                            uint8_t* meta, hipStream_t s) {
  const int64_t nchunks = total / kChunk;
  const dim3 grid((unsigned)grid_for(nchunks)), block(kThreads);
  const uint4* wv = reinterpret_cast<const uint4*>(w);
  if (m == 8 && n == 6)
    hipLaunchKernelGGL((mask_pack_kernel<8, 6>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  else if (m == 8 && n == 8)
    hipLaunchKernelGGL((mask_pack_kernel<8, 8>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  else if (m == 4 && n == 2)
    hipLaunchKernelGGL((mask_pack_kernel<4, 2>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  else if (m == 4 && n == 4)
    hipLaunchKernelGGL((mask_pack_kernel<4, 4>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  else if (m == 8)
    hipLaunchKernelGGL((mask_pack_kernel<8, 0>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  else
    hipLaunchKernelGGL((mask_pack_kernel<4, 0>), grid, block, 0, s, wv, nchunks, n, beta, mask, codes, fmt, packed, meta);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* codes, const uint8_t* mask, int64_t total, int n, int m,
                       int fmt, uint8_t* packed, uint8_t* meta, hipStream_t s) {
  const int64_t nchunks = total / kChunk;
  const dim3 grid((unsigned)grid_for(nchunks)), block(kThreads);
  const uint4* cv = reinterpret_cast<const uint4*>(codes);
  const uint2* mv = reinterpret_cast<const uint2*>(mask);
  if (m == 8)
    hipLaunchKernelGGL((pack_kernel<8>), grid, block, 0, s, cv, mv, nchunks, n, fmt, packed, meta);
  else
    hipLaunchKernelGGL((pack_kernel<4>), grid, block, 0, s, cv, mv, nchunks, n, fmt, packed, meta);
  return hipGetLastError();
}

}  // namespace sbl
