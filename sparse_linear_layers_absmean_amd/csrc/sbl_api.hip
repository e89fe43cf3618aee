// C ABI of libsbl: host-side validation and kernel dispatch.  See include/sbl.h.
#include <mutex>

#include "sbl.h"
#include "sbl_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxK = 131072;            // 127*k < 2^24: fp32(acc) exact
constexpr int64_t kMaxElems = int64_t(1) << 34;
constexpr int64_t kMaxTokens = int64_t(1) << 24;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool nm_ok(int32_t n, int32_t m) { return (m == 4 || m == 8) && n >= 1 && n <= m; }

bool k_ok(int64_t k) { return k >= 64 && k <= kMaxK && k % 64 == 0; }

int launch_status(hipError_t e) {
  if (e == hipSuccess) return SBL_OK;
  g_last_hip_error = (int)e;
  return SBL_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int sbl_abi_version(void) { return SBL_ABI_VERSION; }

const char* sbl_status_string(int status) {
  switch (status) {
    case SBL_OK: return "ok";
    case SBL_ERR_NULL: return "required pointer is NULL";
    case SBL_ERR_SHAPE: return "size out of range or inconsistent";
    case SBL_ERR_ALIGN: return "pointer misaligned";
    case SBL_ERR_UNSUPPORTED: return "unsupported n:m pattern or format";
    case SBL_ERR_LAUNCH: return "HIP launch failed";
    case SBL_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int sbl_last_hip_error(void) { return g_last_hip_error; }

int64_t sbl_packed_bytes(int64_t n_out, int64_t k, int32_t n, int32_t m, int32_t fmt) {
  if (n_out < 1 || !k_ok(k) || n_out * k > kMaxElems) return -1;
  if (fmt == SBL_FMT_DENSE2) return n_out * (k / 4);
  if (fmt == SBL_FMT_NM && nm_ok(n, m)) return n_out * (k / m) * n / 4;
  return -1;
}

int64_t sbl_meta_bytes(int64_t n_out, int64_t k, int32_t fmt) {
  if (n_out < 1 || !k_ok(k) || n_out * k > kMaxElems) return -1;
  if (fmt == SBL_FMT_DENSE2) return 0;
  if (fmt == SBL_FMT_NM) return n_out * (k / 8);
  return -1;
}

int64_t sbl_workspace_bytes(int64_t n_out, int64_t k) {
  if (n_out < 1 || !k_ok(k) || n_out * k > kMaxElems) return -1;
  return sbl::workspace_bytes_for(n_out * k);
}

int sbl_workspace_init(void* workspace, int64_t workspace_bytes, sbl_stream stream) {
  if (!workspace) return SBL_ERR_NULL;
  if (workspace_bytes < 8 || workspace_bytes % 8 != 0) return SBL_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SBL_ERR_ALIGN;
  return launch_status(sbl::launch_workspace_init(reinterpret_cast<uint64_t*>(workspace),
                                                  workspace_bytes / 8,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a && b && a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// own_ws: the item brings its workspace (checked here); false when the call
// supplies the scratch itself (sbl_quant_weights_batch_noalloc).
int check_quant(const sbl_quant_item& it, int32_t n, int32_t m, int32_t fmt, bool own_ws = true) {
  if (!it.w_bf16 || !it.beta) return SBL_ERR_NULL;
  if (it.packed && fmt == SBL_FMT_NM && !it.meta) return SBL_ERR_NULL;
  if (it.n_out < 1 || !k_ok(it.k) || it.n_out * it.k > kMaxElems) return SBL_ERR_SHAPE;
  // outputs must not share bytes (e.g. the row-major mask and the
  // panel-major metadata hold the same bits in different orders)
  if (nm_ok(n, m) && (fmt == SBL_FMT_DENSE2 || fmt == SBL_FMT_NM)) {
    const int64_t mask_b = it.n_out * (it.k / 8);
    const int64_t packed_b = fmt == SBL_FMT_DENSE2 ? it.n_out * (it.k / 4) : it.n_out * (it.k / m) * n / 4;
    const void* meta = (it.packed && fmt == SBL_FMT_NM) ? it.meta : nullptr;
    const void* packed = it.packed;
    if (ranges_overlap(it.mask_bits, mask_b, meta, mask_b) || ranges_overlap(it.mask_bits, mask_b, packed, packed_b) ||
        ranges_overlap(it.codes, it.n_out * it.k, packed, packed_b) ||
        ranges_overlap(it.codes, it.n_out * it.k, it.mask_bits, mask_b) ||
        ranges_overlap(it.codes, it.n_out * it.k, meta, mask_b) || ranges_overlap(packed, packed_b, meta, mask_b))
      return SBL_ERR_SHAPE;
  }
  if (own_ws && (!it.workspace || it.workspace_bytes < sbl::workspace_bytes_for(it.n_out * it.k)))
    return SBL_ERR_WORKSPACE;
  if (!nm_ok(n, m)) return SBL_ERR_UNSUPPORTED;
  if (it.packed && fmt != SBL_FMT_DENSE2 && fmt != SBL_FMT_NM) return SBL_ERR_UNSUPPORTED;
  if (!aligned(it.w_bf16, 16) || !aligned(it.beta, 4) || (own_ws && !aligned(it.workspace, 16)) ||
      (it.mask_bits && !aligned(it.mask_bits, 16)) || (it.codes && !aligned(it.codes, 16)) ||
      (it.packed && !aligned(it.packed, 16)) || (it.meta && !aligned(it.meta, 16)))
    return SBL_ERR_ALIGN;
  return SBL_OK;
}

sbl::QDesc to_qdesc(const sbl_quant_item& it, int32_t fmt) {
  const int64_t total = it.n_out * it.k;
  const sbl::AbsmeanPlan p = sbl::absmean_plan(total);
  sbl::QDesc d;
  d.w = reinterpret_cast<const sbl::u32x4*>(it.w_bf16);
  d.nvec = total / 8;
  d.count = total;
  d.nb = p.nb;
  d.vpt = p.vpt;
  d.beta = it.beta;
  d.ws = reinterpret_cast<uint64_t*>(it.workspace);
  d.ws_words = it.workspace_bytes / 8;
  d.beta_rows = 0;
  d.beta_kblocks = 0;
  d.mask = it.mask_bits;
  d.codes = it.codes;
  d.packed = it.packed;
  d.fmt = it.packed ? fmt : SBL_FMT_DENSE2;
  d.meta = (it.packed && fmt == SBL_FMT_NM) ? it.meta : nullptr;
  d.n_out = it.n_out;
  d.nkb = (int32_t)(it.k / 64);
  return d;
}

// Per group of up to kMaxQDesc matrices: one launch when the group fits on
// the chip (launch_resident decides; the method's order, at most two dropped
// per group), else the absmean pass, then the mask/pack pass.  Up to about one round of mask/pack workgroups (three per
// CU on 256 CUs) each finalizes beta itself, saving a launch; beyond that the
// repeated finalization would sit on the critical path of every round, so the
// finalize kernel runs once in between.  A call that wants only beta runs
// just the finalize kernel.
constexpr int64_t kPrologueMaxWorkgroups = 1024;
constexpr int64_t kPrologueMaxSlots = 512;       // every wave loads all partial sums (beta::kWaveSlots)
// Bound of the one-launch kernel's wait for other workgroups' partial sums
// before it computes the missing ones itself, in microseconds of the chip's
// constant real-time counter.  On an idle chip every sum arrives within ~15 us
// of the launch; the bound only acts when other work delays workgroups.
constexpr uint32_t kResidentWaitUs = 100;

// real-time counter ticks per microsecond of the current device (queried once
// per device; 100 on MI355X)
uint32_t ticks_per_us() {
  static std::mutex mu;
  static int rate_khz[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100;
  std::lock_guard<std::mutex> lock(mu);
  if (rate_khz[dev] <= 0) {
    int r = 0;
    if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess || r <= 0) r = 100000;
    rate_khz[dev] = r;
  }
  const uint32_t t = (uint32_t)(rate_khz[dev] / 1000);
  return t > 0 ? t : 1;
}


int launch_quant(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m, int32_t fmt, int32_t flags,
                 hipStream_t s) {
  const bool kept = (flags & SBL_QW_BETA_KEPT) != 0, mfc = (flags & SBL_QW_MASK_FROM_CODES) != 0;
  const bool one_launch = (flags & (SBL_QW_BETA_KEPT | SBL_QW_MASK_FROM_CODES | SBL_QW_TWO_PASS)) == 0;
  const uint32_t wait_ticks = (flags & SBL_QW_NO_WAIT) ? 0u : kResidentWaitUs * ticks_per_us();
  for (int i0 = 0; i0 < count; i0 += sbl::kMaxQDesc) {
    sbl::QBatch b;
    b.count = count - i0 < sbl::kMaxQDesc ? count - i0 : sbl::kMaxQDesc;
    b.beta_ready = 0;
    bool outputs = false;
    for (int i = 0; i < b.count; ++i) {
      b.d[i] = to_qdesc(items[i0 + i], fmt);
      if (kept) b.d[i].count = b.d[i].count / m * n;   // k % m == 0: exact
      outputs = outputs || b.d[i].mask || b.d[i].codes || b.d[i].packed;
    }
    if (one_launch && outputs) {
      hipError_t err = hipSuccess;
      if (sbl::launch_resident(b, n, m, wait_ticks, s, &err)) {
        const int st = launch_status(err);
        if (st != SBL_OK) return st;
        continue;
      }
    }
    int64_t grid = 0;
    bool wide = false;                              // a matrix with more than 512 partial sums
    for (int i = 0; i < b.count; ++i) wide = wide || b.d[i].nb > kPrologueMaxSlots;
    (void)sbl::launch_mask_pack(b, n, m, s, true, &grid, mfc);
    b.beta_ready = !outputs || wide || grid > kPrologueMaxWorkgroups;
    int st = launch_status(kept ? sbl::launch_absmean_partial_kept(b, n, m, s) : sbl::launch_absmean_partial(b, s));
    if (st == SBL_OK && b.beta_ready) st = launch_status(sbl::launch_absmean_final(b, s));
    if (st == SBL_OK && outputs) st = launch_status(sbl::launch_mask_pack(b, n, m, s, false, nullptr, mfc));
    if (st != SBL_OK) return st;
  }
  return SBL_OK;
}

bool overlaps(const sbl_quant_item& a, const sbl_quant_item& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.workspace), b0 = reinterpret_cast<uintptr_t>(b.workspace);
  return a0 < b0 + (uintptr_t)b.workspace_bytes && b0 < a0 + (uintptr_t)a.workspace_bytes;
}

}  // namespace

extern "C" {

int sbl_quant_weights(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                      float* beta, uint8_t* mask_bits, int8_t* codes, int32_t fmt,
                      uint8_t* packed, uint8_t* meta, void* workspace, int64_t workspace_bytes,
                      sbl_stream stream) {
  const sbl_quant_item it = {w_bf16, n_out, k, beta, mask_bits, codes, packed, meta,
                             workspace, workspace_bytes};
  const int st = check_quant(it, n, m, fmt);
  if (st != SBL_OK) return st;
  return launch_quant(&it, 1, n, m, fmt, 0, reinterpret_cast<hipStream_t>(stream));
}

int sbl_quant_weights_batch(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                            int32_t fmt, sbl_stream stream) {
  return sbl_quant_weights_batch_ex(items, count, n, m, fmt, SBL_QW_DEFAULT, stream);
}

int sbl_quant_weights_batch_ex(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                               int32_t fmt, int32_t flags, sbl_stream stream) {
  if ((flags & ~(SBL_QW_BETA_KEPT | SBL_QW_MASK_FROM_CODES | SBL_QW_TWO_PASS | SBL_QW_NO_WAIT)) != 0 ||
      (flags & (SBL_QW_BETA_KEPT | SBL_QW_MASK_FROM_CODES)) == (SBL_QW_BETA_KEPT | SBL_QW_MASK_FROM_CODES))
    return SBL_ERR_UNSUPPORTED;
  if (!items) return SBL_ERR_NULL;
  if (count < 1 || count > 256) return SBL_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const int st = check_quant(items[i], n, m, fmt);
    if (st != SBL_OK) return st;
    for (int j = 0; j < i; ++j)
      if (overlaps(items[i], items[j])) return SBL_ERR_WORKSPACE;
  }
  return launch_quant(items, count, n, m, fmt, flags, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free weight preparation: the exact-beta scratch of every item
// comes from one fixed device array per GPU instead of caller workspaces.
// The array's name is a host-side stand-in; its device address on each GPU
// is looked up once (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[SBL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};         // device address of `scratch` per device

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SBL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launch_status(e);
    if (!p) return launch_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SBL_OK;
}

}  // namespace

extern "C" {

int sbl_quant_weights_batch_noalloc(const sbl_quant_item* items, int32_t count, int32_t n, int32_t m,
                                    int32_t fmt, sbl_stream stream) {
  if (!items) return SBL_ERR_NULL;
  if (count < 1 || count > 256) return SBL_ERR_SHAPE;
  sbl_quant_item local[256];
  int64_t offset[256];
  int64_t used = 0;
  for (int i = 0; i < count; ++i) {
    const int st = check_quant(items[i], n, m, fmt, false);
    if (st != SBL_OK) return st;
    local[i] = items[i];
    local[i].workspace_bytes = sbl::workspace_bytes_for(items[i].n_out * items[i].k);
    offset[i] = used;
    used += (local[i].workspace_bytes + 255) / 256 * 256;
    if (used > SBL_NOALLOC_SCRATCH_BYTES) return SBL_ERR_WORKSPACE;
  }
  void* base = nullptr;
  const int st = current_scratch(&base);
  if (st != SBL_OK) return st;
  for (int i = 0; i < count; ++i) local[i].workspace = static_cast<uint8_t*>(base) + offset[i];
  return launch_quant(local, count, n, m, fmt, 0, reinterpret_cast<hipStream_t>(stream));
}

int sbl_pack(const int8_t* codes, const uint8_t* mask_bits, int64_t n_out, int64_t k, int32_t n,
             int32_t m, int32_t fmt, uint8_t* packed, uint8_t* meta, sbl_stream stream) {
  if (!codes || !packed) return SBL_ERR_NULL;
  if (fmt == SBL_FMT_NM && !mask_bits) return SBL_ERR_NULL;
  if (n_out < 1 || !k_ok(k) || n_out * k > kMaxElems) return SBL_ERR_SHAPE;
  if (fmt != SBL_FMT_DENSE2 && fmt != SBL_FMT_NM) return SBL_ERR_UNSUPPORTED;
  if (!nm_ok(n, m)) return SBL_ERR_UNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(packed, 16) || (mask_bits && !aligned(mask_bits, 16)) ||
      (meta && !aligned(meta, 16)))
    return SBL_ERR_ALIGN;
  return launch_status(sbl::launch_pack(codes, mask_bits, n_out, k, n, m, fmt, packed,
                                        fmt == SBL_FMT_NM ? meta : nullptr,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int sbl_quant_acts(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                   sbl_stream stream) {
  if (m_tok < 0 || m_tok > kMaxTokens || !k_ok(k)) return SBL_ERR_SHAPE;
  if (m_tok == 0) return SBL_OK;
  if (!x || !xq || !gamma) return SBL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(gamma, 4)) return SBL_ERR_ALIGN;
  return launch_status(sbl::launch_quant_acts(x, m_tok, k, xq, gamma,
                                              reinterpret_cast<hipStream_t>(stream)));
}

namespace {

int check_linear(const sbl_linear_item& it, int32_t fmt, int32_t n, int32_t m) {
  if (it.m_tok < 0 || it.m_tok > kMaxTokens || it.n_out < 0 || !k_ok(it.k) ||
      it.n_out * it.k > kMaxElems)
    return SBL_ERR_SHAPE;
  if (fmt != SBL_FMT_DENSE2 && fmt != SBL_FMT_NM) return SBL_ERR_UNSUPPORTED;
  if (fmt == SBL_FMT_NM && !nm_ok(n, m)) return SBL_ERR_UNSUPPORTED;
  if (it.m_tok == 0 || it.n_out == 0) return SBL_OK;
  if (!it.packed || !it.beta || !it.xq || !it.gamma || !it.y) return SBL_ERR_NULL;
  if (fmt == SBL_FMT_NM && !it.meta) return SBL_ERR_NULL;
  if (!aligned(it.packed, 16) || !aligned(it.xq, 16) || !aligned(it.y, 4) ||
      !aligned(it.beta, 4) || !aligned(it.gamma, 4) || (it.acc && !aligned(it.acc, 4)) ||
      (it.meta && !aligned(it.meta, 16)))
    return SBL_ERR_ALIGN;
  return SBL_OK;
}

sbl::LinearArgs to_args(const sbl_linear_item& it, int32_t fmt) {
  sbl::LinearArgs a;
  a.packed = it.packed;
  a.meta = fmt == SBL_FMT_NM ? it.meta : nullptr;
  a.beta = it.beta;
  a.xq = it.xq;
  a.gamma = it.gamma;
  a.m_tok = it.m_tok;
  a.n_out = it.n_out;
  a.k = it.k;
  a.y = it.y;
  a.acc = it.acc;
  return a;
}

}  // namespace

int sbl_linear(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
               const float* beta, const int8_t* xq, const float* gamma, int64_t m_tok,
               int64_t n_out, int64_t k, float* y, int32_t* acc, sbl_stream stream) {
  const sbl_linear_item it = {packed, meta, beta, xq, gamma, m_tok, n_out, k, y, acc};
  const int st = check_linear(it, fmt, n, m);
  if (st != SBL_OK || m_tok == 0 || n_out == 0) return st;
  const sbl::LinearArgs a = to_args(it, fmt);
  return launch_status(sbl::launch_linear_batch(&a, 1, fmt, n, m, reinterpret_cast<hipStream_t>(stream)));
}

int sbl_linear_acts_batch(const float* x, int64_t m_tok, int64_t k, int8_t* xq, float* gamma,
                          const sbl_linear_item* items, int32_t count, int32_t fmt, int32_t n, int32_t m,
                          sbl_stream stream) {
  if (!items) return SBL_ERR_NULL;
  if (count < 1 || count > 256) return SBL_ERR_SHAPE;
  if (m_tok < 0 || m_tok > kMaxTokens || !k_ok(k)) return SBL_ERR_SHAPE;
  if (m_tok > 0 && (!x || !xq || !gamma)) return SBL_ERR_NULL;
  if (m_tok > 0 && (!aligned(x, 16) || !aligned(xq, 16) || !aligned(gamma, 4))) return SBL_ERR_ALIGN;
  sbl::LinearArgs args[256];
  for (int i = 0; i < count; ++i) {
    sbl_linear_item it = items[i];
    if (it.m_tok != m_tok || it.k != k) return SBL_ERR_SHAPE;
    it.xq = xq;
    it.gamma = gamma;
    const int st = check_linear(it, fmt, n, m);
    if (st != SBL_OK) return st;
    args[i] = to_args(it, fmt);
  }
  if (m_tok == 0) return SBL_OK;
  return launch_status(sbl::launch_linear_acts(x, m_tok, k, xq, gamma, args, count, fmt, n, m,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int sbl_linear_batch(const sbl_linear_item* items, int32_t count, int32_t fmt, int32_t n,
                     int32_t m, sbl_stream stream) {
  if (!items) return SBL_ERR_NULL;
  if (count < 1 || count > 256) return SBL_ERR_SHAPE;
  sbl::LinearArgs args[256];
  for (int i = 0; i < count; ++i) {
    const int st = check_linear(items[i], fmt, n, m);
    if (st != SBL_OK) return st;
    args[i] = to_args(items[i], fmt);
  }
  return launch_status(sbl::launch_linear_batch(args, count, fmt, n, m, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// group scales: rows_per_group rows x cols_per_group features per beta
int64_t workspace_bytes_groups(int64_t n_out, int64_t k, int64_t rpg, int64_t cpg) {
  if (n_out < 1 || !k_ok(k) || n_out * k > kMaxElems || rpg < 1 || cpg < 64 || cpg % 64 != 0 || k % cpg != 0)
    return -1;
  const sbl::GroupPlan p = sbl::group_plan(n_out, k, rpg, cpg);
  if (p.gr > 65535 || p.gk > 65535) return -1;       // grid rows and layers of the partial-sum launch
  return (8 * p.groups * p.region + 4095) / 4096 * 4096;
}

int quant_weights_groups(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m, int64_t rpg,
                         int64_t cpg, float* beta, uint8_t* mask_bits, int8_t* codes, int32_t fmt, uint8_t* packed,
                         uint8_t* meta, void* workspace, int64_t workspace_bytes, sbl_stream stream) {
  if (rpg < 1 || cpg < 64 || cpg % 64 != 0 || k % cpg != 0) return SBL_ERR_SHAPE;
  // the per-matrix checks (their workspace size aside), then the group workspace's size
  const sbl_quant_item it{w_bf16, n_out, k, beta, mask_bits, codes, packed, meta, workspace, INT64_MAX};
  int st = check_quant(it, n, m, fmt);
  if (st != SBL_OK) return st;
  const int64_t need = workspace_bytes_groups(n_out, k, rpg, cpg);
  if (need < 0) return SBL_ERR_SHAPE;                // more than 65535 row or column groups
  if (workspace_bytes < need) return SBL_ERR_WORKSPACE;
  const int64_t groups = (n_out + rpg - 1) / rpg * (k / cpg);
  const int64_t mask_b = n_out * (k / 8);
  const int64_t packed_b = fmt == SBL_FMT_DENSE2 ? n_out * (k / 4) : n_out * (k / m) * n / 4;
  if (ranges_overlap(beta, 4 * groups, mask_bits, mask_b) || ranges_overlap(beta, 4 * groups, codes, n_out * k) ||
      ranges_overlap(beta, 4 * groups, packed, packed_b) ||
      ranges_overlap(beta, 4 * groups, packed && fmt == SBL_FMT_NM ? meta : nullptr, mask_b) ||
      ranges_overlap(beta, 4 * groups, workspace, workspace_bytes))
    return SBL_ERR_SHAPE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = launch_status(sbl::launch_grouped_beta(w_bf16, n_out, k, rpg, cpg, beta,
                                              reinterpret_cast<uint64_t*>(workspace), s));
  if (st != SBL_OK || (!mask_bits && !codes && !packed)) return st;
  sbl::QBatch b;
  b.count = 1;
  b.beta_ready = 1;
  b.d[0] = to_qdesc(it, fmt);
  b.d[0].beta_rows = rpg;
  b.d[0].beta_kblocks = cpg == k ? 0 : (int32_t)(cpg / 64);
  return launch_status(sbl::launch_mask_pack(b, n, m, s));
}

int linear_kgroups(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m, const float* beta,
                   int64_t rpg, bool per_block, const int8_t* xq, const float* gamma, int64_t kg, int64_t m_tok,
                   int64_t n_out, int64_t k, float* y, sbl_stream stream) {
  if (rpg < 1 || kg < 64 || kg % 64 != 0 || k % kg != 0 || m_tok > 65535) return SBL_ERR_SHAPE;
  const sbl_linear_item it{packed, meta, beta, xq, gamma, m_tok, n_out, k, y, nullptr};
  const int st = check_linear(it, fmt, n, m);
  if (st != SBL_OK || m_tok == 0 || n_out == 0) return st;
  const int64_t betas = (n_out + rpg - 1) / rpg * (per_block ? k / kg : 1);
  if (ranges_overlap(y, m_tok * n_out * 4, gamma, m_tok * (k / kg) * 4) ||
      ranges_overlap(y, m_tok * n_out * 4, beta, 4 * betas))
    return SBL_ERR_SHAPE;
  return launch_status(sbl::launch_linear_kgrouped(packed, fmt == SBL_FMT_NM ? meta : nullptr, fmt, n, m, beta, rpg,
                                                   per_block, xq, gamma, kg, m_tok, n_out, k, y,
                                                   reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int64_t sbl_workspace_bytes_grouped(int64_t n_out, int64_t k, int64_t rows_per_group) {
  return workspace_bytes_groups(n_out, k, rows_per_group, k);
}

int sbl_quant_weights_grouped(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                              int64_t rows_per_group, float* beta, uint8_t* mask_bits, int8_t* codes, int32_t fmt,
                              uint8_t* packed, uint8_t* meta, void* workspace, int64_t workspace_bytes,
                              sbl_stream stream) {
  if (!k_ok(k)) return SBL_ERR_SHAPE;
  return quant_weights_groups(w_bf16, n_out, k, n, m, rows_per_group, k, beta, mask_bits, codes, fmt, packed, meta,
                              workspace, workspace_bytes, stream);
}

int64_t sbl_workspace_bytes_blocked(int64_t n_out, int64_t k, int64_t rows_per_group, int64_t cols_per_group) {
  return workspace_bytes_groups(n_out, k, rows_per_group, cols_per_group);
}

int sbl_quant_weights_blocked(const uint16_t* w_bf16, int64_t n_out, int64_t k, int32_t n, int32_t m,
                              int64_t rows_per_group, int64_t cols_per_group, float* beta, uint8_t* mask_bits,
                              int8_t* codes, int32_t fmt, uint8_t* packed, uint8_t* meta, void* workspace,
                              int64_t workspace_bytes, sbl_stream stream) {
  return quant_weights_groups(w_bf16, n_out, k, n, m, rows_per_group, cols_per_group, beta, mask_bits, codes, fmt,
                              packed, meta, workspace, workspace_bytes, stream);
}

int sbl_linear_grouped(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                       const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t m_tok,
                       int64_t n_out, int64_t k, float* y, int32_t* acc, sbl_stream stream) {
  if (rows_per_group < 1) return SBL_ERR_SHAPE;
  const sbl_linear_item it{packed, meta, beta, xq, gamma, m_tok, n_out, k, y, acc};
  const int st = check_linear(it, fmt, n, m);
  if (st != SBL_OK || m_tok == 0 || n_out == 0) return st;
  const int64_t groups = (n_out + rows_per_group - 1) / rows_per_group;
  if (ranges_overlap(y, m_tok * n_out * 4, beta, 4 * groups) ||
      (acc && (ranges_overlap(acc, m_tok * n_out * 4, beta, 4 * groups) ||
               ranges_overlap(y, m_tok * n_out * 4, acc, m_tok * n_out * 4))))
    return SBL_ERR_SHAPE;
  sbl::LinearArgs a = to_args(it, fmt);
  a.beta_rows = rows_per_group < n_out ? rows_per_group : 0;   // the products' epilogues read beta per row
  return launch_status(sbl::launch_linear_batch(&a, 1, fmt, n, m, reinterpret_cast<hipStream_t>(stream)));
}

int sbl_quant_acts_kgrouped(const float* x, int64_t m_tok, int64_t k, int64_t kg, int8_t* xq, float* gamma,
                            sbl_stream stream) {
  if (m_tok < 0 || m_tok > 65535 || !k_ok(k) || kg < 64 || kg % 64 != 0 || k % kg != 0 || k / kg > 65535)
    return SBL_ERR_SHAPE;
  if (m_tok == 0) return SBL_OK;
  if (!x || !xq || !gamma) return SBL_ERR_NULL;
  if (!aligned(x, 4) || !aligned(gamma, 4)) return SBL_ERR_ALIGN;
  if (ranges_overlap(x, m_tok * k * 4, xq, m_tok * k) || ranges_overlap(x, m_tok * k * 4, gamma, m_tok * (k / kg) * 4) ||
      ranges_overlap(xq, m_tok * k, gamma, m_tok * (k / kg) * 4))
    return SBL_ERR_SHAPE;
  return launch_status(sbl::launch_quant_acts_kgrouped(x, m_tok, k, kg, xq, gamma,
                                                       reinterpret_cast<hipStream_t>(stream)));
}

int sbl_linear_kgrouped(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                        const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t kg,
                        int64_t m_tok, int64_t n_out, int64_t k, float* y, sbl_stream stream) {
  return linear_kgroups(packed, meta, fmt, n, m, beta, rows_per_group, false, xq, gamma, kg, m_tok, n_out, k, y,
                        stream);
}

int sbl_linear_blocked(const uint8_t* packed, const uint8_t* meta, int32_t fmt, int32_t n, int32_t m,
                       const float* beta, int64_t rows_per_group, const int8_t* xq, const float* gamma, int64_t kg,
                       int64_t m_tok, int64_t n_out, int64_t k, float* y, sbl_stream stream) {
  return linear_kgroups(packed, meta, fmt, n, m, beta, rows_per_group, true, xq, gamma, kg, m_tok, n_out, k, y,
                        stream);
}

}  // extern "C"

namespace {

// the argument checks of both backward entry points; SBL_OK with `a` filled
int backward_args(const uint16_t* dy_bf16, int64_t m_tok, int64_t n_out, int64_t k, const uint8_t* packed,
                  const uint8_t* meta, int32_t fmt, int32_t n, int32_t m, const float* beta, const float* x,
                  const int8_t* xq, const float* gamma, float* dx, float* dw, sbl::BackwardArgs& a) {
  if (m_tok < 1 || m_tok > kMaxTokens || n_out < 8 || n_out % 8 != 0 || !k_ok(k) || n_out * k > kMaxElems)
    return SBL_ERR_SHAPE;
  if (!dy_bf16 || !gamma) return SBL_ERR_NULL;
  if (dx) {
    if (!packed || !beta || !x) return SBL_ERR_NULL;
    if (fmt != SBL_FMT_DENSE2 && fmt != SBL_FMT_NM) return SBL_ERR_UNSUPPORTED;
    if (fmt == SBL_FMT_NM && !nm_ok(n, m)) return SBL_ERR_UNSUPPORTED;
    if (fmt == SBL_FMT_NM && !meta) return SBL_ERR_NULL;
  }
  if (dw && !xq) return SBL_ERR_NULL;
  if (!aligned(dy_bf16, 16) || !aligned(gamma, 4) || (dx && (!aligned(packed, 16) || !aligned(beta, 4) ||
                                                              !aligned(x, 4) || !aligned(dx, 4) ||
                                                              (fmt == SBL_FMT_NM && !aligned(meta, 16)))) ||
      (dw && (!aligned(xq, 16) || !aligned(dw, 4))))
    return SBL_ERR_ALIGN;
  // outputs must not overlap each other or any input
  const int64_t dyb = m_tok * n_out * 2, xb = m_tok * k * 4, xqb = m_tok * k, gb = m_tok * 4;
  const int64_t dxb = m_tok * k * 4, dwb = n_out * k * 4;
  const int64_t pb = fmt == SBL_FMT_NM && nm_ok(n, m) ? n_out * (k / m) * n / 4 : n_out * (k / 4);
  const void* outs[2] = {dx, dw};
  const int64_t outb[2] = {dxb, dwb};
  if (ranges_overlap(dx, dxb, dw, dwb)) return SBL_ERR_SHAPE;
  for (int o = 0; o < 2; ++o) {
    if (!outs[o]) continue;
    if (ranges_overlap(outs[o], outb[o], dy_bf16, dyb) || ranges_overlap(outs[o], outb[o], gamma, gb) ||
        (dx && (ranges_overlap(outs[o], outb[o], x, xb) || ranges_overlap(outs[o], outb[o], packed, pb) ||
                ranges_overlap(outs[o], outb[o], beta, 4) ||
                (fmt == SBL_FMT_NM && ranges_overlap(outs[o], outb[o], meta, n_out * (k / 8))))) ||
        (dw && ranges_overlap(outs[o], outb[o], xq, xqb)))
      return SBL_ERR_SHAPE;
  }
  a.dy = dy_bf16;
  a.m_tok = m_tok;
  a.n_out = n_out;
  a.k = k;
  a.packed = packed;
  a.meta = fmt == SBL_FMT_NM ? meta : nullptr;
  a.fmt = fmt;
  a.n = n;
  a.m = m;
  a.beta = beta;
  a.x = x;
  a.xq = xq;
  a.gamma = gamma;
  a.dx = dx;
  a.dw = dw;
  return SBL_OK;
}

}  // namespace

extern "C" {

int sbl_linear_backward(const uint16_t* dy_bf16, int64_t m_tok, int64_t n_out, int64_t k, const uint8_t* packed,
                        const uint8_t* meta, int32_t fmt, int32_t n, int32_t m, const float* beta, const float* x,
                        const int8_t* xq, const float* gamma, float* dx, float* dw, sbl_stream stream) {
  if (!dx && !dw) {
    if (m_tok < 1 || m_tok > kMaxTokens || n_out < 8 || n_out % 8 != 0 || !k_ok(k) || n_out * k > kMaxElems)
      return SBL_ERR_SHAPE;
    return SBL_OK;
  }
  sbl::BackwardArgs a;
  const int st = backward_args(dy_bf16, m_tok, n_out, k, packed, meta, fmt, n, m, beta, x, xq, gamma, dx, dw, a);
  if (st != SBL_OK) return st;
  return launch_status(sbl::launch_backward(a, reinterpret_cast<hipStream_t>(stream)));
}

int64_t sbl_backward_workspace_bytes(int64_t m_tok, int64_t n_out, int64_t k) {
  if (m_tok < 1 || m_tok > kMaxTokens || n_out < 8 || n_out % 8 != 0 || !k_ok(k) || n_out * k > kMaxElems) return -1;
  return sbl::backward_ws_bytes(m_tok, n_out, k);
}

int sbl_linear_backward_ws(const uint16_t* dy_bf16, int64_t m_tok, int64_t n_out, int64_t k, const uint8_t* packed,
                           const uint8_t* meta, int32_t fmt, int32_t n, int32_t m, const float* beta, const float* x,
                           const int8_t* xq, const float* gamma, float* dx, float* dw, void* workspace,
                           int64_t workspace_bytes, sbl_stream stream) {
  if (!dx && !dw) {
    if (m_tok < 1 || m_tok > kMaxTokens || n_out < 8 || n_out % 8 != 0 || !k_ok(k) || n_out * k > kMaxElems)
      return SBL_ERR_SHAPE;
    return SBL_OK;
  }
  sbl::BackwardArgs a;
  const int st = backward_args(dy_bf16, m_tok, n_out, k, packed, meta, fmt, n, m, beta, x, xq, gamma, dx, dw, a);
  if (st != SBL_OK) return st;
  if (!workspace) return SBL_ERR_NULL;
  if (!aligned(workspace, 256)) return SBL_ERR_ALIGN;
  const int64_t wb = sbl::backward_ws_bytes(m_tok, n_out, k);
  if (workspace_bytes < wb) return SBL_ERR_SHAPE;
  // the workspace must not overlap any input or output
  const int64_t pb = fmt == SBL_FMT_NM && nm_ok(n, m) ? n_out * (k / m) * n / 4 : n_out * (k / 4);
  if (ranges_overlap(workspace, wb, dy_bf16, m_tok * n_out * 2) || ranges_overlap(workspace, wb, gamma, m_tok * 4) ||
      ranges_overlap(workspace, wb, dx, m_tok * k * 4) || ranges_overlap(workspace, wb, dw, n_out * k * 4) ||
      (dx && (ranges_overlap(workspace, wb, x, m_tok * k * 4) || ranges_overlap(workspace, wb, packed, pb) ||
              ranges_overlap(workspace, wb, beta, 4) ||
              (fmt == SBL_FMT_NM && ranges_overlap(workspace, wb, meta, n_out * (k / 8))))) ||
      (dw && ranges_overlap(workspace, wb, xq, m_tok * k)))
    return SBL_ERR_SHAPE;
  return launch_status(sbl::launch_backward_ws(a, workspace, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
