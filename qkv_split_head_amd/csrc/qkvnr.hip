// Host side of libqkvnr.so: argument validation, launch planning, dispatch.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing and the checks can be exercised on a machine with no GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "muon.h"
#include "proj.h"
#include "qkvnr.h"

// The weight-grad slots of qkvnr_backward_noalloc: the library's own device
// memory, one copy per GPU (each device that loads the library holds it until
// the process ends).  In host code `scratch` is only a stand-in for the
// symbol, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device (library_scratch below).
static __device__ __align__(256) uint8_t scratch[QKVNR_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace qkvnr;

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

// ------------------------------------------------------------------ device

struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int cus = 0;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mu;

// Compute units of the current device, or an error if it is not a gfx950.
// `index`, when given, receives the device's index.
int current_device(int* cus, int* index = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QKVNR_EUNSUPPORTED, "no HIP device is current: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(QKVNR_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_devices_mu);
  DeviceInfo& d = g_devices[dev];
  if (!d.known) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(QKVNR_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.known = true;
  }
  if (!d.gfx950) return fail(QKVNR_EUNSUPPORTED, "device %d is not gfx950; this library has kernels for gfx950 only", dev);
  *cus = d.cus;
  if (index) *index = dev;
  return QKVNR_OK;
}

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QKVNR_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return QKVNR_OK;
}

// ------------------------------------------------------------------ validation

int elem_bytes(int32_t dtype) { return dtype == QKVNR_BF16 ? 2 : 4; }

// Bytes a packed [T, in_row_stride] tensor's rows actually span: the last row
// ends after `width` values, so a strided view of a wider buffer (padding or
// other columns after it) is not counted past its own end.
int64_t rows_extent(const qkvnr_layout* L, int es) {
  return L->T == 0 ? 0 : ((L->T - 1) * L->in_row_stride + L->width) * es;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Layout checks shared by every entry point.
int check_layout(const qkvnr_layout* L) {
  if (!L) return fail(QKVNR_EINVAL, "layout is NULL");
  if (L->kind != QKVNR_INTERLEAVED && L->kind != QKVNR_SECTIONED && L->kind != QKVNR_LATENT)
    return fail(QKVNR_EINVAL, "unknown layout kind %d", L->kind);
  if (L->dtype != QKVNR_BF16 && L->dtype != QKVNR_FP32) return fail(QKVNR_EINVAL, "unknown dtype %d", L->dtype);
  if (L->T < 0 || L->T > INT32_MAX) return fail(QKVNR_EINVAL, "T = %lld out of [0, 2^31)", (long long)L->T);
  if (L->kind == QKVNR_LATENT) {
    if (L->norm_dim <= 0 || L->rope_dim < 0 || (L->rope_dim & 1))
      return fail(QKVNR_EINVAL, "latent norm_dim %d / rope_dim %d invalid", L->norm_dim, L->rope_dim);
    if (L->width != static_cast<int64_t>(L->norm_dim) + L->rope_dim)
      return fail(QKVNR_EINVAL, "latent width %lld != norm_dim + rope_dim = %d", (long long)L->width,
                  L->norm_dim + L->rope_dim);
    if (L->dtype != QKVNR_BF16 || L->norm_dim != 512 || L->rope_dim != 64)
      return fail(QKVNR_EUNSUPPORTED, "latent rows: only bf16 with norm_dim 512 and rope_dim 64 have a kernel");
  } else {
    if (L->n_kv < 1 || L->q_per_kv < 1 || L->head_dim < 1)
      return fail(QKVNR_EINVAL, "n_kv %d, q_per_kv %d, head_dim %d must be >= 1", L->n_kv, L->q_per_kv, L->head_dim);
    const int64_t n_q = static_cast<int64_t>(L->n_kv) * L->q_per_kv;
    const int64_t blocks = n_q + 2 * static_cast<int64_t>(L->n_kv);
    // exact-total guard: the packed width must be (n_q + 2 n_kv) * head_dim
    if (L->width != blocks * L->head_dim)
      return fail(QKVNR_EINVAL, "width %lld is not the exact total (n_q + 2 n_kv) * head_dim = %lld",
                  (long long)L->width, (long long)(blocks * L->head_dim));
    if (L->rope_dim < 0 || (L->rope_dim & 1) || L->rope_dim > L->head_dim)
      return fail(QKVNR_EINVAL, "rope_dim %d must be even and in [0, head_dim]", L->rope_dim);
    if (L->head_dim != 64 && L->head_dim != 128)
      return fail(QKVNR_EUNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", L->head_dim);
    if (L->rope_dim != 0 && L->rope_dim != L->head_dim)
      return fail(QKVNR_EUNSUPPORTED, "rope_dim %d: kernels rotate the whole head (rope_dim = head_dim) or nothing",
                  L->rope_dim);
    if (blocks > 65535) return fail(QKVNR_EUNSUPPORTED, "%lld head blocks per token exceed 65535", (long long)blocks);
  }
  if (L->in_row_stride < L->width)
    return fail(QKVNR_EINVAL, "in_row_stride %lld < width %lld", (long long)L->in_row_stride, (long long)L->width);
  if ((L->in_row_stride * elem_bytes(L->dtype)) % 16 != 0)
    return fail(QKVNR_EALIGN, "input row stride of %lld bytes is not a multiple of 16",
                (long long)(L->in_row_stride * elem_bytes(L->dtype)));
  return QKVNR_OK;
}

int need16(const void* p, const char* name) {
  if (!p) return fail(QKVNR_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(QKVNR_EALIGN, "%s is not 16-byte aligned", name);
  return QKVNR_OK;
}

int need4(const void* p, const char* name) {
  if (!p) return fail(QKVNR_EINVAL, "%s is NULL", name);
  if (!aligned4(p)) return fail(QKVNR_EALIGN, "%s is not 4-byte aligned", name);
  return QKVNR_OK;
}

int must_be_null(const void* p, const char* name) {
  if (p) return fail(QKVNR_EINVAL, "%s must be NULL for latent rows", name);
  return QKVNR_OK;
}

int check_scalars(const qkvnr_layout* L, float eps, double theta) {
  if (!std::isfinite(eps) || eps < 0.0f) return fail(QKVNR_EINVAL, "eps %g must be finite and >= 0", (double)eps);
  if (L->rope_dim > 0 && (!std::isfinite(theta) || !(theta > 0.0)))
    return fail(QKVNR_EINVAL, "theta %g must be finite and > 0", theta);
  return QKVNR_OK;
}

struct Span {
  const void* p;
  int64_t bytes;
};

bool overlaps(Span a, Span b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

int check_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (const Span& o : outs) {
    for (const Span& i : ins)
      if (overlaps(o, i)) return fail(QKVNR_EINVAL, "an output overlaps an input");
    for (const Span& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return fail(QKVNR_EINVAL, "two outputs overlap");
  }
  return QKVNR_OK;
}

int check_paged(const int32_t* bt, int32_t bt_stride, int32_t tokens_per_req, int32_t page_size, int32_t num_pages) {
  if (int rc = need4(bt, "block_table")) return rc;
  if (bt_stride < 1 || tokens_per_req < 1 || page_size < 1 || num_pages < 1)
    return fail(QKVNR_EINVAL, "bt_stride %d, tokens_per_req %d, page_size %d, num_pages %d must be >= 1", bt_stride,
                tokens_per_req, page_size, num_pages);
  return QKVNR_OK;
}

// ------------------------------------------------------------------ planning

int heads_per_iter(int32_t dtype, int32_t D) { return kWave * (16 / elem_bytes(dtype)) / D; }

// turns[i] = theta^(-2i/R) / (2 pi) for the R/2 rotate-half pairs, in long double.
void fill_turns(double* turns, double theta, int R) {
  for (int i = 0; i < kMaxPairs; ++i) turns[i] = 0.0;
  if (R <= 0) return;
  const long double two_pi = 6.283185307179586476925286766559005768L;
  for (int i = 0; i < R / 2 && i < kMaxPairs; ++i)
    turns[i] = static_cast<double>(std::pow(static_cast<long double>(theta), -2.0L * i / R) / two_pi);
}

// Fill in the GQA launch arguments that depend only on the layout and the unit size U.
void plan_gqa(GqaArgs& a, const qkvnr_layout* L, int U, double theta) {
  const int hpi = heads_per_iter(L->dtype, L->head_dim);
  a.T = L->T;
  a.n_kv = L->n_kv;
  a.q_per_kv = L->q_per_kv;
  a.n_q = L->n_kv * L->q_per_kv;
  a.heads = a.n_q + 2 * L->n_kv;
  a.kind = L->kind == QKVNR_INTERLEAVED ? kInterleaved : kSectioned;
  a.iters = (a.heads + hpi - 1) / hpi;
  a.upt = (a.iters + U - 1) / U;
  a.units = L->T * a.upt;
  // ceil(2^64 / upt); upt == 1 would need 2^64, so 0 marks "no division" there
  a.upt_magic = a.upt == 1 ? 0ull
                           : static_cast<uint64_t>(((static_cast<unsigned __int128>(1) << 64) + a.upt - 1) /
                                                   static_cast<unsigned __int128>(a.upt));
  const uint32_t d = static_cast<uint32_t>(a.q_per_kv);
  a.q_magic = static_cast<uint32_t>((0x100000000ull + d - 1) / d);
  a.row_bytes = L->in_row_stride * elem_bytes(L->dtype);
  a.inv_d = 1.0f / static_cast<float>(L->head_dim);
  fill_turns(a.turns, theta, L->rope_dim);
}

#ifndef QKVNR_FWD_LDS
#define QKVNR_FWD_LDS 0
#endif
#ifndef QKVNR_BWD_LDS
#define QKVNR_BWD_LDS 0
#endif

// Blocks per launch.  A dispatch holds fewer than 2^32 work-items, so a batch with more blocks
// (for instance 2^24 tokens of a few small heads) is launched in pieces of this many blocks,
// each piece told its first work unit (or token).
constexpr int64_t kMaxLaunchBlocks = int64_t(1) << 22;

// Launches launch(grid) once per piece of at most kMaxLaunchBlocks blocks over `items` work
// items of `per_block` per block, after set_first(first item of the piece); stops at the first
// launch that fails.  `enqueued`, when given, is set if at least one piece went out.
template <typename SetFirst, typename Launch>
int launch_pieces(int64_t items, int per_block, const char* what, SetFirst&& set_first, Launch&& launch,
                  bool* enqueued = nullptr) {
  const int64_t blocks = (items + per_block - 1) / per_block;
  for (int64_t b0 = 0; b0 < blocks; b0 += kMaxLaunchBlocks) {
    set_first(b0 * per_block);
    launch(dim3(static_cast<uint32_t>(std::min(kMaxLaunchBlocks, blocks - b0))));
    if (int rc = launched(what)) return rc;
    if (enqueued) *enqueued = true;
  }
  return QKVNR_OK;
}

// Below this many work units of kFwdU iterations (8 waves per CU of the
// part), a batch is latency-bound: the forward then uses one iteration per wave.
constexpr int64_t kSmallBatchUnits = 2048;

// One forward launch, the layout a template argument (the interleaved one maps heads to row blocks).
template <typename IO, int DD, bool R, bool PAGED, int U, int DEPTH>
void fwd_gqa_launch(const GqaArgs& a, dim3 g, dim3 b, hipStream_t s) {
  if (a.kind == kInterleaved)
    hipLaunchKernelGGL((fwd_gqa_kernel<IO, DD, R, PAGED, U, DEPTH, true>), g, b, QKVNR_FWD_LDS, s, a);
  else
    hipLaunchKernelGGL((fwd_gqa_kernel<IO, DD, R, PAGED, U, DEPTH, false>), g, b, QKVNR_FWD_LDS, s, a);
}

template <typename IO, int DD, bool R>
void bwd_gqa_launch(const GqaArgs& a, dim3 g, dim3 b, hipStream_t s) {
  if (a.kind == kInterleaved)
    hipLaunchKernelGGL((bwd_gqa_kernel<IO, DD, R, true>), g, b, QKVNR_BWD_LDS, s, a);
  else
    hipLaunchKernelGGL((bwd_gqa_kernel<IO, DD, R, false>), g, b, QKVNR_BWD_LDS, s, a);
}

template <bool PAGED, int U, int DEPTH>
int launch_fwd_gqa(GqaArgs a, int32_t dtype, int32_t D, bool rope, hipStream_t s) {
  const dim3 b(kBlockThreads);
  auto launch = [&](dim3 g) {
#define QKVNR_FWD(IO, DD, R) fwd_gqa_launch<IO, DD, R, PAGED, U, DEPTH>(a, g, b, s)
    if (dtype == QKVNR_BF16) {
      if (D == 64) { if (rope) QKVNR_FWD(uint16_t, 64, true); else QKVNR_FWD(uint16_t, 64, false); }
      else         { if (rope) QKVNR_FWD(uint16_t, 128, true); else QKVNR_FWD(uint16_t, 128, false); }
    } else {
      if (D == 64) { if (rope) QKVNR_FWD(float, 64, true); else QKVNR_FWD(float, 64, false); }
      else         { if (rope) QKVNR_FWD(float, 128, true); else QKVNR_FWD(float, 128, false); }
    }
#undef QKVNR_FWD
  };
  return launch_pieces(a.units, kWavesPerBlock, "forward", [&](int64_t u0) { a.unit0 = u0; }, launch);
}

int launch_bwd_gqa(GqaArgs a, int32_t dtype, int32_t D, bool rope, hipStream_t s, bool* enqueued) {
  const dim3 b(kBwdBlockThreads);
  auto launch = [&](dim3 g) {
#define QKVNR_BWD(IO, DD, R) bwd_gqa_launch<IO, DD, R>(a, g, b, s)
    if (dtype == QKVNR_BF16) {
      if (D == 64) { if (rope) QKVNR_BWD(uint16_t, 64, true); else QKVNR_BWD(uint16_t, 64, false); }
      else         { if (rope) QKVNR_BWD(uint16_t, 128, true); else QKVNR_BWD(uint16_t, 128, false); }
    } else {
      if (D == 64) { if (rope) QKVNR_BWD(float, 64, true); else QKVNR_BWD(float, 64, false); }
      else         { if (rope) QKVNR_BWD(float, 128, true); else QKVNR_BWD(float, 128, false); }
    }
#undef QKVNR_BWD
  };
  return launch_pieces(a.units, kBwdWavesPerBlock, "backward", [&](int64_t u0) { a.unit0 = u0; }, launch,
                       enqueued);
}

constexpr int kLatentBlocksPerCu = 8;

int latent_forward(const qkvnr_layout* L, const void* qkv, const int32_t* positions, const void* k_norm_w,
                   float eps, double theta, void* out, int64_t out_bytes, const int32_t* bt, int32_t bt_stride,
                   int32_t tokens_per_req, int32_t page_size, int32_t num_pages, bool paged, hipStream_t stream) {
  if (L->T == 0) return QKVNR_OK;  // nothing is read or written
  if (int rc = need16(qkv, "qkv")) return rc;
  if (int rc = need4(positions, "positions")) return rc;
  if (int rc = need16(k_norm_w, "k_norm_w (latent norm weight)")) return rc;
  if (int rc = need16(out, paged ? "k_pool" : "k")) return rc;
  const int64_t row_bytes = L->in_row_stride * 2;
  if (int rc = check_disjoint({{out, out_bytes}}, {{qkv, rows_extent(L, 2)}, {positions, L->T * 4}, {k_norm_w, 1024}}))
    return rc;
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  LatentArgs a{};
  a.rows = static_cast<const uint8_t*>(qkv);
  a.row_bytes = row_bytes;
  a.pos = positions;
  a.w = static_cast<const uint8_t*>(k_norm_w);
  a.out = static_cast<uint8_t*>(out);
  a.eps = eps;
  fill_turns(a.turns, theta, L->rope_dim);
  a.T = L->T;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.tokens_per_req = tokens_per_req;
  a.page_size = page_size;
  a.num_pages = num_pages;
  int64_t grid = (L->T + kWavesPerBlock - 1) / kWavesPerBlock;
  if (grid > static_cast<int64_t>(cus) * kLatentBlocksPerCu) grid = static_cast<int64_t>(cus) * kLatentBlocksPerCu;
  if (paged)
    hipLaunchKernelGGL((fwd_latent_kernel<true>), dim3(grid), dim3(kBlockThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_latent_kernel<false>), dim3(grid), dim3(kBlockThreads), 0, stream, a);
  return launched("latent forward");
}

int gqa_forward(const qkvnr_layout* L, const void* qkv, const int32_t* positions, const void* q_norm_w,
                const void* k_norm_w, float eps, double theta, void* q, void* k, void* v, int64_t kv_bytes,
                const int32_t* bt, int32_t bt_stride, int32_t tokens_per_req, int32_t page_size,
                int32_t num_pages, bool paged, hipStream_t stream) {
  const bool rope = L->rope_dim > 0;
  const int es = elem_bytes(L->dtype);
  if (L->T == 0) return QKVNR_OK;  // nothing is read or written
  if (int rc = need16(qkv, "qkv")) return rc;
  if (rope || paged) {
    if (int rc = need4(positions, "positions")) return rc;
  }
  if (int rc = need16(q_norm_w, "q_norm_w")) return rc;
  if (int rc = need16(k_norm_w, "k_norm_w")) return rc;
  if (int rc = need16(q, "q")) return rc;
  if (int rc = need16(k, paged ? "k_pool" : "k")) return rc;
  if (int rc = need16(v, paged ? "v_pool" : "v")) return rc;
  const int64_t D = L->head_dim, n_q = static_cast<int64_t>(L->n_kv) * L->q_per_kv;
  const int64_t wbytes = D * es;
  if (int rc = check_disjoint({{q, L->T * n_q * D * es}, {k, kv_bytes}, {v, kv_bytes}},
                              {{qkv, rows_extent(L, es)},
                               {positions, positions ? L->T * 4 : 0},
                               {q_norm_w, wbytes},
                               {k_norm_w, wbytes}}))
    return rc;
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  GqaArgs a{};
  plan_gqa(a, L, kFwdU, theta);
  const bool small = a.units < kSmallBatchUnits;
  if (small) plan_gqa(a, L, 1, theta);
  a.qkv = static_cast<const uint8_t*>(qkv);
  a.pos = positions;
  a.wq = static_cast<const uint8_t*>(q_norm_w);
  a.wk = static_cast<const uint8_t*>(k_norm_w);
  a.q = static_cast<uint8_t*>(q);
  a.k = static_cast<uint8_t*>(k);
  a.v = static_cast<uint8_t*>(v);
  a.eps = eps;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.tokens_per_req = tokens_per_req;
  a.page_size = page_size;
  a.num_pages = num_pages;
  if (paged) {
    if (small) return launch_fwd_gqa<true, 1, 1>(a, L->dtype, L->head_dim, rope, stream);
    return launch_fwd_gqa<true, kFwdU, kFwdDepth>(a, L->dtype, L->head_dim, rope, stream);
  }
  if (small) return launch_fwd_gqa<false, 1, 1>(a, L->dtype, L->head_dim, rope, stream);
  return launch_fwd_gqa<false, kFwdU, kFwdDepth>(a, L->dtype, L->head_dim, rope, stream);
}

// ------------------------------------------------------------------ backward

static_assert(static_cast<int64_t>(kWgradSlots) * 2 * 128 * sizeof(float) <= QKVNR_NOALLOC_SCRATCH_BYTES,
              "the library's scratch holds the slots of the widest head");

struct ScratchState {
  void* ptr = nullptr;  // device address of `scratch` on this device
  bool dirty = true;    // zero it before the next use (first use, or a call whose fold failed to launch)
};
ScratchState g_scratch[kMaxDevices];  // guarded by g_scratch_mu
std::mutex g_scratch_mu;

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The device address of this device's scratch, looked up on its first use, and
// zeroed on `stream` (a kernel, so that a caller may capture it) when it may
// hold anything but zeros.
int library_scratch(int dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& st = g_scratch[dev];
  if (!st.ptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QKVNR_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    st.ptr = p;
  }
  if (st.dirty) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(4), dim3(1024), 0, stream, static_cast<uint32_t*>(st.ptr),
                       QKVNR_NOALLOC_SCRATCH_BYTES / 4);
    if (int rc = launched("scratch zeroing")) return rc;
    st.dirty = false;
  }
  *out = st.ptr;
  return QKVNR_OK;
}

void mark_scratch_dirty(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].dirty = true;
}

// qkvnr_backward (caller's workspace) and qkvnr_backward_noalloc (the library's
// scratch, when use_scratch) share everything but where the slots live.
int backward_impl(const qkvnr_layout* layout, const void* qkv, const int32_t* positions, const void* q_norm_w,
                  const void* k_norm_w, float eps, double theta, const void* dq, const void* dk, const void* dv,
                  void* dqkv, float* dq_norm_w, float* dk_norm_w, void* workspace, int64_t workspace_bytes,
                  bool use_scratch, hipStream_t stream) {
  if (int rc = check_layout(layout)) return rc;
  const qkvnr_layout* L = layout;
  if (L->kind == QKVNR_LATENT) return fail(QKVNR_EUNSUPPORTED, "backward of latent rows has no kernel");
  if (int rc = check_scalars(L, eps, theta)) return rc;
  const bool rope = L->rope_dim > 0;
  const int es = elem_bytes(L->dtype);
  if (int rc = need4(dq_norm_w, "dq_norm_w")) return rc;
  if (int rc = need4(dk_norm_w, "dk_norm_w")) return rc;
  const int64_t D = L->head_dim, n_q = static_cast<int64_t>(L->n_kv) * L->q_per_kv;
  if (overlaps({dq_norm_w, D * 4}, {dk_norm_w, D * 4})) return fail(QKVNR_EINVAL, "two outputs overlap");
  const int64_t ws_need = static_cast<int64_t>(kWgradSlots) * 2 * D * static_cast<int64_t>(sizeof(float));
  if (use_scratch && ws_need > QKVNR_NOALLOC_SCRATCH_BYTES)
    return fail(QKVNR_EINVAL, "head_dim %lld needs %lld bytes of weight-grad slots; the library's scratch holds %d",
                (long long)D, (long long)ws_need, QKVNR_NOALLOC_SCRATCH_BYTES);
  int cus = 0, dev = -1;
  if (L->T == 0) {  // no token is read and the slots are not touched: the weight grads are zero
    if (int rc = current_device(&cus)) return rc;
    hipLaunchKernelGGL(zero2_f32_kernel, dim3(1), dim3(256), 0, stream, dq_norm_w, dk_norm_w, static_cast<int>(D));
    return launched("weight-grad zeroing");
  }
  if (int rc = need16(qkv, "qkv")) return rc;
  if (rope) {
    if (int rc = need4(positions, "positions")) return rc;
  }
  if (int rc = need16(q_norm_w, "q_norm_w")) return rc;
  if (int rc = need16(k_norm_w, "k_norm_w")) return rc;
  if (int rc = need16(dq, "dq")) return rc;
  if (int rc = need16(dk, "dk")) return rc;
  if (int rc = need16(dv, "dv")) return rc;
  if (int rc = need16(dqkv, "dqkv")) return rc;
  if (!use_scratch) {
    if (int rc = need16(workspace, "workspace")) return rc;
    if (workspace_bytes < ws_need)
      return fail(QKVNR_EINVAL, "workspace of %lld bytes is smaller than the %lld needed", (long long)workspace_bytes,
                  (long long)ws_need);
  }
  const int64_t kvb = L->T * L->n_kv * D * es;
  if (int rc = check_disjoint(
          {{dqkv, rows_extent(L, es)}, {dq_norm_w, D * 4}, {dk_norm_w, D * 4}, {workspace, use_scratch ? 0 : ws_need}},
          {{qkv, rows_extent(L, es)}, {positions, positions ? L->T * 4 : 0}, {q_norm_w, D * es},
           {k_norm_w, D * es}, {dq, L->T * n_q * D * es}, {dk, kvb}, {dv, kvb}}))
    return rc;
  if (int rc = current_device(&cus, &dev)) return rc;
  if (use_scratch) {
    if (int rc = library_scratch(dev, stream, &workspace)) return rc;
  }
  GqaArgs a{};
  plan_gqa(a, L, kBwdU, theta);
  a.qkv = static_cast<const uint8_t*>(qkv);
  a.pos = positions;
  a.wq = static_cast<const uint8_t*>(q_norm_w);
  a.wk = static_cast<const uint8_t*>(k_norm_w);
  a.dq = static_cast<const uint8_t*>(dq);
  a.dk = static_cast<const uint8_t*>(dk);
  a.dv = static_cast<const uint8_t*>(dv);
  a.dqkv = static_cast<uint8_t*>(dqkv);
  a.dwq = dq_norm_w;
  a.dwk = dk_norm_w;
  a.slots = static_cast<float*>(workspace);
  a.eps = eps;
  bool enqueued = false;
  const int rc_bwd = launch_bwd_gqa(a, L->dtype, L->head_dim, rope, stream, &enqueued);
  if (!enqueued) return rc_bwd;  // nothing reached the slots
  // Once any piece is enqueued its atomics reach the slots, so the fold, which
  // zeroes them again, is enqueued even when a later piece failed to launch.
  if (D == 64)
    hipLaunchKernelGGL(wgrad_fold_kernel<64>, dim3(1), dim3(kFoldThreads), 0, stream, a.slots, dq_norm_w, dk_norm_w);
  else
    hipLaunchKernelGGL(wgrad_fold_kernel<128>, dim3(1), dim3(kFoldThreads), 0, stream, a.slots, dq_norm_w, dk_norm_w);
  const hipError_t fold_err = hipGetLastError();
  if (fold_err == hipSuccess) return rc_bwd;
  // the slots keep this call's partial sums: they must be zeroed before the next use
  if (use_scratch) mark_scratch_dirty(dev);
  if (rc_bwd != QKVNR_OK) return rc_bwd;  // keep the first failure's message
  return fail(QKVNR_EHIP, "weight-grad fold launch failed: %s", hipGetErrorString(fold_err));
}

template <int D, bool ROPE>
void launch_proj(const ProjArgs& a, bool tail, dim3 grid, dim3 block, hipStream_t stream) {
  if (tail) hipLaunchKernelGGL((proj_qkv_kernel<D, ROPE, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((proj_qkv_kernel<D, ROPE, false>), grid, block, 0, stream, a);
}

}  // namespace

extern "C" {

int qkvnr_forward(const qkvnr_layout* layout, const void* qkv, const int32_t* positions, const void* q_norm_w,
                  const void* k_norm_w, float eps, double theta, void* q, void* k, void* v, hipStream_t stream) {
  if (int rc = check_layout(layout)) return rc;
  if (int rc = check_scalars(layout, eps, theta)) return rc;
  const qkvnr_layout* L = layout;
  if (L->kind == QKVNR_LATENT) {
    if (int rc = must_be_null(q_norm_w, "q_norm_w")) return rc;
    if (int rc = must_be_null(q, "q")) return rc;
    if (int rc = must_be_null(v, "v")) return rc;
    return latent_forward(L, qkv, positions, k_norm_w, eps, theta, k, L->T * L->width * 2, nullptr, 0, 1, 1, 1,
                          false, stream);
  }
  const int64_t kv_bytes = L->T * L->n_kv * static_cast<int64_t>(L->head_dim) * elem_bytes(L->dtype);
  return gqa_forward(L, qkv, positions, q_norm_w, k_norm_w, eps, theta, q, k, v, kv_bytes, nullptr, 0, 1, 1, 1,
                     false, stream);
}

int qkvnr_forward_paged(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                        const void* q_norm_w, const void* k_norm_w, float eps, double theta,
                        const int32_t* block_table, int32_t bt_stride, int32_t tokens_per_req, int32_t page_size,
                        int32_t num_pages, void* q, void* k_pool, void* v_pool, hipStream_t stream) {
  if (int rc = check_layout(layout)) return rc;
  if (int rc = check_scalars(layout, eps, theta)) return rc;
  if (int rc = check_paged(block_table, bt_stride, tokens_per_req, page_size, num_pages)) return rc;
  const qkvnr_layout* L = layout;
  const int64_t slots = static_cast<int64_t>(num_pages) * page_size;
  if (L->kind == QKVNR_LATENT) {
    if (int rc = must_be_null(q_norm_w, "q_norm_w")) return rc;
    if (int rc = must_be_null(q, "q")) return rc;
    if (int rc = must_be_null(v_pool, "v_pool")) return rc;
    return latent_forward(L, qkv, positions, k_norm_w, eps, theta, k_pool, slots * L->width * 2, block_table,
                          bt_stride, tokens_per_req, page_size, num_pages, true, stream);
  }
  const int64_t kv_bytes = slots * L->n_kv * static_cast<int64_t>(L->head_dim) * elem_bytes(L->dtype);
  return gqa_forward(L, qkv, positions, q_norm_w, k_norm_w, eps, theta, q, k_pool, v_pool, kv_bytes, block_table,
                     bt_stride, tokens_per_req, page_size, num_pages, true, stream);
}

int64_t qkvnr_backward_workspace_bytes(const qkvnr_layout* layout) {
  const int64_t D = layout && layout->head_dim > 0 ? layout->head_dim : 128;
  return static_cast<int64_t>(kWgradSlots) * 2 * D * static_cast<int64_t>(sizeof(float));
}

int qkvnr_backward(const qkvnr_layout* layout, const void* qkv, const int32_t* positions, const void* q_norm_w,
                   const void* k_norm_w, float eps, double theta, const void* dq, const void* dk, const void* dv,
                   void* dqkv, float* dq_norm_w, float* dk_norm_w, void* workspace, int64_t workspace_bytes,
                   hipStream_t stream) {
  return backward_impl(layout, qkv, positions, q_norm_w, k_norm_w, eps, theta, dq, dk, dv, dqkv, dq_norm_w,
                       dk_norm_w, workspace, workspace_bytes, false, stream);
}

int qkvnr_backward_noalloc(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                           const void* q_norm_w, const void* k_norm_w, float eps, double theta, const void* dq,
                           const void* dk, const void* dv, void* dqkv, float* dq_norm_w, float* dk_norm_w,
                           hipStream_t stream) {
  return backward_impl(layout, qkv, positions, q_norm_w, k_norm_w, eps, theta, dq, dk, dv, dqkv, dq_norm_w,
                       dk_norm_w, nullptr, 0, true, stream);
}

int qkvnr_rope_inplace(int32_t dtype, int64_t T, int32_t heads, int64_t token_stride, int32_t head_stride,
                       int32_t rope_offset, int32_t rope_dim, const int32_t* positions, double theta, void* x,
                       hipStream_t stream) {
  if (dtype != QKVNR_BF16 && dtype != QKVNR_FP32) return fail(QKVNR_EINVAL, "unknown dtype %d", dtype);
  if (dtype != QKVNR_BF16) return fail(QKVNR_EUNSUPPORTED, "rope_inplace: only bf16 has a kernel");
  if (T < 0 || T > INT32_MAX) return fail(QKVNR_EINVAL, "T = %lld out of [0, 2^31)", (long long)T);
  if (heads < 1) return fail(QKVNR_EINVAL, "heads %d must be >= 1", heads);
  if (rope_dim != 64 && rope_dim != 128)
    return fail(QKVNR_EUNSUPPORTED, "rope_inplace: rope_dim %d: kernels exist for 64 and 128", rope_dim);
  if (rope_offset < 0 || head_stride < 1 || static_cast<int64_t>(rope_offset) + rope_dim > head_stride)
    return fail(QKVNR_EINVAL, "rope part [%d, %d) does not fit a head of stride %d", rope_offset,
                rope_offset + rope_dim, head_stride);
  if (static_cast<int64_t>(heads) * head_stride > token_stride)
    return fail(QKVNR_EINVAL, "%d heads of stride %d do not fit a token stride of %lld", heads, head_stride,
                (long long)token_stride);
  if ((rope_offset * 2) % 16 || (head_stride * 2) % 16 || (token_stride * 2) % 16)
    return fail(QKVNR_EALIGN, "rope offset, head stride and token stride must be multiples of 8 values");
  if (!std::isfinite(theta) || theta <= 0.0) return fail(QKVNR_EINVAL, "theta %g must be finite and > 0", theta);
  if (T == 0) return QKVNR_OK;  // nothing is read or written
  if (int rc = need16(x, "x")) return rc;
  if (int rc = need4(positions, "positions")) return rc;
  const int64_t x_bytes = (T - 1) * token_stride * 2 + static_cast<int64_t>(heads) * head_stride * 2;
  if (overlaps({x, x_bytes}, {positions, T * 4})) return fail(QKVNR_EINVAL, "x overlaps positions");
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  RopeArgs a{};
  a.x = static_cast<uint8_t*>(x);
  a.T = T;
  a.token_bytes = token_stride * 2;
  a.head_bytes = head_stride * 2;
  a.rope_off_bytes = rope_offset * 2;
  a.heads = heads;
  const int hpi = kWave / (rope_dim / 8);
  a.iters = (heads + hpi - 1) / hpi;
  a.pos = positions;
  fill_turns(a.turns, theta, rope_dim);
  const dim3 b(kBlockThreads);
  return launch_pieces(
      T, kWavesPerBlock, "rope in place", [&](int64_t t0) { a.t0 = t0; },
      [&](dim3 g) {
        if (rope_dim == 64)
          hipLaunchKernelGGL(rope_inplace_kernel<64>, g, b, 0, stream, a);
        else
          hipLaunchKernelGGL(rope_inplace_kernel<128>, g, b, 0, stream, a);
      });
}

int qkvnr_fused_head_blocks(int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t weight_rows, int64_t* blocks) {
  if (!blocks) return fail(QKVNR_EINVAL, "blocks is NULL");
  *blocks = 0;
  if (n_q < 0 || n_kv < 0 || n_q + static_cast<int64_t>(n_kv) < 1 || head_dim < 1)
    return fail(QKVNR_EINVAL, "n_q %d, n_kv %d, head_dim %d do not describe heads", n_q, n_kv, head_dim);
  const int64_t heads = n_q + 2 * static_cast<int64_t>(n_kv);
  if (weight_rows != heads * head_dim)
    return fail(QKVNR_EINVAL, "weight of %lld rows is not the exact fused total (n_q + 2 n_kv) * head_dim = %lld",
                (long long)weight_rows, (long long)(heads * head_dim));
  *blocks = heads;
  return QKVNR_OK;
}

int qkvnr_gram_partials(int64_t blocks, int32_t d, int64_t cols, const void* x, int32_t parts, float* out,
                        hipStream_t stream) {
  if (blocks < 0 || blocks > kMaxLaunchBlocks)  // one launch, one workgroup (row) per block
    return fail(QKVNR_EINVAL, "blocks %lld out of [0, 2^22]", (long long)blocks);
  if (d != 32 && d != 64 && d != 96 && d != 128)
    return fail(QKVNR_EUNSUPPORTED, "block side %d: kernels exist for 32, 64, 96 and 128", d);
  if (cols < 1 || cols % 8) return fail(QKVNR_EALIGN, "cols %lld must be a positive multiple of 8", (long long)cols);
  if (cols > (1 << 30)) return fail(QKVNR_EINVAL, "cols %lld above 2^30", (long long)cols);
  if (parts < 1 || parts > 65535) return fail(QKVNR_EINVAL, "parts %d out of [1, 65535]", parts);
  if (blocks == 0) return QKVNR_OK;
  if (blocks > (INT64_MAX / 8) / (int64_t(d) * std::max<int64_t>(cols, int64_t(parts) * d)))
    return fail(QKVNR_EINVAL, "%lld blocks of %d x %lld do not fit a 64-bit byte count", (long long)blocks, d,
                (long long)cols);
  if (int rc = need16(x, "x")) return rc;
  if (int rc = need4(out, "out")) return rc;
  const int64_t n_out = blocks * parts * d * d;
  if (overlaps({x, blocks * d * cols * 2}, {out, n_out * 4})) return fail(QKVNR_EINVAL, "out overlaps x");
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  // column slices of a multiple of 16, as even as that allows
  const int sl = static_cast<int>(((cols + parts - 1) / parts + 15) / 16 * 16);
  const dim3 g(static_cast<uint32_t>(blocks), static_cast<uint32_t>(parts));
  const auto* xs = static_cast<const uint16_t*>(x);
  const int c = static_cast<int>(cols);
  switch (d) {
    case 32: hipLaunchKernelGGL(gram_partials_kernel<32>, g, dim3(kWave * 1), 0, stream, xs, c, sl, out); break;
    case 64: hipLaunchKernelGGL(gram_partials_kernel<64>, g, dim3(kWave * 2), 0, stream, xs, c, sl, out); break;
    case 96: hipLaunchKernelGGL(gram_partials_kernel<96>, g, dim3(kWave * 3), 0, stream, xs, c, sl, out); break;
    default: hipLaunchKernelGGL(gram_partials_kernel<128>, g, dim3(kWave * 4), 0, stream, xs, c, sl, out); break;
  }
  return launched("Gram partials");
}

int qkvnr_ns_poly(int32_t dtype, int64_t blocks, int32_t d, float* gram, int32_t parts, int32_t first,
                  float scale, float eps, void* p, hipStream_t stream) {
  if (dtype != QKVNR_BF16 && dtype != QKVNR_FP32) return fail(QKVNR_EINVAL, "unknown dtype %d", dtype);
  if (blocks < 0 || blocks > kMaxLaunchBlocks)  // one launch, one workgroup (row) per block
    return fail(QKVNR_EINVAL, "blocks %lld out of [0, 2^22]", (long long)blocks);
  if (d < 1 || d > kNsMaxD) return fail(QKVNR_EUNSUPPORTED, "block side %d: the kernel holds 1..%d", d, kNsMaxD);
  if (parts < 1) return fail(QKVNR_EINVAL, "parts %d must be >= 1", parts);
  if (!std::isfinite(scale) || scale <= 0.0f) return fail(QKVNR_EINVAL, "scale %g must be finite and > 0", (double)scale);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(QKVNR_EINVAL, "eps %g must be finite and >= 0", (double)eps);
  if (blocks == 0) return QKVNR_OK;
  if (int rc = need16(gram, "gram")) return rc;
  if (!p) return fail(QKVNR_EINVAL, "p is NULL");
  if (reinterpret_cast<uintptr_t>(p) % elem_bytes(dtype)) return fail(QKVNR_EALIGN, "p is not aligned to its dtype");
  const int64_t n = blocks * d * d;
  if (overlaps({gram, n * parts * 4}, {p, n * elem_bytes(dtype)})) return fail(QKVNR_EINVAL, "p overlaps gram");
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  const dim3 grid(static_cast<uint32_t>(blocks), static_cast<uint32_t>((d + 31) / 32));
  const int fi = first ? 1 : 0;
  if (dtype == QKVNR_BF16) {
    auto* o = static_cast<uint16_t*>(p);
    if (d == 128) hipLaunchKernelGGL((ns_poly_kernel<uint16_t, 128>), grid, dim3(kNsThreads), 0, stream, gram, o, d, parts, fi, scale, eps);
    else hipLaunchKernelGGL((ns_poly_kernel<uint16_t, 0>), grid, dim3(kNsThreads), 0, stream, gram, o, d, parts, fi, scale, eps);
  } else {
    auto* o = static_cast<float*>(p);
    if (d == 128) hipLaunchKernelGGL((ns_poly_kernel<float, 128>), grid, dim3(kNsThreads), 0, stream, gram, o, d, parts, fi, scale, eps);
    else hipLaunchKernelGGL((ns_poly_kernel<float, 0>), grid, dim3(kNsThreads), 0, stream, gram, o, d, parts, fi, scale, eps);
  }
  return launched("Newton-Schulz polynomial");
}

int qkvnr_ns_update(int64_t blocks, int32_t d, int64_t cols, const void* p, const void* x, void* y,
                    int32_t parts, float* gram, hipStream_t stream) {
  if (blocks < 0 || blocks > kMaxLaunchBlocks)  // one launch, one workgroup (row) per block
    return fail(QKVNR_EINVAL, "blocks %lld out of [0, 2^22]", (long long)blocks);
  if (d != 64 && d != 128) return fail(QKVNR_EUNSUPPORTED, "block side %d: the update kernel exists for 64 and 128", d);
  if (cols < 1 || cols % 8) return fail(QKVNR_EALIGN, "cols %lld must be a positive multiple of 8", (long long)cols);
  if (cols > (1 << 30)) return fail(QKVNR_EINVAL, "cols %lld above 2^30", (long long)cols);
  if (parts < 1 || parts > 65535) return fail(QKVNR_EINVAL, "parts %d out of [1, 65535]", parts);
  if (blocks == 0) return QKVNR_OK;
  if (blocks > (INT64_MAX / 8) / (int64_t(d) * std::max<int64_t>(cols, int64_t(parts) * d)))
    return fail(QKVNR_EINVAL, "%lld blocks of %d x %lld do not fit a 64-bit byte count", (long long)blocks, d,
                (long long)cols);
  if (int rc = need16(p, "p")) return rc;
  if (int rc = need16(x, "x")) return rc;
  if (int rc = need16(y, "y")) return rc;
  if (gram) {
    if (int rc = need4(gram, "gram")) return rc;
  }
  const int64_t xb = blocks * d * cols * 2, pb = blocks * d * d * 2, gb = blocks * parts * d * d * 4;
  if (overlaps({y, xb}, {x, xb}) || overlaps({y, xb}, {p, pb})) return fail(QKVNR_EINVAL, "y overlaps x or p");
  if (gram && (overlaps({gram, gb}, {x, xb}) || overlaps({gram, gb}, {y, xb}) || overlaps({gram, gb}, {p, pb})))
    return fail(QKVNR_EINVAL, "gram overlaps p, x or y");
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  const int sl = static_cast<int>(((cols + parts - 1) / parts + 15) / 16 * 16);  // the Gram kernel's slices
  const dim3 g(static_cast<uint32_t>(blocks), static_cast<uint32_t>(parts));
  const auto* ps = static_cast<const uint16_t*>(p);
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* ys = static_cast<uint16_t*>(y);
  const int c = static_cast<int>(cols);
  if (d == 128) {
    if (gram) hipLaunchKernelGGL((ns_update_kernel<128, true>), g, dim3(kWave * 4), 0, stream, ps, xs, ys, c, sl, gram);
    else hipLaunchKernelGGL((ns_update_kernel<128, false>), g, dim3(kWave * 4), 0, stream, ps, xs, ys, c, sl, gram);
  } else {
    if (gram) hipLaunchKernelGGL((ns_update_kernel<64, true>), g, dim3(kWave * 2), 0, stream, ps, xs, ys, c, sl, gram);
    else hipLaunchKernelGGL((ns_update_kernel<64, false>), g, dim3(kWave * 2), 0, stream, ps, xs, ys, c, sl, gram);
  }
  return launched("Newton-Schulz update");
}

int qkvnr_ns_collapse(int64_t blocks, int32_t d, const float* gram, int32_t parts, int32_t steps, float scale,
                      float eps, void* m, hipStream_t stream) {
  if (blocks < 0 || blocks > kMaxLaunchBlocks)  // one launch, one workgroup per block
    return fail(QKVNR_EINVAL, "blocks %lld out of [0, 2^22]", (long long)blocks);
  if (d != 64 && d != 128) return fail(QKVNR_EUNSUPPORTED, "block side %d: the collapse kernel exists for 64 and 128", d);
  if (parts < 1 || parts > 65535) return fail(QKVNR_EINVAL, "parts %d out of [1, 65535]", parts);
  if (steps < 1 || steps > 64) return fail(QKVNR_EINVAL, "steps %d out of [1, 64]", steps);
  if (!std::isfinite(scale) || scale <= 0.0f) return fail(QKVNR_EINVAL, "scale %g must be finite and > 0", (double)scale);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(QKVNR_EINVAL, "eps %g must be finite and >= 0", (double)eps);
  if (blocks == 0) return QKVNR_OK;
  if (int rc = need16(gram, "gram")) return rc;
  if (int rc = need16(m, "m")) return rc;
  const int64_t n = blocks * d * d;
  if (overlaps({gram, n * parts * 4}, {m, n * 2 * 2})) return fail(QKVNR_EINVAL, "m overlaps gram");
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  auto* mo = static_cast<uint16_t*>(m);
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (d == 128)
    hipLaunchKernelGGL((ns_collapse_kernel<128>), grid, dim3(kWave * ns_collapse_waves(128)), 0, stream, gram, parts,
                       steps, scale, eps, mo);
  else
    hipLaunchKernelGGL((ns_collapse_kernel<64>), grid, dim3(kWave * ns_collapse_waves(64)), 0, stream, gram, parts,
                       steps, scale, eps, mo);
  return launched("Newton-Schulz collapse");
}

int qkvnr_ns_apply(int64_t blocks, int32_t d, int64_t cols, const void* m, const void* x, void* y, int32_t parts,
                   hipStream_t stream) {
  if (blocks < 0 || blocks > kMaxLaunchBlocks)  // one launch, one workgroup (row) per block
    return fail(QKVNR_EINVAL, "blocks %lld out of [0, 2^22]", (long long)blocks);
  if (d != 64 && d != 128) return fail(QKVNR_EUNSUPPORTED, "block side %d: the update kernel exists for 64 and 128", d);
  if (cols < 1 || cols % 8) return fail(QKVNR_EALIGN, "cols %lld must be a positive multiple of 8", (long long)cols);
  if (cols > (1 << 30)) return fail(QKVNR_EINVAL, "cols %lld above 2^30", (long long)cols);
  if (parts < 1 || parts > 65535) return fail(QKVNR_EINVAL, "parts %d out of [1, 65535]", parts);
  if (blocks == 0) return QKVNR_OK;
  if (blocks > (INT64_MAX / 8) / (int64_t(d) * std::max<int64_t>(cols, 2 * d)))
    return fail(QKVNR_EINVAL, "%lld blocks of %d x %lld do not fit a 64-bit byte count", (long long)blocks, d,
                (long long)cols);
  if (int rc = need16(m, "m")) return rc;
  if (int rc = need16(x, "x")) return rc;
  if (int rc = need16(y, "y")) return rc;
  const int64_t xb = blocks * d * cols * 2, mb = blocks * 2 * d * d * 2;
  if (int rc = check_disjoint({{y, xb}}, {{x, xb}, {m, mb}})) return rc;
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  const int sl = static_cast<int>(((cols + parts - 1) / parts + 15) / 16 * 16);  // as qkvnr_ns_update
  const dim3 g(static_cast<uint32_t>(blocks), static_cast<uint32_t>(parts));
  const auto* ms = static_cast<const uint16_t*>(m);
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* ys = static_cast<uint16_t*>(y);
  const int c = static_cast<int>(cols);
  if (d == 128)
    hipLaunchKernelGGL((ns_update_kernel<128, false, true>), g, dim3(kWave * 4), 0, stream, ms, xs, ys, c, sl, nullptr);
  else
    hipLaunchKernelGGL((ns_update_kernel<64, false, true>), g, dim3(kWave * 2), 0, stream, ms, xs, ys, c, sl, nullptr);
  return launched("Newton-Schulz apply");
}

int qkvnr_proj_forward(const qkvnr_layout* layout, int64_t hidden, const void* x, const void* w_qkv,
                       const int32_t* positions, const void* q_norm_w, const void* k_norm_w, float eps,
                       double theta, void* q, void* k, void* v, hipStream_t stream) {
  if (int rc = check_layout(layout)) return rc;
  const qkvnr_layout* L = layout;
  if (L->kind == QKVNR_LATENT) return fail(QKVNR_EUNSUPPORTED, "the fused projection has no latent kernel");
  if (L->dtype != QKVNR_BF16) return fail(QKVNR_EUNSUPPORTED, "the fused projection is bf16 only");
  if (int rc = check_scalars(L, eps, theta)) return rc;
  if (hidden < kProjBK || hidden % kProjBK || hidden > (1 << 30))
    return fail(QKVNR_EINVAL, "hidden %lld must be a positive multiple of %d, at most 2^30", (long long)hidden,
                kProjBK);
  if (L->width > INT32_MAX) return fail(QKVNR_EINVAL, "width %lld above 2^31", (long long)L->width);
  if (L->T == 0) return QKVNR_OK;  // nothing is read or written
  const bool rope = L->rope_dim > 0;
  if (int rc = need16(x, "x")) return rc;
  if (int rc = need16(w_qkv, "w_qkv")) return rc;
  if (rope) {
    if (int rc = need4(positions, "positions")) return rc;
  }
  if (int rc = need16(q_norm_w, "q_norm_w")) return rc;
  if (int rc = need16(k_norm_w, "k_norm_w")) return rc;
  if (int rc = need16(q, "q")) return rc;
  if (int rc = need16(k, "k")) return rc;
  if (int rc = need16(v, "v")) return rc;
  const int64_t D = L->head_dim, n_q = static_cast<int64_t>(L->n_kv) * L->q_per_kv;
  const int64_t kv_bytes = L->T * L->n_kv * D * 2;
  if (int rc = check_disjoint({{q, L->T * n_q * D * 2}, {k, kv_bytes}, {v, kv_bytes}},
                              {{x, L->T * hidden * 2},
                               {w_qkv, L->width * hidden * 2},
                               {positions, rope ? L->T * 4 : 0},
                               {q_norm_w, D * 2},
                               {k_norm_w, D * 2}}))
    return rc;
  const int64_t tiles_m = (L->T + kProjBM - 1) / kProjBM, tiles_n = (L->width + kProjBN - 1) / kProjBN;
  if (tiles_m * tiles_n > INT32_MAX) return fail(QKVNR_EINVAL, "T %lld: too many tiles for one launch", (long long)L->T);
  int cus = 0;
  if (int rc = current_device(&cus)) return rc;
  ProjArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w_qkv);
  a.pos = positions;
  a.wq = static_cast<const uint16_t*>(q_norm_w);
  a.wk = static_cast<const uint16_t*>(k_norm_w);
  a.q = static_cast<uint16_t*>(q);
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.T = L->T;
  a.hidden = static_cast<int32_t>(hidden);
  a.width = static_cast<int32_t>(L->width);
  a.tiles_n = static_cast<int32_t>(tiles_n);
  a.tiles_m = static_cast<int32_t>(tiles_m);
  a.kind = L->kind == QKVNR_INTERLEAVED ? 0 : 1;
  a.n_kv = L->n_kv;
  a.q_per_kv = L->q_per_kv;
  a.n_q = static_cast<int32_t>(n_q);
  a.heads = static_cast<int32_t>(n_q + 2 * L->n_kv);
  a.eps = eps;
  if (rope) fill_turns(a.turns, theta, L->rope_dim);
  // persistent workgroups, one per CU (each holds 130 KB of LDS), or one per tile when there are fewer
  const dim3 grid(static_cast<uint32_t>(std::min<int64_t>(tiles_m * tiles_n, cus))), block(kProjThreads);
  // the K loop runs in groups of kProjStages steps; a step count that is not a multiple of it takes
  // the variant that skips the products of the steps past the end
  const bool tail = (hidden / kProjBK) % kProjStages != 0;
  if (D == 128) {
    if (rope) launch_proj<128, true>(a, tail, grid, block, stream);
    else launch_proj<128, false>(a, tail, grid, block, stream);
  } else {
    if (rope) launch_proj<64, true>(a, tail, grid, block, stream);
    else launch_proj<64, false>(a, tail, grid, block, stream);
  }
  return launched("fused projection");
}

const char* qkvnr_strerror(int code) {
  switch (code) {
    case QKVNR_OK:
      return "ok";
    case QKVNR_EINVAL:
    case QKVNR_EALIGN:
    case QKVNR_EUNSUPPORTED:
    case QKVNR_EHIP:
      return g_msg[0] ? g_msg : "error";
    default:
      return "unknown qkvnr return code";
  }
}

int qkvnr_version(void) { return QKVNR_VERSION; }

}  // extern "C"
