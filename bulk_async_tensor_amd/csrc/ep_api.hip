// C ABI of libep.so: argument validation, the process-wide compute-unit
// budget and variant, per-device attributes, and launches on the caller's
// stream.  Every host-detectable error is reported before any HIP call is
// made, so argument checks run on machines without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <map>
#include <utility>

#include "ep.h"
#include "ep_internal.hpp"

static_assert(EP_MAX_TOPK == ep::kMaxK, "the kernels' largest k is the ABI's");

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_num_cus{-1};  // -1: not read from the environment yet
std::atomic<int> g_variant{static_cast<int>(ep::Variant::Auto)};
std::atomic<int> g_slab{0};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(EP_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int num_cus_setting() {
  int v = g_num_cus.load();
  if (v < 0) {
    const char* env = getenv("EP_NUM_CUS");
    int n = env ? atoi(env) : 0;
    if (n < 0) n = 0;
    int expected = -1;
    g_num_cus.compare_exchange_strong(expected, n);
    v = g_num_cus.load();
  }
  return v;
}

struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int cus = 0;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Compute units a launch on `stream` may use: the stream's CU mask (a
// stream made by ep_stream_create_cu_masked, or any other masked stream)
// narrows b->device_cus, so that grids, persistent budgets and the kernel
// choices that depend on the CU count follow the mask.  A stream whose mask
// cannot be read counts as unmasked; the failed query's error is cleared so
// that the launch checks after it do not see it.
void apply_stream_mask(hipStream_t stream, ep::Budget* b) {
  uint32_t mask[64];
  if (hipExtStreamGetCUMask(stream, 64, mask) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  const int words = (b->all_cus + 31) / 32;
  int n = 0;
  for (int i = 0; i < words && i < 64; ++i) {
    uint32_t m = mask[i];
    const int bits = b->all_cus - 32 * i;
    if (bits < 32) m &= (1u << bits) - 1u;
    n += __builtin_popcount(m);
  }
  if (n > 0 && n < b->device_cus) b->device_cus = n;
}

// Device of the calling thread, checked once: gfx950 and its CU count; then
// the CU count that `stream` may use.
int current_device(ep::Budget* b, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(EP_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.known) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.known = true;
  }
  if (!d.gfx950) return fail(EP_ERR_UNSUPPORTED, "libep is built for gfx950 only");
  b->device_cus = d.cus;
  b->all_cus = d.cus;
  b->num_cus = num_cus_setting();
  b->slab_vpl = g_slab.load();
  apply_stream_mask(static_cast<hipStream_t>(stream), b);
  return EP_OK;
}

int check_common(int T, int k, int H_or_E, const char* what) {
  (void)H_or_E;
  if (T < 0) return fail(EP_ERR_INVALID_ARG, "%s: T = %d < 0", what, T);
  if (k < 1 || k > EP_MAX_TOPK) return fail(EP_ERR_INVALID_ARG, "%s: k = %d outside [1, %d]", what, k, EP_MAX_TOPK);
  if ((int64_t)T * k > EP_MAX_ENTRIES)
    return fail(EP_ERR_INVALID_ARG, "%s: T * k = %lld exceeds EP_MAX_ENTRIES", what, (long long)T * k);
  return EP_OK;
}

// Rows of H elements (T token rows or recv_rows receive rows): their count
// in 512-element slabs, the finest slab a kernel runs, must stay within
// EP_MAX_ENTRIES (unit counters are 32-bit).
int check_slabs(int64_t rows, int H, const char* name, const char* what) {
  const int64_t slabs = rows * ((H + 511) / 512);
  if (slabs > EP_MAX_ENTRIES)
    return fail(EP_ERR_INVALID_ARG, "%s: %s * ceil(H / 512) = %lld exceeds EP_MAX_ENTRIES", what, name,
                (long long)slabs);
  return EP_OK;
}

int check_rows(int H, int64_t recv_rows, int T, const char* what) {
  if (H <= 0 || H % 8 != 0) return fail(EP_ERR_INVALID_ARG, "%s: H = %d must be a positive multiple of 8", what, H);
  if (recv_rows < 0 || recv_rows > EP_MAX_ENTRIES)
    return fail(EP_ERR_INVALID_ARG, "%s: recv_rows = %lld outside [0, EP_MAX_ENTRIES]", what, (long long)recv_rows);
  int rc = check_slabs(recv_rows, H, "recv_rows", what);
  if (rc) return rc;
  return T > 0 ? check_slabs(T, H, "T", what) : EP_OK;
}

// Scratch of ep_layout_noalloc: the (chunk, expert) count table and the
// per-chunk status words of the two- and three-launch layout paths, in a
// static device array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = EP_LAYOUT_NOALLOC_MAX_SCRATCH;
static_assert(kStaticScratchBytes % 256 == 0, "the scratch holds 256-byte aligned tables");
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

int static_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EP_OK;
}

}  // namespace

namespace ep {

// Raises a kernel's dynamic-LDS limit on the current device when a launch
// needs more than was set before; launches within the limit already set only
// look it up.  (The limit cannot simply be set to a CU's whole LDS: a kernel's
// static LDS counts against it.)
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> limit;
  std::lock_guard<std::mutex> lock(mu);
  auto it = limit.find({dev, kernel});
  if (it != limit.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) limit[{dev, kernel}] = bytes;
  return e;
}

}  // namespace ep

extern "C" {

int ep_set_num_cus(int n) {
  if (n < 0 || n > 4096) return fail(EP_ERR_INVALID_ARG, "ep_set_num_cus: n = %d outside [0, 4096]", n);
  g_num_cus.store(n);
  return EP_OK;
}

int ep_get_num_cus(void) { return num_cus_setting(); }

int ep_set_variant(const char* name) {
  if (!name) return fail(EP_ERR_INVALID_ARG, "ep_set_variant: null name");
  static const struct {
    const char* name;
    ep::Variant v;
  } table[] = {{"auto", ep::Variant::Auto}, {"vgpr", ep::Variant::Vgpr}, {"vgpr2", ep::Variant::Vgpr2},
               {"lds1", ep::Variant::Lds1}, {"lds2", ep::Variant::Lds2}, {"vgpr_cached", ep::Variant::VgprCached},
               {"phase", ep::Variant::Phase}, {"lds3", ep::Variant::Lds3}, {"pc", ep::Variant::Pc},
               {"vgpr_wg", ep::Variant::VgprWg}};
  for (const auto& e : table) {
    if (strcmp(e.name, name) == 0) {
      g_variant.store(static_cast<int>(e.v));
      return EP_OK;
    }
  }
  return fail(EP_ERR_UNSUPPORTED, "ep_set_variant: unknown variant '%s'", name);
}

const char* ep_get_variant(void) {
  switch (static_cast<ep::Variant>(g_variant.load())) {
    case ep::Variant::Vgpr: return "vgpr";
    case ep::Variant::Vgpr2: return "vgpr2";
    case ep::Variant::Lds1: return "lds1";
    case ep::Variant::Lds2: return "lds2";
    case ep::Variant::VgprCached: return "vgpr_cached";
    case ep::Variant::Phase: return "phase";
    case ep::Variant::Lds3: return "lds3";
    case ep::Variant::Pc: return "pc";
    case ep::Variant::VgprWg: return "vgpr_wg";
    default: return "auto";
  }
}

int ep_set_slab(int vectors_per_lane) {
  static const int ok[] = {0, 1, 2, 4, 7, 8, 14, 16};
  for (int v : ok) {
    if (v == vectors_per_lane) {
      g_slab.store(v);
      return EP_OK;
    }
  }
  return fail(EP_ERR_UNSUPPORTED, "ep_set_slab: %d is not one of 0, 1, 2, 4, 7, 8, 14, 16", vectors_per_lane);
}

int ep_get_slab(void) { return g_slab.load(); }

size_t ep_layout_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k < 1 || k > EP_MAX_TOPK || E < 1 || E > EP_MAX_EXPERTS) return 0;
  return ep::layout_workspace_bytes(T, k, E);
}

}  // extern "C"

namespace {

// check_workspace = false: the call brings its own scratch (ep_layout_noalloc).
int check_layout_args(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                      int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
                      size_t workspace_bytes, const char* what, bool check_workspace = true) {
  int rc = check_common(T, k, E, what);
  if (rc) return rc;
  if (E < 1 || E > EP_MAX_EXPERTS) return fail(EP_ERR_INVALID_ARG, "%s: E = %d outside [1, %d]", what, E, EP_MAX_EXPERTS);
  if (k > E) return fail(EP_ERR_INVALID_ARG, "%s: k = %d > E = %d", what, k, E);
  if (!counts || !offsets) return fail(EP_ERR_INVALID_ARG, "%s: null counts/offsets", what);
  if (T > 0 && (!topk_idx || !dest_row)) return fail(EP_ERR_INVALID_ARG, "%s: null topk_idx/dest_row", what);
  const void* ptrs[] = {topk_idx, counts, offsets, dest_row, src_token, status};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return fail(EP_ERR_ALIGNMENT, "%s: int32 tensor not 4-byte aligned", what);
  const size_t need = ep::layout_workspace_bytes(T, k, E);
  if (check_workspace && need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(EP_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(EP_ERR_ALIGNMENT, "%s: workspace not 16-byte aligned", what);
  }
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* dest_row,
              int32_t* src_token, int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layout_args(topk_idx, T, k, E, counts, offsets, dest_row, src_token, status, workspace,
                             workspace_bytes, "ep_layout");
  if (rc) return rc;
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_layout(topk_idx, T, k, E, counts, offsets, dest_row, src_token, status, workspace,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_layout launch");
  return EP_OK;
}

int ep_layout_noalloc(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                      int32_t* dest_row, int32_t* src_token, int32_t* status, void* stream) {
  // the same checks as ep_layout, with the static scratch standing in for the workspace
  int rc = check_layout_args(topk_idx, T, k, E, counts, offsets, dest_row, src_token, status, nullptr, 0,
                             "ep_layout_noalloc", false);
  if (rc) return rc;
  const size_t need = ep::layout_workspace_bytes(T, k, E);
  if (need > kStaticScratchBytes)
    return fail(EP_ERR_WORKSPACE,
                "ep_layout_noalloc: T = %d, k = %d, E = %d needs %zu bytes of scratch, above the static %zu; "
                "use ep_layout with a workspace",
                T, k, E, need, kStaticScratchBytes);
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  rc = static_scratch(dev, &ws);
  if (rc) return rc;
  e = ep::launch_layout(topk_idx, T, k, E, counts, offsets, dest_row, src_token, status, ws,
                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_layout_noalloc launch");
  return EP_OK;
}

int ep_dispatch(const void* x, int T, int H, const int32_t* dest_row, int k, void* recv, int64_t recv_rows,
                void* stream) {
  int rc = check_common(T, k, H, "ep_dispatch");
  if (rc) return rc;
  rc = check_rows(H, recv_rows, T, "ep_dispatch");
  if (rc) return rc;
  if (T > 0 && (!x || !dest_row || (!recv && recv_rows > 0)))
    return fail(EP_ERR_INVALID_ARG, "ep_dispatch: null x/dest_row/recv");
  if ((x && !aligned(x, 16)) || (recv && !aligned(recv, 16)))
    return fail(EP_ERR_ALIGNMENT, "ep_dispatch: bf16 tensor not 16-byte aligned");
  if (dest_row && !aligned(dest_row, 4)) return fail(EP_ERR_ALIGNMENT, "ep_dispatch: dest_row not 4-byte aligned");
  if (T == 0 || recv_rows == 0) return EP_OK;
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_dispatch(static_cast<ep::Variant>(g_variant.load()), b, x, T, H, dest_row, k, recv,
                                     recv_rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_dispatch launch");
  return EP_OK;
}

int ep_layout_dispatch(const int32_t* topk_idx, int T, int k, int E, const void* x, int H, int32_t* counts,
                       int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* recv, int64_t recv_rows, void* stream) {
  int rc = check_layout_args(topk_idx, T, k, E, counts, offsets, dest_row, src_token, status, workspace,
                             workspace_bytes, "ep_layout_dispatch");
  if (rc) return rc;
  rc = check_rows(H, recv_rows, T, "ep_layout_dispatch");
  if (rc) return rc;
  if (T > 0 && (!x || (!recv && recv_rows > 0)))
    return fail(EP_ERR_INVALID_ARG, "ep_layout_dispatch: null x/recv");
  if ((x && !aligned(x, 16)) || (recv && !aligned(recv, 16)))
    return fail(EP_ERR_ALIGNMENT, "ep_layout_dispatch: bf16 tensor not 16-byte aligned");
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_layout_dispatch(static_cast<ep::Variant>(g_variant.load()), b, topk_idx, T, k, E, x, H,
                                            counts, offsets, dest_row, src_token, status, workspace, recv, recv_rows,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_layout_dispatch launch");
  return EP_OK;
}

int ep_dispatch_rows(const void* x, int T, int H, const int32_t* src_token, void* recv, int64_t recv_rows,
                     void* stream) {
  if (T < 0) return fail(EP_ERR_INVALID_ARG, "ep_dispatch_rows: T = %d < 0", T);
  int rc = check_rows(H, recv_rows, T, "ep_dispatch_rows");
  if (rc) return rc;
  if (recv_rows > 0 && (!x || !src_token || !recv))
    return fail(EP_ERR_INVALID_ARG, "ep_dispatch_rows: null x/src_token/recv");
  if ((x && !aligned(x, 16)) || (recv && !aligned(recv, 16)))
    return fail(EP_ERR_ALIGNMENT, "ep_dispatch_rows: bf16 tensor not 16-byte aligned");
  if (src_token && !aligned(src_token, 4))
    return fail(EP_ERR_ALIGNMENT, "ep_dispatch_rows: src_token not 4-byte aligned");
  if (T == 0 || recv_rows == 0) return EP_OK;
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_dispatch_rows(static_cast<ep::Variant>(g_variant.load()), b, x, T, H, src_token, recv,
                                          recv_rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_dispatch_rows launch");
  return EP_OK;
}

int ep_combine(const void* y, int64_t recv_rows, int H, const int32_t* dest_row, const float* topk_w, int T, int k,
               void* out, void* stream) {
  int rc = check_common(T, k, H, "ep_combine");
  if (rc) return rc;
  rc = check_rows(H, recv_rows, T, "ep_combine");
  if (rc) return rc;
  if (T > 0 && (!dest_row || !topk_w || !out || (!y && recv_rows > 0)))
    return fail(EP_ERR_INVALID_ARG, "ep_combine: null y/dest_row/topk_w/out");
  if ((y && !aligned(y, 16)) || (out && !aligned(out, 16)))
    return fail(EP_ERR_ALIGNMENT, "ep_combine: bf16 tensor not 16-byte aligned");
  if ((dest_row && !aligned(dest_row, 4)) || (topk_w && !aligned(topk_w, 4)))
    return fail(EP_ERR_ALIGNMENT, "ep_combine: dest_row/topk_w not 4-byte aligned");
  if (T == 0) return EP_OK;
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_combine(static_cast<ep::Variant>(g_variant.load()), b, y, recv_rows, H, dest_row, topk_w,
                                    T, k, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_combine launch");
  return EP_OK;
}

size_t ep_combine_reduce_workspace_bytes(int T, int H) {
  if (T <= 0 || H <= 0 || H % 8 != 0) return 0;
  return ep::combine_reduce_workspace_bytes(T, H);
}

int ep_combine_reduce(const void* y, int64_t recv_rows, int H, const int32_t* src_token, const int32_t* dest_row,
                      const float* topk_w, int T, int k, void* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = check_common(T, k, H, "ep_combine_reduce");
  if (rc) return rc;
  rc = check_rows(H, recv_rows, T, "ep_combine_reduce");
  if (rc) return rc;
  if (T > 0 && (!dest_row || !topk_w || !out || (recv_rows > 0 && (!y || !src_token))))
    return fail(EP_ERR_INVALID_ARG, "ep_combine_reduce: null y/src_token/dest_row/topk_w/out");
  if ((y && !aligned(y, 16)) || (out && !aligned(out, 16)))
    return fail(EP_ERR_ALIGNMENT, "ep_combine_reduce: bf16 tensor not 16-byte aligned");
  if ((src_token && !aligned(src_token, 4)) || (dest_row && !aligned(dest_row, 4)) ||
      (topk_w && !aligned(topk_w, 4)))
    return fail(EP_ERR_ALIGNMENT, "ep_combine_reduce: src_token/dest_row/topk_w not 4-byte aligned");
  if (T == 0) return EP_OK;
  const size_t need = ep::combine_reduce_workspace_bytes(T, H);
  if (!workspace || workspace_bytes < need)
    return fail(EP_ERR_WORKSPACE, "ep_combine_reduce: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(EP_ERR_ALIGNMENT, "ep_combine_reduce: workspace not 16-byte aligned");
  ep::Budget b;
  rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_combine_reduce(b, y, recv_rows, H, src_token, dest_row, topk_w, T, k, out, workspace,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_combine_reduce launch");
  return EP_OK;
}

const char* ep_status_string(int code) {
  switch (code) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_ALIGNMENT: return "misaligned pointer";
    case EP_ERR_UNSUPPORTED: return "unsupported device or variant";
    case EP_ERR_WORKSPACE: return "workspace missing or too small";
    case EP_ERR_HIP: return "HIP runtime error";
    default: return "unknown code";
  }
}

const char* ep_last_error(void) { return g_err; }

int ep_bw_probe(int mode, const void* src, void* dst, int64_t bytes, void* stream) {
  if (mode < 0 || (mode & ~0x737) != 0 || ((mode >> 4) & 3) == 3 || ((mode >> 8) & 7) > 5)
    return fail(EP_ERR_INVALID_ARG, "ep_bw_probe: mode 0x%x", mode);
  const int op = mode & 7;
  if (op >= 4 && bytes % (op == 7 ? 131072 : op == 6 ? 65536 : 8192) != 0)
    return fail(EP_ERR_INVALID_ARG,
                "ep_bw_probe: mixed operations need bytes in multiples of 8 KiB (64 KiB for 6, 128 KiB for 7)");
  if (bytes < 0 || bytes % 16) return fail(EP_ERR_INVALID_ARG, "ep_bw_probe: bytes must be a multiple of 16");
  if (((mode & 7) != 2 && !src) || !dst) return fail(EP_ERR_INVALID_ARG, "ep_bw_probe: null pointer");
  if (((mode & 7) == 1 || (mode & 7) == 3) && bytes > ((int64_t)1 << 40))
    return fail(EP_ERR_INVALID_ARG, "ep_bw_probe: size");
  if ((src && !aligned(src, 16)) || !aligned(dst, 16)) return fail(EP_ERR_ALIGNMENT, "ep_bw_probe: alignment");
  if (bytes == 0) return EP_OK;
  ep::Budget b;
  int rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_bw_probe(b, mode, src, dst, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_bw_probe launch");
  return EP_OK;
}

int ep_inflight_probe(int waves_per_cu, int vectors_per_lane, int cached, const void* src, int64_t bytes, void* sink,
                      const int64_t* chain, int64_t chain_len, int64_t hops, int64_t* out, void* stream) {
  if (cached != 0 && cached != 1) return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: cached = %d not 0 or 1", cached);
  if (waves_per_cu < 1 || waves_per_cu > 16)
    return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: waves_per_cu = %d outside [1, 16]", waves_per_cu);
  if (vectors_per_lane != 1 && vectors_per_lane != 2 && vectors_per_lane != 4 && vectors_per_lane != 8 &&
      vectors_per_lane != 16)
    return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: vectors_per_lane = %d not 1, 2, 4, 8 or 16",
                vectors_per_lane);
  if (vectors_per_lane == 16 && waves_per_cu > 8)
    return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: 16 vectors per lane allow at most 8 waves per CU");
  if (bytes < 0 || bytes % 16) return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: bytes must be a multiple of 16");
  if (hops < 0 || chain_len < 0) return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: negative hops or chain_len");
  if (!sink || (bytes > 0 && !src)) return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: null src/sink");
  if (hops > 0 && (!chain || !out || chain_len < 1))
    return fail(EP_ERR_INVALID_ARG, "ep_inflight_probe: a chase needs chain, chain_len >= 1 and out");
  if ((src && !aligned(src, 16)) || !aligned(sink, 16) || (chain && !aligned(chain, 8)) || (out && !aligned(out, 8)))
    return fail(EP_ERR_ALIGNMENT, "ep_inflight_probe: alignment");
  ep::Budget b;
  int rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_inflight_probe(b, waves_per_cu, vectors_per_lane, cached, src, bytes, sink, chain,
                                           chain_len, hops, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_inflight_probe launch");
  return EP_OK;
}

int ep_probe_placement(int32_t* out, int n_groups, void* stream) {
  if (!out || n_groups < 1 || n_groups > 65536)
    return fail(EP_ERR_INVALID_ARG, "ep_probe_placement: bad output or n_groups");
  if (!aligned(out, 4)) return fail(EP_ERR_ALIGNMENT, "ep_probe_placement: alignment");
  ep::Budget b;
  int rc = current_device(&b, stream);
  if (rc) return rc;
  int launched = 0;
  hipError_t e = ep::launch_placement(b, n_groups, out, static_cast<hipStream_t>(stream), &launched);
  if (e != hipSuccess) return hip_fail(e, "ep_probe_placement launch");
  return launched;
}

int ep_mfma_probe(int n_groups, int iters, float* out, void* stream) {
  if (!out || n_groups < 1 || n_groups > 65536 || iters < 0)
    return fail(EP_ERR_INVALID_ARG, "ep_mfma_probe: bad output, n_groups or iters");
  if (!aligned(out, 4)) return fail(EP_ERR_ALIGNMENT, "ep_mfma_probe: alignment");
  ep::Budget b;
  int rc = current_device(&b, stream);
  if (rc) return rc;
  hipError_t e = ep::launch_mfma_probe(n_groups, iters, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ep_mfma_probe launch");
  return EP_OK;
}

int ep_stream_create_cu_masked(const uint32_t* mask, int mask_words, void** stream) {
  if (!mask || !stream) return fail(EP_ERR_INVALID_ARG, "ep_stream_create_cu_masked: null pointer");
  if (mask_words < 1 || mask_words > 64)
    return fail(EP_ERR_INVALID_ARG, "ep_stream_create_cu_masked: mask_words = %d outside [1, 64]", mask_words);
  uint32_t any = 0;
  for (int i = 0; i < mask_words; ++i) any |= mask[i];
  if (!any) return fail(EP_ERR_INVALID_ARG, "ep_stream_create_cu_masked: empty mask");
  // The runtime numbers CUs round-robin over the XCDs (bit i selects a CU of
  // XCD i mod the XCD count; measured on MI355X with the placement probe),
  // and a masked stream's queue runs on every XCD: a mask that leaves an XCD
  // without a CU is refused, with an error that the next HIP call would
  // also report.  Check it here first.
  int dev = 0, cus = 0, xccs = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && xccs > 1 && cus > 0) {
    for (int x = 0; x < xccs; ++x) {
      bool has = false;
      for (int i = x; i < cus && i < 32 * mask_words && !has; i += xccs) has = (mask[i / 32] >> (i % 32)) & 1u;
      if (!has)
        return fail(EP_ERR_INVALID_ARG,
                    "ep_stream_create_cu_masked: no CU of XCD %d in the mask (bit i selects a CU of XCD i mod %d; "
                    "every XCD needs one)",
                    x, xccs);
    }
  } else {
    (void)hipGetLastError();
  }
  hipStream_t s = nullptr;
  hipError_t e = hipExtStreamCreateWithCUMask(&s, (uint32_t)mask_words, mask);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the refusal for the next HIP call to report
    return hip_fail(e, "hipExtStreamCreateWithCUMask");
  }
  *stream = s;
  return EP_OK;
}

int ep_stream_destroy(void* stream) {
  if (!stream) return fail(EP_ERR_INVALID_ARG, "ep_stream_destroy: null stream");
  hipError_t e = hipStreamDestroy(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamDestroy");
  return EP_OK;
}

}  // extern "C"
