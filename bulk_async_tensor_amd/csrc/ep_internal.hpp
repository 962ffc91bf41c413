// Host-side interfaces between the C ABI (ep_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

enum class Variant : int {
  Auto = 0,
  Vgpr = 1,
  Vgpr2 = 2,
  Lds1 = 3,
  Lds2 = 4,
  VgprCached = 5,
  Phase = 6,
  Lds3 = 7,
  Pc = 8,
  VgprWg = 9
};

// Launch geometry chosen by the host for the row-movement kernels.
struct Budget {
  int num_cus;     // > 0: persistent grid of this many workgroups, one per CU
  int device_cus;  // compute units the launch may use: the device's, or fewer on a CU-masked stream
  int all_cus;     // compute units of the current device
  int slab_vpl;    // 16-byte vectors per lane per row slab (0: the kernel's default)
};

// One CU holds 160 KiB of LDS; a workgroup that asks for more than half of it
// can never share a CU with another one.
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr size_t kExclusiveLds = 80 * 1024 + 1024;

// A large dispatch runs as a persistent grid on this many CUs when no budget
// is set: at k = 8 its traffic is 8/9 writes, and HBM write throughput was
// measured highest with about a quarter of the CUs issuing them.
constexpr int kWriteCus = 64;

// The default persistent budget by k.  The share of reads grows as k falls
// (1/(1+k) of the bytes), and reads need more CUs in flight to hide their
// latency: measured at H = 7168, 64 CUs stay best for k >= 5, 96 for
// k = 2..4 (k = 2: 7.0 against 5.7 TB/s on 64) and 128 for k = 1.
inline int dispatch_write_cus(int k) { return k >= 5 ? kWriteCus : k >= 2 ? 96 : 128; }

// Largest k the kernels accept (the ABI's EP_MAX_TOPK).
constexpr int kMaxK = 32;

// ---- layout (layout.hip)
int layout_chunk_tokens(int k);
int layout_num_chunks(int T, int k);
size_t layout_workspace_bytes(int T, int k, int E);
hipError_t launch_layout(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                         int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
                         hipStream_t stream);

// ---- dispatch (dispatch.hip)
hipError_t launch_dispatch(Variant v, const Budget& b, const void* x, int T, int H, const int32_t* dest_row,
                           int k, void* recv, int64_t recv_rows, hipStream_t stream);

hipError_t launch_dispatch_rows(Variant v, const Budget& b, const void* x, int T, int H, const int32_t* src_token,
                                void* recv, int64_t recv_rows, hipStream_t stream);

// Vectors per lane of the default dispatch slab for a row of row_vec 16-byte
// vectors, at most `cap` (a requested size is rounded down to a compiled one).
int dispatch_slab_vpl(int row_vec, int cap, int requested);

// The workgroup-phased register dispatch (vgpr_wg) runs workgroups of
// kWgWaves waves; each wave holds wg_units_of(vpl) units of vpl vectors per
// lane between its loads and its stores (at most 224 VGPRs of row data).
constexpr int kWgWaves = 4;
constexpr int wg_units_of(int vpl) { return vpl > 14 ? 2 : 4; }

// ---- its whole-row kernel (dispatch_rows.hip): rows of row_vec vectors,
// at most 16 per lane (a partial last KiB allowed), k = 1 .. 8; nullptr
// otherwise.  launch_wg_rows runs it on `grid` workgroups of `wpg` waves.
const void* wg_rows_kernel(int row_vec, int k);
hipError_t launch_wg_rows(const void* kernel, int grid, int wpg, size_t lds_bytes, hipStream_t stream, const void* x,
                          void* recv, const int32_t* dest_row, int64_t recv_rows, int T, int trips, int row_vec);

// True when variant "auto" dispatches T tokens with its large-batch kernels
// (at least 8 tokens per CU of the launch), which stream x instead of
// staging it through cacheable direct-to-LDS loads.
bool dispatch_auto_large(const Budget& b, int64_t T);

// ---- fused layout + dispatch (layout_dispatch.hip)
// One launch for small batches and, with the lds1-style copy, for wide ones;
// otherwise launch_layout then launch_dispatch (workspace as for the layout).
hipError_t launch_layout_dispatch(Variant v, const Budget& b, const int32_t* idx, int T, int k, int E, const void* x,
                                  int H, int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token,
                                  int32_t* status, void* workspace, void* recv, int64_t recv_rows,
                                  hipStream_t stream);

// ---- combine (combine.hip)
hipError_t launch_combine(Variant v, const Budget& b, const void* y, int64_t recv_rows, int H,
                          const int32_t* dest_row, const float* w, int T, int k, void* out, hipStream_t stream);

// ---- reduce-on-store combine (combine_reduce.hip)
size_t combine_reduce_workspace_bytes(int T, int H);
hipError_t launch_combine_reduce(const Budget& b, const void* y, int64_t recv_rows, int H, const int32_t* src_token,
                                 const int32_t* dest_row, const float* w, int T, int k, void* out, void* acc,
                                 hipStream_t stream);

// ---- probes (probe.hip)
hipError_t launch_bw_probe(const Budget& b, int mode, const void* src, void* dst, int64_t bytes,
                           hipStream_t stream);
hipError_t launch_placement(const Budget& b, int n_groups, int32_t* out, hipStream_t stream, int* launched);
hipError_t launch_inflight_probe(const Budget& b, int waves_per_cu, int vec_per_lane, int cached, const void* src,
                                 int64_t bytes, void* sink, const int64_t* chain, int64_t chain_len, int64_t hops,
                                 int64_t* out, hipStream_t stream);
hipError_t launch_mfma_probe(int n_groups, int iters, float* out, hipStream_t stream);

// Raise the dynamic-LDS limit of a kernel once (needed above 64 KiB).
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes);

}  // namespace ep
