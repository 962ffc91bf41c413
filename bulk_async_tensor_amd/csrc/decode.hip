// ep_layout_dispatch: layout and dispatch of a small batch in one launch --
// the low-latency shape (tens to hundreds of tokens), where launches, not
// bytes, set the time.  It plays the role of the low-latency kernel family
// that [DeepEP-TMA] lists beside the intranode and internode ones (section
// "TMA Implementation Across Kernel Types"), here on one GPU.
//
// Up to 1024 (token, slot) entries.  Every workgroup (4 waves) reads all the
// ids (at most 4 KiB), builds the expert histogram in LDS, scans it, and
// ranks the entries exactly as ep_layout does: lanes with the same expert
// find each other with one ballot per id bit, rank themselves with mbcnt,
// and per-step group sizes give the rows taken by earlier steps.  The
// destination rows land in LDS; workgroup 0 also writes the layout outputs.
// The workgroup then copies its share of (token, slab) units, reading the
// destinations from LDS.  The result is identical to ep_layout followed by
// ep_dispatch.  Threads share data through LDS only, so the barriers order
// LDS alone and the row loads issued at the start stay in flight across them.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "row_io.hpp"

namespace ep {

namespace {

constexpr int kLdThreads = 256;
constexpr int kLdWaves = kLdThreads / kWave;
constexpr int kLdMaxEntries = 1024;
constexpr int kLdSteps = kLdMaxEntries / kWave;        // 16 steps of 64 entries
constexpr int kLdStepsPerWave = kLdSteps / kLdWaves;   // 4
constexpr int kLdExpertsPerThread = 4;  // 256 threads x 4 = up to 1024 experts
constexpr int kStatusOutOfRange = 1;
constexpr int kStatusDuplicate = 2;

template <int VPL, int K, bool EVEN>
__global__ __launch_bounds__(kLdThreads) void layout_dispatch_kernel(
    const int32_t* __restrict__ idx, int T, int k_rt, int E, int nbits, const u32x4* __restrict__ x,
    u32x4* __restrict__ recv, int64_t recv_rows, int row_vec, int nslab, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;                     // [E]
  int32_t* stepc = cnt + E;               // [16][E] group sizes per step
  int32_t* base = stepc + kLdSteps * E;   // [E] first row of each expert
  int32_t* rows = base + E;               // [1024] destination row of each entry
  int32_t* ids = rows + kLdMaxEntries;    // [1024] the expert ids
  __shared__ int32_t s_wave[kLdWaves + 1];
  __shared__ int32_t s_status;

  const int k = K > 0 ? K : k_rt;
  const int N = T * k;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;

  for (int i = tid; i < (kLdSteps + 1) * E; i += kLdThreads) cnt[i] = 0;
  if (tid == 0) s_status = 0;
  // thread tid holds entries tid + 256 q: step wave + 4 q, lane `lane`
  int e[kLdStepsPerWave];
#pragma unroll
  for (int q = 0; q < kLdStepsPerWave; ++q) {
    const int i = tid + q * kLdThreads;
    e[q] = i < N ? idx[i] : -1;
  }
  // The rows to copy do not depend on the layout: issue the first unit's
  // loads now (after the id loads, so waiting for the ids does not wait for
  // them) and let their latency pass while the layout is computed.
  const int units = T * nslab;
  const int u0 = blockIdx.x * kLdWaves + wave_in_group();
  Unit un0 = unit_of<VPL>(u0 < units ? u0 : 0, nslab, row_vec, lane);
  u32x4 v0[VPL];
  load_slab_fixed<VPL, true>(v0, x + un0.t * row_vec, un0, row_vec);
#pragma unroll
  for (int q = 0; q < kLdStepsPerWave; ++q) ids[tid + q * kLdThreads] = e[q];
  lds_barrier();

  int bad = 0;
#pragma unroll
  for (int q = 0; q < kLdStepsPerWave; ++q) {
    const int i = tid + q * kLdThreads;
    if (i < N) {
      if ((unsigned)e[q] < (unsigned)E) atomicAdd(&cnt[e[q]], 1);
      else bad |= kStatusOutOfRange;
    }
  }
  if (blockIdx.x == 0) {
    for (int t = tid; t < T; t += kLdThreads) {
      const int32_t* r = ids + t * k;
      for (int j = 1; j < k; ++j) {
        const int v = r[j];
        if ((unsigned)v >= (unsigned)E) continue;
        for (int j2 = 0; j2 < j; ++j2)
          if (r[j2] == v) bad |= kStatusDuplicate;
      }
    }
  }
  if (bad) atomicOr(&s_status, bad);
  lds_barrier();

  // offsets: thread tid scans experts [4 tid, 4 tid + 4)
  int own[kLdExpertsPerThread];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kLdExpertsPerThread; ++i) {
    const int ex = tid * kLdExpertsPerThread + i;
    own[i] = ex < E ? cnt[ex] : 0;
    sum += own[i];
  }
  int total = 0;
  int run = block_excl_scan<kLdWaves>(sum, s_wave, &total);
#pragma unroll
  for (int i = 0; i < kLdExpertsPerThread; ++i) {
    const int ex = tid * kLdExpertsPerThread + i;
    if (ex < E) {
      base[ex] = run;
      if (blockIdx.x == 0) {
        counts[ex] = own[i];
        offsets[ex] = run;
      }
    }
    run += own[i];
  }
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = total;
    if (status) status[0] = s_status;
  }

  // ranks inside each 64-entry step
  int rank[kLdStepsPerWave];
  bool ok[kLdStepsPerWave];
#pragma unroll
  for (int q = 0; q < kLdStepsPerWave; ++q) {
    const int i = tid + q * kLdThreads;
    ok[q] = i < N && (unsigned)e[q] < (unsigned)E;
    const uint64_t m = same_value_lanes(ok[q], e[q], nbits);
    rank[q] = mask_rank(m);
    if (ok[q] && (m >> lane) == 1ull) stepc[(wave + q * kLdWaves) * E + e[q]] = __builtin_popcountll(m);
  }
  lds_barrier();
#pragma unroll
  for (int q = 0; q < kLdStepsPerWave; ++q) {
    const int i = tid + q * kLdThreads;
    const int step = wave + q * kLdWaves;
    if (i < N) {
      int r = -1;
      if (ok[q]) {
        r = base[e[q]] + rank[q];
        for (int s2 = 0; s2 < step; ++s2) r += stepc[s2 * E + e[q]];
        if (blockIdx.x == 0 && src_token) src_token[r] = i / k;
      }
      rows[i] = r;
      if (blockIdx.x == 0) dest_row[i] = r;
    }
  }
  lds_barrier();

  // dispatch this workgroup's units (the first one is already loaded)
  for (int u = u0; u < units; u += gridDim.x * kLdWaves) {
    const Unit un = u == u0 ? un0 : unit_of<VPL>(u, nslab, row_vec, lane);
    u32x4 v[VPL];
    if (u == u0) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) v[i] = v0[i];
    } else {
      load_slab<VPL, EVEN, true>(v, x + un.t * row_vec, un, row_vec);
    }
    auto one = [&](int j) {
      const int64_t d = __builtin_amdgcn_readfirstlane(rows[un.t * k + j]);
      if ((uint64_t)d < (uint64_t)recv_rows) store_one<VPL, EVEN, true>(v, recv + d * row_vec, un, row_vec);
    };
    if constexpr (K > 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) one(j);
    } else {
      for (int j = 0; j < k; ++j) one(j);
    }
  }
}

using LdFn = void (*)(const int32_t*, int, int, int, int, const u32x4*, u32x4*, int64_t, int, int, int32_t*,
                      int32_t*, int32_t*, int32_t*, int32_t*);

template <int VPL, bool EVEN>
LdFn ld_pick_k(int k) {
  switch (k) {
    case 2: return layout_dispatch_kernel<VPL, 2, EVEN>;
    case 6: return layout_dispatch_kernel<VPL, 6, EVEN>;
    case 8: return layout_dispatch_kernel<VPL, 8, EVEN>;
    default: return layout_dispatch_kernel<VPL, 0, EVEN>;
  }
}

}  // namespace

bool layout_dispatch_fits(int T, int k, int E) {
  return (int64_t)T * k <= kLdMaxEntries && E <= kLdThreads * kLdExpertsPerThread;
}

hipError_t launch_layout_dispatch(const Budget& b, const int32_t* idx, int T, int k, int E, const void* x, int H,
                                  int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token,
                                  int32_t* status, void* recv, int64_t recv_rows, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int row_vec = H / 8;
  const bool even = row_vec % kWave == 0;
  // 2 KiB slabs: many small units spread a few hundred rows over many CUs
  const int vpl = 2;
  const int nslab = (row_vec + vpl * kWave - 1) / (vpl * kWave);
  const int units = T * nslab;
  int grid = (units + kLdWaves - 1) / kLdWaves;
  int cap = b.num_cus > 0 ? (b.num_cus < b.device_cus ? b.num_cus : b.device_cus) : b.device_cus;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  LdFn fn = even ? ld_pick_k<2, true>(k) : ld_pick_k<2, false>(k);
  const size_t lds = (size_t)((kLdSteps + 2) * E + 2 * kLdMaxEntries) * sizeof(int32_t);
  if (lds > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kLdThreads), lds, stream, idx, T, k, E, nbits,
                     static_cast<const u32x4*>(x), static_cast<u32x4*>(recv), recv_rows, row_vec, nslab, counts,
                     offsets, dest_row, src_token, status);
  return hipGetLastError();
}

}  // namespace ep
