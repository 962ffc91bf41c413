// ep_layout_dispatch: layout and dispatch in one launch, so that the
// layout's own launch and the gap before the copy disappear.  It plays the
// role of the low-latency kernel family that [DeepEP-TMA] lists beside the
// intranode and internode ones (section "TMA Implementation Across Kernel
// Types"), here on one GPU, and serves wide batches as well.  The result is
// identical to ep_layout followed by ep_dispatch.
//
// Small batches (up to 1024 (token, slot) entries) that the wide kernel
// does not take (few experts, other k, another dispatch variant): every
// workgroup (4 waves) reads all the ids (at most 4 KiB), builds the expert
// histogram in LDS, scans it, and ranks the entries exactly as ep_layout
// does: lanes with the same expert find each other with one ballot per id
// bit, rank themselves with mbcnt, and per-step group sizes give the rows
// taken by earlier steps.  The destination rows land in LDS; workgroup 0
// also writes the layout outputs.  The workgroup then copies its share of
// (token, slab) units, reading the destinations from LDS.
//
// Batches of up to 64 Ki entries with 65 to 256 experts and k in
// {2, 4, 6, 8}, decode batches included: a persistent grid (one workgroup
// of 16 waves per CU: the budget, or 64 CUs for large batches and 128 below
// that) in which workgroup g owns a contiguous range of tokens.  Each
// workgroup histograms all T*k ids into two LDS histograms, the tokens
// before its range and the rest, so that it knows every expert's total
// (hence the offsets) and the rows that earlier workgroups take,
// without any communication between workgroups.  It then ranks only its own
// entries, writes their dest_row and src_token, and copies its own rows
// through per-wave LDS slices filled by direct-to-LDS loads, as the lds1
// dispatch does.  The first slab of every wave is requested before the
// histogram, so its load overlaps the layout work.
//
// Threads share data through LDS only, so the barriers order LDS alone and
// the row loads issued at the start stay in flight across them.
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
    // repeated expert inside one token: every entry against the earlier
    // entries of its token, entries spread over all threads
    for (int i = tid; i < N; i += kLdThreads) {
      const int v = ids[i];
      if ((unsigned)v >= (unsigned)E) continue;
      for (int i2 = i - i % k; i2 < i; ++i2)
        if (ids[i2] == v) bad |= kStatusDuplicate;
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

// k known at compile time up to 8: against the run-time-k form, E = 64,
// H = 7168, T = 32 .. 170, cold, 1-11% faster (k = 4, T = 170: 10.8 against
// 12.1 us), bit-identical.
template <int VPL, bool EVEN>
LdFn ld_pick_k(int k) {
  switch (k) {
    case 1: return layout_dispatch_kernel<VPL, 1, EVEN>;
    case 2: return layout_dispatch_kernel<VPL, 2, EVEN>;
    case 3: return layout_dispatch_kernel<VPL, 3, EVEN>;
    case 4: return layout_dispatch_kernel<VPL, 4, EVEN>;
    case 5: return layout_dispatch_kernel<VPL, 5, EVEN>;
    case 6: return layout_dispatch_kernel<VPL, 6, EVEN>;
    case 7: return layout_dispatch_kernel<VPL, 7, EVEN>;
    case 8: return layout_dispatch_kernel<VPL, 8, EVEN>;
    default: return layout_dispatch_kernel<VPL, 0, EVEN>;
  }
}


// ---- wide batches
constexpr int kWdThreads = 1024;
constexpr int kWdWaves = kWdThreads / kWave;
// Expert range and batch size of the wide path, from measurements on the
// training shape family (E = 256, k = 8): one launch saves 5.9 us against
// the layout launch followed by the dispatch at T = 4096 and 6.9 us at
// T = 8192.  Every workgroup histograms all T*k ids at about 3 LDS atomics
// per clock, so past 64 Ki ids the separate layout launch is cheaper.  With
// E <= 64 (and skewed routing) the lanes of an atomic collide on a few
// addresses: the prefill shape ran 56 us slower fused, so such batches take
// the separate launches, as the layout does.
constexpr int kWdMinExperts = 65;
constexpr int kWdMaxExperts = 256;   // group sizes per step: 16 x E ints of LDS
#ifndef EP_LAYOUT_DISPATCH_WIDE_MAX_ENTRIES
#define EP_LAYOUT_DISPATCH_WIDE_MAX_ENTRIES (64 * 1024)
#endif

// Reads the k ids of token t and adds them to the histogram cnt2 (tokens
// before the workgroup's range count in cnt2[e], the others in cnt2[E + e]).
// The k loads are unconditional and contiguous, so they go out as a few wide
// loads; each id is one LDS atomic.  (Aggregating equal ids of a wave first,
// as the layout's count kernel does, measured 5x slower here with uniform
// routing over 256 experts, and skewed routing over few experts is left to
// the separate layout launch.)
template <int K>
__device__ __forceinline__ void wide_count(const int32_t* __restrict__ idx, int t, int t0, int E, bool check_dups,
                                           int32_t* cnt2, int& bad) {
  int e[K];
#pragma unroll
  for (int j = 0; j < K; ++j) e[j] = idx[(int64_t)t * K + j];
  const int side = t < t0 ? 0 : E;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if ((unsigned)e[j] < (unsigned)E) {
      atomicAdd(&cnt2[side + e[j]], 1);
      if (check_dups) {
#pragma unroll
        for (int j2 = 0; j2 < j; ++j2)
          if (e[j2] == e[j]) bad |= kStatusDuplicate;
      }
    } else {
      bad |= kStatusOutOfRange;
    }
  }
}

template <int VPL, int K, bool EVEN>
__global__ __launch_bounds__(kWdThreads) void layout_dispatch_wide_kernel(
    const int32_t* __restrict__ idx, int T, int E, int nbits, int tpg, const u32x4* __restrict__ x,
    u32x4* __restrict__ recv, int64_t recv_rows, int row_vec, int nslab, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
    int32_t* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) char wd_lds[];
  // [16 slices of VPL KiB][cnt2: 2E][base: E][stepc: 16 x E][rows: tpg x K]
  int32_t* cnt2 = reinterpret_cast<int32_t*>(wd_lds + kWdWaves * VPL * kWaveVecBytes);
  int32_t* base = cnt2 + 2 * E;
  int32_t* stepc = base + E;
  int32_t* rows = stepc + kWdWaves * E;
  __shared__ int32_t s_wave[kWdWaves + 1];
  __shared__ int32_t s_status;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_in_group();
  const int t0 = blockIdx.x * tpg;
  const int nt = min(tpg, T - t0);  // >= 1: the host sizes the grid so
  const int n = nt * K;
  const int units = nt * nslab;
  char* slice = wd_lds + wave * (VPL * kWaveVecBytes);

  // this wave's first slab: its load runs while the layout is computed
  if (wave < units) {
    Unit un = unit_of<VPL>(wave, nslab, row_vec, lane);
    un.t += t0;
    dma_slab<VPL, EVEN>(x + un.t * row_vec, slice, un, row_vec);
  }
  for (int i = tid; i < (3 + kWdWaves) * E; i += kWdThreads) cnt2[i] = 0;
  if (tid == 0) s_status = 0;
  lds_barrier();

  // Histogram of all tokens, thread per token, two tokens per trip.  Only
  // workgroup 0 reports the status, so only it looks for repeated experts.
  int bad = 0;
  const bool dups = blockIdx.x == 0;
  for (int t = tid; t < T; t += 2 * kWdThreads) {
    wide_count<K>(idx, t, t0, E, dups, cnt2, bad);
    if (t + kWdThreads < T) wide_count<K>(idx, t + kWdThreads, t0, E, dups, cnt2, bad);
  }
  if (bad) atomicOr(&s_status, bad);
  lds_barrier();

  // offsets (thread e holds expert e), and the first row of each expert that
  // this workgroup's entries take
  const int before = tid < E ? cnt2[tid] : 0;
  const int tot = tid < E ? before + cnt2[E + tid] : 0;
  int all = 0;
  const int excl = block_excl_scan<kWdWaves>(tot, s_wave, &all);
  if (tid < E) base[tid] = excl + before;
  if (blockIdx.x == 0) {
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = excl;
    }
    if (tid == 0) {
      offsets[E] = all;
      if (status) status[0] = s_status;
    }
  }
  lds_barrier();

  // Own entries, 1024 per round (one 64-entry step per wave).  After a
  // round, each expert's first row moves past the rows the round took.
  const int64_t i0 = (int64_t)t0 * K;
  for (int r0 = 0; r0 < n; r0 += kWdThreads) {
    const int i = r0 + tid;
    const bool in_range = i < n;
    const int e = in_range ? idx[i0 + i] : -1;
    const bool ok = in_range && (unsigned)e < (unsigned)E;
    const uint64_t m = same_value_lanes(ok, e, nbits);
    const int rank = mask_rank(m);
    if (ok && (m >> lane) == 1ull) stepc[wave * E + e] = __builtin_popcountll(m);
    lds_barrier();
    if (in_range) {
      int r = -1;
      if (ok) {
        r = base[e] + rank;
        for (int w = 0; w < wave; ++w) r += stepc[w * E + e];
        if (src_token) src_token[r] = t0 + i / K;
      }
      rows[i] = r;
      dest_row[i0 + i] = r;
    }
    lds_barrier();
    if (r0 + kWdThreads < n) {
      for (int ex = tid; ex < E; ex += kWdThreads) {
        int sum = 0;
        for (int w = 0; w < kWdWaves; ++w) {
          sum += stepc[w * E + ex];
          stepc[w * E + ex] = 0;
        }
        base[ex] += sum;
      }
      lds_barrier();
    }
  }

  // copy this workgroup's rows: wave w takes units w, w + 16, ...
  for (int u = wave; u < units; u += kWdWaves) {
    Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    const int tl = (int)un.t;
    un.t += t0;
    int32_t d[K];
#pragma unroll
    for (int j = 0; j < K; ++j) d[j] = __builtin_amdgcn_readfirstlane(rows[tl * K + j]);
    if (u != wave) dma_slab<VPL, EVEN>(x + un.t * row_vec, slice, un, row_vec);
    wait_vmcnt<0>();  // slice filled (this also drains the previous unit's stores)
    u32x4 v[VPL];
    read_slab<VPL>(v, slice, lane);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t dj = d[j];
      if ((uint64_t)dj < (uint64_t)recv_rows) store_one<VPL, EVEN, true>(v, recv + dj * row_vec, un, row_vec);
    }
  }
}

using WideFn = void (*)(const int32_t*, int, int, int, int, const u32x4*, u32x4*, int64_t, int, int, int32_t*,
                        int32_t*, int32_t*, int32_t*, int32_t*);

template <int VPL, int K>
WideFn wide_pick_even(bool even) {
  return even ? layout_dispatch_wide_kernel<VPL, K, true> : layout_dispatch_wide_kernel<VPL, K, false>;
}

// Odd k against the small kernel or the two calls it used before, E = 256,
// H = 7168, cold: T = 128 8.5-10.5 against 8.9-12.8 us, T = 512 11.2-18.6
// against 13.7-19.5 us; bit-identical.
template <int VPL>
WideFn wide_pick_k(int k, bool even) {
  switch (k) {
    case 1: return wide_pick_even<VPL, 1>(even);
    case 2: return wide_pick_even<VPL, 2>(even);
    case 3: return wide_pick_even<VPL, 3>(even);
    case 4: return wide_pick_even<VPL, 4>(even);
    case 5: return wide_pick_even<VPL, 5>(even);
    case 6: return wide_pick_even<VPL, 6>(even);
    case 7: return wide_pick_even<VPL, 7>(even);
    case 8: return wide_pick_even<VPL, 8>(even);
    default: return nullptr;
  }
}

WideFn wide_pick(int vpl, int k, bool even) {
  switch (vpl) {
    case 2: return wide_pick_k<2>(k, even);
    case 4: return wide_pick_k<4>(k, even);
    case 7: return wide_pick_k<7>(k, even);
    case 8: return wide_pick_k<8>(k, even);
    default: return nullptr;
  }
}

}  // namespace

namespace {

bool small_fits(int T, int k, int E) {
  return (int64_t)T * k <= kLdMaxEntries && E <= kLdThreads * kLdExpertsPerThread;
}

hipError_t launch_small(const Budget& b, const int32_t* idx, int T, int k, int E, int nbits, const void* x, int H,
                        int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* status,
                        void* recv, int64_t recv_rows, hipStream_t stream) {
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

// Launch geometry of the wide kernel, or ok = false where it does not apply:
// k above 8, E outside [kWdMinExperts, kWdMaxExperts],
// more ids than a workgroup histograms faster than the separate layout
// launch, or LDS beyond a CU's.
struct WidePlan {
  bool ok = false;
  int grid = 0, tpg = 0, vpl = 0, nslab = 0;
  size_t lds = 0;
};

WidePlan wide_plan(const Budget& b, int T, int k, int E, int H) {
  WidePlan p;
  if (k < 1 || k > 8 || E < kWdMinExperts || E > kWdMaxExperts) return p;
  if ((int64_t)T * k > EP_LAYOUT_DISPATCH_WIDE_MAX_ENTRIES) return p;
  const int row_vec = H / 8;
  p.vpl = dispatch_slab_vpl(row_vec, 8, b.slab_vpl);
  p.nslab = (row_vec + p.vpl * kWave - 1) / (p.vpl * kWave);
  // With no budget: the dispatch's CUs for large batches (64 at k >= 6,
  // whose traffic is mostly writes, which peak there; 96 at k = 2 and 4);
  // smaller batches spread over 128 CUs, where a copy phase of a few
  // microseconds gains from more CUs (T = 128 at H = 7168: 7.2 against
  // 8.4 us on 64 CUs; T = 1024: 27.1 against 28.0 us).
  const int64_t units = (int64_t)T * p.nslab;
  const int write_cus = dispatch_write_cus(k);
  int cus = b.num_cus > 0 ? b.num_cus : (units >= (int64_t)write_cus * 16 * 4 ? write_cus : 2 * kWriteCus);
  if (cus > b.device_cus) cus = b.device_cus;
  p.tpg = (T + cus - 1) / cus;
  p.grid = (T + p.tpg - 1) / p.tpg;  // every workgroup owns at least one token
  p.lds = (size_t)kWdWaves * p.vpl * kWaveVecBytes + (size_t)((3 + kWdWaves) * E + p.tpg * k) * sizeof(int32_t);
  if (p.lds < kExclusiveLds) p.lds = kExclusiveLds;  // one workgroup per CU
  // the kernel's static LDS (s_wave, s_status) is well under 1 KiB
  if (p.lds + 1024 > kLdsPerCu) return p;
  p.ok = true;
  return p;
}

hipError_t launch_wide(const WidePlan& p, const int32_t* idx, int T, int k, int E, int nbits, const void* x, int H,
                       int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* status,
                       void* recv, int64_t recv_rows, hipStream_t stream) {
  const int row_vec = H / 8;
  const bool even = row_vec % kWave == 0;
  WideFn fn = wide_pick(p.vpl, k, even);
  if (!fn) return hipErrorInvalidValue;
  hipError_t e = allow_dynamic_lds((const void*)fn, p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(p.grid), dim3(kWdThreads), p.lds, stream, idx, T, E, nbits, p.tpg,
                     static_cast<const u32x4*>(x), static_cast<u32x4*>(recv), recv_rows, row_vec, p.nslab, counts,
                     offsets, dest_row, src_token, status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layout_dispatch(Variant v, const Budget& b, const int32_t* idx, int T, int k, int E, const void* x,
                                  int H, int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token,
                                  int32_t* status, void* workspace, void* recv, int64_t recv_rows,
                                  hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // The wide kernel copies as the lds1 dispatch does: taken for "lds1", and
  // for "auto" below the batch size from which the default dispatch runs
  // the workgroup-phased kernel (its cacheable loads of x are fast only
  // while x is cached).  It is
  // also the faster one for decode batches where it applies (T = 128,
  // E = 256, k = 8: 8.1 against 8.7 us for the small kernel; T = 64: 6.5
  // against 7.6 us), so the small kernel serves the rest: few experts,
  // other k, other variants.
  if (T > 0 && (v == Variant::Lds1 || (v == Variant::Auto && !dispatch_auto_large(b, T)))) {
    const WidePlan p = wide_plan(b, T, k, E, H);
    if (p.ok)
      return launch_wide(p, idx, T, k, E, nbits, x, H, counts, offsets, dest_row, src_token, status, recv,
                         recv_rows, stream);
  }
  if (T > 0 && small_fits(T, k, E))
    return launch_small(b, idx, T, k, E, nbits, x, H, counts, offsets, dest_row, src_token, status, recv, recv_rows,
                        stream);
  hipError_t e = launch_layout(idx, T, k, E, counts, offsets, dest_row, src_token, status, workspace, stream);
  if (e == hipSuccess && T > 0 && recv_rows > 0)
    e = launch_dispatch(v, b, x, T, H, dest_row, k, recv, recv_rows, stream);
  return e;
}

}  // namespace ep
