// Measurement kernels under the same compute-unit budget as dispatch and
// combine: a streaming copy / read / write that gives the HBM ceiling a
// given number of CUs can reach, and a placement probe that reports which
// XCD, shader engine and CU each workgroup of the persistent grid ran on.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

namespace {

// Probe parameters packed in `mode`: bits [1:0] operation (0 copy, 1 read,
// 2 write, 3 read into LDS by direct-to-LDS loads), bits [5:4] depth (16-byte
// vectors in flight per lane: 8, 16 or 32), bits [10:8] cache policy of the
// loads (0 nt, 1 none, 2 sc0, 3 sc1, 4 sc0+sc1, 5 nt through a buffer load).
constexpr int kPolicyAux[6] = {2, 0, 1, 16, 17, 2};  // gfx940-family CPol bits: sc0 = 1, nt = 2, sc1 = 16

template <int POL>
__device__ __forceinline__ u32x4 probe_load(const u32x4* __restrict__ src, __amdgpu_buffer_rsrc_t rsrc, int64_t c,
                                            int64_t win_base) {
  if constexpr (POL == 0) {
    return ld16<true>(src + c);
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)((c - win_base) * 16), 0, kPolicyAux[POL]);
    return __builtin_bit_cast(u32x4, v);
  }
}

template <int OP, int D, int POL>
__global__ __launch_bounds__(1024) void bw_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                  int64_t nvec) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int64_t wpg = blockDim.x >> 6;
  const int64_t chunk = (int64_t)D * kWave;
  const int64_t stride = (int64_t)gridDim.x * wpg * chunk;
  u32x4 sum = {0u, 0u, 0u, 0u};
  // buffer loads address a window of at most 2 GiB at a time
  constexpr int64_t kWin = (int64_t)1 << 27;  // vectors
  int64_t win_base = -1;
  __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, 0x7FFFFFFF, 0x00020000);
  char* slice = lds + wave * (D * kWaveVecBytes);
  for (int64_t base = ((int64_t)blockIdx.x * wpg + wave) * chunk; base < nvec; base += stride) {
    if constexpr (POL != 0) {
      const int64_t wb = base & ~(kWin - 1);
      if (wb != win_base) {
        win_base = wb;
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(src + wb), 0, 0x7FFFFFFF, 0x00020000);
      }
    }
    if constexpr (OP == 3) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int64_t c = base + i * kWave + lane;
        if (c < nvec) __builtin_amdgcn_global_load_lds(src + c, (lds_void_t*)(slice + i * kWaveVecBytes), 16, 0,
                                                       kPolicyAux[POL]);
      }
      wait_vmcnt<0>();
      u32x4 v;
      lds_read16_async(v, lds_addr_of(slice) + lane * kVecBytes);
      lds_wait_all();
      lds_fence_value(v);
      sum ^= v;
    } else {
      u32x4 v[D];
      if constexpr (OP != 2) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int64_t c = base + i * kWave + lane;
          if (c < nvec) v[i] = probe_load<POL>(src, rsrc, c, win_base < 0 ? 0 : win_base);
        }
      }
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int64_t c = base + i * kWave + lane;
        if (c < nvec) {
          if constexpr (OP == 0) st16<true>(dst + c, v[i]);
          else if constexpr (OP == 1) sum ^= v[i];
          else st16<true>(dst + c, u32x4{(uint32_t)c, 0x5a5a5a5au, (uint32_t)(c >> 32), 0xa5a5a5a5u});
        }
      }
    }
  }
  // keeps the reads alive; true only for a vanishingly unlikely checksum
  if ((OP == 1 || OP == 3) && sum[0] == 0x9e3779b9u && sum[1] == 0x7f4a7c15u && sum[2] == 0x94d049bbu) dst[0] = sum;
}

// Mixed-ratio streams.  DIR 0 (8:1, the combine mix): a wave reads 8 KiB
// contiguous and writes 1 KiB.  DIR 1 (1:8, the dispatch mix): a wave reads
// 1 KiB and writes 8 KiB contiguous.  nvec counts the larger side (multiple
// of 512 vectors).
template <int DIR>
__global__ __launch_bounds__(1024) void bw_mix_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                      int64_t nvec) {
  const int lane = lane_id();
  const int64_t wpg = blockDim.x >> 6;
  const int64_t nchunk = nvec / (8 * kWave);
  for (int64_t q = (int64_t)blockIdx.x * wpg + wave_in_group(); q < nchunk; q += (int64_t)gridDim.x * wpg) {
    if constexpr (DIR == 0) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ld16<true>(src + q * 8 * kWave + i * kWave + lane);
      u32x4 x = v[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) x ^= v[i];
      st16<true>(dst + q * kWave + lane, x);
    } else {
      const u32x4 v = ld16<true>(src + q * kWave + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) st16<true>(dst + q * 8 * kWave + i * kWave + lane, v ^ u32x4{(uint32_t)i, 0u, 0u, 0u});
    }
  }
}

// The 8:1 mix with burstier writes: a wave reads 64 KiB contiguous (8 rounds
// of 8 KiB, folded into 8 accumulators) and then writes 8 KiB contiguous.
// nvec counts the read side (multiple of 4096 vectors).
// Arrival count and generation of the soft grid barrier (zero when the code
// object loads).  Every workgroup of a launch arrives exactly once; the last
// arrival resets the count and advances the generation.
__device__ unsigned int g_probe_barrier[2];

// Waits until every workgroup of the grid has arrived or `timeout` ticks of
// the 100 MHz real-time clock have passed, whichever comes first.  The wait
// orders nothing that correctness depends on: it only holds the grid's
// writes back until its reads are done.  Called by all threads.
__device__ void soft_grid_barrier(unsigned int* bar, uint64_t timeout) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned gen = __hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned arrived = __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    if (arrived == gridDim.x) {
      __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen &&
             __builtin_amdgcn_s_memrealtime() - t0 < timeout)
        __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Operation 7 with depth field 2: the 8:1 phases of operation 7 done once per
// wave (the launch needs no more chunks than waves), with a soft grid
// barrier (at most 20 us) between every wave's reads and its writes.
__global__ __launch_bounds__(1024) void bw_phase_bar_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t nvec) {
  constexpr int kHeld = 16;
  const int lane = lane_id();
  const int64_t nchunk = nvec / (8 * kHeld * kWave);
  const int64_t q = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_group();
  const bool has = q < nchunk;
  u32x4 acc[kHeld];
  if (has) {
    const u32x4* s = src + q * 8 * kHeld * kWave + lane;
#pragma unroll
    for (int i = 0; i < kHeld; ++i) acc[i] = ld16<true>(s + i * kWave);
#pragma unroll
    for (int g = 2; g < 16; ++g) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ld16<true>(s + (g * 8 + i) * kWave);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[(g & 1) * 8 + i] ^= v[i];
    }
  }
  soft_grid_barrier(g_probe_barrier, 2000);
  if (has) {
#pragma unroll
    for (int i = 0; i < kHeld; ++i) st16<true>(dst + q * kHeld * kWave + i * kWave + lane, acc[i]);
  }
}

// Operation 7: the 8:1 mix in two phases per wave.  A wave reads 128 KiB
// (eight 16 KiB blocks folded into 16 vectors per lane) before it writes its
// 16 KiB.  Launched with one chunk per wave, every wave of the grid reads
// first and writes at the end, so reads and writes meet only while the grid
// starts and drains.
__global__ __launch_bounds__(1024) void bw_phase_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t nvec) {
  constexpr int kHeld = 16;
  const int lane = lane_id();
  const int64_t wpg = blockDim.x >> 6;
  const int64_t nchunk = nvec / (8 * kHeld * kWave);
  for (int64_t q = (int64_t)blockIdx.x * wpg + wave_in_group(); q < nchunk; q += (int64_t)gridDim.x * wpg) {
    const u32x4* s = src + q * 8 * kHeld * kWave + lane;
    u32x4 acc[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) acc[i] = ld16<true>(s + i * kWave);
    // groups of 8 loads (8 KiB per wave in flight); the scheduling barrier
    // keeps each group's loads ahead of its xors
#pragma unroll
    for (int g = 2; g < 16; ++g) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ld16<true>(s + (g * 8 + i) * kWave);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[(g & 1) * 8 + i] ^= v[i];
    }
#pragma unroll
    for (int i = 0; i < kHeld; ++i) st16<true>(dst + q * kHeld * kWave + i * kWave + lane, acc[i]);
  }
}

// Operation 7 with depth field 1: the 1:8 mix in two phases per wave.  A
// wave reads 16 KiB and then writes it eight times (vector i of copy r with
// r folded into its first word), 128 KiB.
__global__ __launch_bounds__(1024) void bw_phase_out_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t nvec) {
  constexpr int kHeld = 16;
  const int lane = lane_id();
  const int64_t wpg = blockDim.x >> 6;
  const int64_t nchunk = nvec / (8 * kHeld * kWave);
  for (int64_t q = (int64_t)blockIdx.x * wpg + wave_in_group(); q < nchunk; q += (int64_t)gridDim.x * wpg) {
    u32x4 v[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) v[i] = ld16<true>(src + (q * kHeld + i) * kWave + lane);
    u32x4* d = dst + q * 8 * kHeld * kWave + lane;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int i = 0; i < kHeld; ++i) {
        u32x4 o = v[i];
        o[0] ^= (unsigned)r;
        st16<true>(d + (r * kHeld + i) * kWave, o);
      }
    }
  }
}

__global__ __launch_bounds__(1024) void bw_mix_burst_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t nvec) {
  const int lane = lane_id();
  const int64_t wpg = blockDim.x >> 6;
  const int64_t nchunk = nvec / (64 * kWave);
  for (int64_t q = (int64_t)blockIdx.x * wpg + wave_in_group(); q < nchunk; q += (int64_t)gridDim.x * wpg) {
    u32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = u32x4{0u, 0u, 0u, 0u};
    for (int r = 0; r < 8; ++r) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ld16<true>(src + q * 64 * kWave + (r * 8 + i) * kWave + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] ^= v[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) st16<true>(dst + q * 8 * kWave + i * kWave + lane, acc[i]);
  }
}

// ---- in-flight read probe with a pointer chase
//
// Every wave but one streams reads of src (streaming nt loads, or cacheable
// ones with NTL = false) in batches of V 16-byte vectors per lane; the next batch is issued before the current one is folded, so V
// to 2V vectors per lane stay in flight.  Wave 0 of workgroup 0 instead
// follows `hops` links of `chain` (element i holds the index of the next
// element; an index outside [0, chain_len) restarts at 0), one dependent
// vector load at a time, and records the 100 MHz real-time ticks and
// shader-clock cycles it took: the load latency seen on a CU whose other
// waves keep streaming (or, with nothing to stream, unloaded).
__device__ __forceinline__ int64_t chase_load(const int64_t* p) {
  int64_t v;
  // a vector load (not a scalar one) and its wait in one statement
  asm volatile("global_load_dwordx2 %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Two batches of V vectors per lane: 16 leave room for 8 waves per CU only.
template <int V>
constexpr int inflight_max_threads() {
  return V >= 16 ? 512 : 1024;
}

template <int V, bool NTL>
__global__ __launch_bounds__(inflight_max_threads<V>()) void inflight_kernel(const u32x4* __restrict__ src, int64_t nvec,
                                                        u32x4* __restrict__ sink, const int64_t* __restrict__ chain,
                                                        int64_t chain_len, int64_t hops, int64_t* __restrict__ out) {
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int chasers = hops > 0 ? 1 : 0;
  if (chasers && blockIdx.x == 0 && wave == 0) {
    int64_t idx = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    for (int64_t h = 0; h < hops; ++h) {
      const int64_t nx = chase_load(chain + idx);
      idx = (uint64_t)nx < (uint64_t)chain_len ? nx : 0;
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      out[0] = (int64_t)(t1 - t0);
      out[1] = (int64_t)(c1 - c0);
      out[2] = idx;
      out[3] = (int64_t)hw_id_reg() | ((int64_t)(xcc_id_reg() & 0xF) << 32);
    }
    return;
  }
  const int64_t nstream = (int64_t)gridDim.x * wpg - chasers;
  const int64_t sid = (int64_t)blockIdx.x * wpg + wave - chasers;
  constexpr int64_t kChunk = (int64_t)V * kWave;
  const int64_t stride = nstream * kChunk;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 a[V], b[V];
  int64_t c = sid * kChunk;
  if (c < nvec) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int64_t e = c + i * kWave + lane;
      a[i] = e < nvec ? ld16<NTL>(src + e) : acc;
    }
    for (;;) {
      int64_t n1 = c + stride;
      if (n1 < nvec) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int64_t e = n1 + i * kWave + lane;
          b[i] = e < nvec ? ld16<NTL>(src + e) : acc;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i) acc ^= a[i];
      if (n1 >= nvec) break;
      c = n1;
      n1 = c + stride;
      if (n1 < nvec) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int64_t e = n1 + i * kWave + lane;
          a[i] = e < nvec ? ld16<NTL>(src + e) : acc;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i) acc ^= b[i];
      if (n1 >= nvec) break;
      c = n1;
    }
  }
  // keeps the reads alive; true only for a vanishingly unlikely checksum
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0x94d049bbu) sink[0] = acc;
}

using BwFn = void (*)(const u32x4*, u32x4*, int64_t);

template <int OP, int D>
BwFn bw_pick_pol(int pol) {
  switch (pol) {
    case 1: return bw_kernel<OP, D, 1>;
    case 2: return bw_kernel<OP, D, 2>;
    case 3: return bw_kernel<OP, D, 3>;
    case 4: return bw_kernel<OP, D, 4>;
    case 5: return bw_kernel<OP, D, 5>;
    default: return bw_kernel<OP, D, 0>;
  }
}

template <int OP>
BwFn bw_pick_depth(int depth, int pol) {
  switch (depth) {
    case 1: return bw_pick_pol<OP, 16>(pol);
    case 2: return bw_pick_pol<OP, 32>(pol);
    default: return bw_pick_pol<OP, 8>(pol);
  }
}

// Each workgroup records where it runs, then holds its CU for ~50 us (a
// bounded wait on the 100 MHz real-time counter) so that all workgroups of
// the grid are resident at once.
__global__ __launch_bounds__(64) void placement_kernel(int32_t* __restrict__ out) {
  if (threadIdx.x == 0) {
    const uint32_t hw = hw_id_reg();
    const uint32_t xcc = xcc_id_reg() & 0xF;
    const uint32_t cu = (hw >> 8) & 0xF;
    const uint32_t sh = (hw >> 12) & 0x1;
    const uint32_t se = (hw >> 13) & 0x7;
    out[4 * blockIdx.x + 0] = (int32_t)xcc;
    out[4 * blockIdx.x + 1] = (int32_t)se;
    out[4 * blockIdx.x + 2] = (int32_t)((sh << 4) | cu);
    out[4 * blockIdx.x + 3] = (int32_t)hw;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < 5000ull) __builtin_amdgcn_s_sleep(2);
}

}  // namespace

hipError_t launch_bw_probe(const Budget& b, int mode, const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int op = mode & 7;
  const int depth_code = (mode >> 4) & 3;
  const int pol = (mode >> 8) & 7;
  const int depth = depth_code == 1 ? 16 : depth_code == 2 ? 32 : 8;
  if (depth_code == 3 || pol > 5) return hipErrorInvalidValue;
  const int64_t nvec = bytes / 16;

  BwFn fn = op == 0 ? bw_pick_depth<0>(depth_code, 0)
          : op == 1 ? bw_pick_depth<1>(depth_code, pol)
          : op == 2 ? bw_pick_depth<2>(depth_code, 0)
          : op == 3 ? bw_pick_depth<3>(depth_code, pol)
          : op == 4 ? (BwFn)bw_mix_kernel<0>
          : op == 5 ? (BwFn)bw_mix_kernel<1>
          : op == 6 ? (BwFn)bw_mix_burst_kernel
          : depth_code == 1 ? (BwFn)bw_phase_out_kernel
          : depth_code == 2 ? (BwFn)bw_phase_bar_kernel
                    : (BwFn)bw_phase_kernel;
  const size_t per_wave = op == 3 ? (size_t)depth * kWaveVecBytes : 0;
  int wpg, grid;
  size_t lds = 0;
  if (b.num_cus > 0 || op == 7) {
    // one workgroup of 16 waves per CU (operation 7 always runs this way)
    wpg = 16;
    if (per_wave && (int)(kLdsPerCu / per_wave) < wpg) wpg = (int)(kLdsPerCu / per_wave);
    grid = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    lds = per_wave * wpg;
    if (lds < kExclusiveLds) lds = kExclusiveLds;
  } else {
    wpg = 4;
    const int64_t per_group = (int64_t)depth * kWave * wpg;
    const int64_t want = (nvec + per_group - 1) / per_group;
    int per_cu = per_wave ? (int)(kLdsPerCu / (per_wave * wpg)) : 8;
    if (per_cu > 8) per_cu = 8;
    if (per_cu < 1) per_cu = 1;
    const int64_t cap = (int64_t)b.device_cus * per_cu;
    grid = (int)(want < cap ? want : cap);
    lds = per_wave * wpg;
  }
  if (grid < 1) grid = 1;
  // the barrier kernel handles one chunk per wave
  if (op == 7 && depth_code == 2 && nvec / (8 * 16 * kWave) > (int64_t)grid * wpg) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), nvec);
  return hipGetLastError();
}

using InflightFn = void (*)(const u32x4*, int64_t, u32x4*, const int64_t*, int64_t, int64_t, int64_t*);

template <bool NTL>
InflightFn inflight_pick(int vec_per_lane) {
  return vec_per_lane == 1 ? inflight_kernel<1, NTL> : vec_per_lane == 2 ? inflight_kernel<2, NTL>
       : vec_per_lane == 4 ? inflight_kernel<4, NTL> : vec_per_lane == 8 ? inflight_kernel<8, NTL>
       : vec_per_lane == 16 ? inflight_kernel<16, NTL> : nullptr;
}

hipError_t launch_inflight_probe(const Budget& b, int waves_per_cu, int vec_per_lane, int cached, const void* src,
                                 int64_t bytes, void* sink, const int64_t* chain, int64_t chain_len, int64_t hops,
                                 int64_t* out, hipStream_t stream) {
  InflightFn fn = cached ? inflight_pick<false>(vec_per_lane) : inflight_pick<true>(vec_per_lane);
  if (!fn) return hipErrorInvalidValue;
  // one workgroup per CU of the budget (exclusive LDS), waves_per_cu waves each
  int grid = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  if (grid < 1) grid = 1;
  const size_t lds = kExclusiveLds;
  hipError_t e = allow_dynamic_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(waves_per_cu * kWave), lds, stream, static_cast<const u32x4*>(src),
                     bytes / 16, static_cast<u32x4*>(sink), chain, chain_len, hops, out);
  return hipGetLastError();
}

hipError_t launch_placement(const Budget& b, int n_groups, int32_t* out, hipStream_t stream, int* launched) {
  int grid = n_groups;
  if (b.num_cus > 0) {
    const int cus = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    if (cus < grid) grid = cus;
  }
  if (grid < 1) grid = 1;
  const size_t lds = kExclusiveLds;
  hipError_t e = allow_dynamic_lds((const void*)placement_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(placement_kernel, dim3(grid), dim3(64), lds, stream, out);
  *launched = grid;
  return hipGetLastError();
}

}  // namespace ep

namespace ep {

namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// A compute-bound stand-in for the expert GEMM beside the copy kernels: each
// wave runs `iters` rounds of four independent 32x32x8 bf16 matrix-core
// products on register operands (no memory traffic).  The sum of the
// accumulators is compared with a value it never takes, so the work stays
// live without a store; out is written only in that impossible case.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const int lane = lane_id();
  bf16x4_t a, b;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q] = (short)(0x3F80 + ((lane + q) & 7));  // small positive bf16 values
    b[q] = (short)(0x3F80 + ((lane * 3 + q) & 7));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) s += c0[q] + c1[q] + c2[q] + c3[q];
  if (s == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int n_groups, int iters, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_groups), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace ep
