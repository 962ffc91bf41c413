// ep_combine_reduce: the combine done from the expert side, by reduce-on-store.
//
//   acc[t, :] = 0                                   (fp32 [T, H], workspace)
//   for every receive row r with token t = src_token[r] and slot j
//   (dest_row[t, j] == r):  acc[t, :] += w[t, j] * f32(y[r, :])   (atomics)
//   out[t, :] = bf16_rne(acc[t, :])
//
// [TMA-notes], section "TMA 的其他特性（单卡 / Cluster 内）", item 3, describes a
// bulk store from shared memory that reduces element-wise (add, min, max)
// into its global destination, so that several producers can accumulate into
// one output.  gfx950 has no such store; the reduction here is an fp32 atomic
// add per element, executed by the GPU's caches.  y is read
// once, in receive-row order, as one sequential stream; the price is k
// read-modify-write operations per accumulator element and a zeroing and a
// conversion pass over the fp32 accumulator.  The order in which the k
// products of an element are added is not fixed, so the result is not
// bit-reproducible: it is correct to fp32 rounding of a k-term sum, then
// rounded once to bf16.  Products are rounded separately (no fused
// multiply-add), as in ep_combine.
//
// Three launches on the caller's stream: zero, scatter-add, convert.  A work
// unit of the scatter pass is (receive row, slab of VPL KiB).  Each lane
// loads 16 bytes (8 bf16) and forms 8 products; the wave writes them to its
// LDS slice in element order and reads them back transposed, so that each
// atomic instruction covers 64 consecutive floats (256 contiguous bytes)
// instead of 64 floats spread over 2 KiB.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "row_io.hpp"

namespace ep {

namespace {

constexpr int kRedVpl = 2;                        // 2 KiB of y per unit
constexpr int kRedSliceBytes = kRedVpl * 2 * kWaveVecBytes;  // 8 floats per lane per vector

__global__ __launch_bounds__(1024) void reduce_zero_kernel(u32x4* __restrict__ acc, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) acc[i] = z;
}

// out vector i (8 bf16) = round(acc floats 8i .. 8i + 7); acc and out are
// both contiguous [T, H].
__global__ __launch_bounds__(1024) void reduce_convert_kernel(const u32x4* __restrict__ acc, u32x4* __restrict__ out,
                                                             int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 a = ld16<true>(acc + 2 * i);
    const u32x4 b = ld16<true>(acc + 2 * i + 1);
    u32x4 o;
    o[0] = pack_bf16x2(__uint_as_float(a[0]), __uint_as_float(a[1]));
    o[1] = pack_bf16x2(__uint_as_float(a[2]), __uint_as_float(a[3]));
    o[2] = pack_bf16x2(__uint_as_float(b[0]), __uint_as_float(b[1]));
    o[3] = pack_bf16x2(__uint_as_float(b[2]), __uint_as_float(b[3]));
    st16<true>(out + i, o);
  }
}

// Slot of receive row r in token t's routing, or -1 (then the row is not
// added: its src_token entry is stale or the routing does not list it).
template <int K>
__device__ __forceinline__ int slot_of(const int32_t* __restrict__ dr, int k, int64_t r) {
  int jr = -1;
  if constexpr (K > 0) {
    int32_t d[K];
#pragma unroll
    for (int j = 0; j < K; ++j) d[j] = dr[j];
#pragma unroll
    for (int j = K - 1; j >= 0; --j)
      if (d[j] == r) jr = j;
  } else {
    for (int j = 0; j < k; ++j) {
      if (dr[j] == r) {
        jr = j;
        break;
      }
    }
  }
  return jr;
}

// Routing of one scatter unit: its receive row, token, slot weight, and
// whether the row is to be added at all.  Loads stay unconditional (token 0's
// routing stands in for a row that adds nothing), so that no branch sits
// between a unit's loads and their use.
struct RedUnit {
  Unit un;
  int64_t r;
  int t;
  float wt;
  bool ok;
};

template <int K>
__device__ __forceinline__ RedUnit red_route(int u, int nslab, int row_vec, int lane,
                                             const int32_t* __restrict__ src_token,
                                             const int32_t* __restrict__ dest_row, const float* __restrict__ w, int T,
                                             int k) {
  RedUnit ru;
  ru.un = unit_of<kRedVpl>(u, nslab, row_vec, lane);
  ru.r = ru.un.t;
  const int t = src_token[ru.r];
  const bool tok = (unsigned)t < (unsigned)T;
  ru.t = tok ? t : 0;
  const int j = slot_of<K>(dest_row + (int64_t)ru.t * k, k, ru.r);
  ru.ok = tok && j >= 0;
  ru.wt = w[(int64_t)ru.t * k + (j >= 0 ? j : 0)];
  return ru;
}

// Products of one unit go to the wave's LDS slice in element order (lane L's
// 8 floats of vector group i at slice[512 i + 8 L ..]) and come back
// transposed (lane L takes elements 64 q + L), so that each atomic covers 256
// contiguous bytes.  A unit that adds nothing adds +0.0 to token 0 instead
// (x + 0 == x, and the accumulator, started at +0, never holds -0).
template <bool EVEN>
__device__ __forceinline__ void red_process(const RedUnit& ru, const u32x4 (&v)[kRedVpl], float* slice,
                                            float* __restrict__ acc, int lane, int H) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < kRedVpl; ++i) {
    float p[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = ru.wt * bf16_lo(v[i][q]);
      const float hi = ru.wt * bf16_hi(v[i][q]);
      p[2 * q] = ru.ok ? lo : 0.0f;
      p[2 * q + 1] = ru.ok ? hi : 0.0f;
    }
    float4* s4 = reinterpret_cast<float4*>(slice + 512 * i + 8 * lane);
    s4[0] = make_float4(p[0], p[1], p[2], p[3]);
    s4[1] = make_float4(p[4], p[5], p[6], p[7]);
  }
  // one wave: its LDS writes complete before its later LDS reads; the fence
  // keeps the compiler from moving the reads of other lanes' values up
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float val[kRedVpl][8];
#pragma unroll
  for (int i = 0; i < kRedVpl; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) val[i][q] = slice[512 * i + 64 * q + lane];
  float* arow = acc + (int64_t)ru.t * H;
  const int e0 = 8 * (ru.un.c0 - lane);  // first element of the slab
#pragma unroll
  for (int i = 0; i < kRedVpl; ++i) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // elements past the unit's slab (a short last slab) are past the row end
      const int e = e0 + 512 * i + 64 * q + lane;
      if (i < ru.un.nvec && (EVEN || e < H))
        __hip_atomic_fetch_add(arow + e, val[i][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the next unit rewrites the slice: these reads must have completed
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two units per wave in flight: the next unit's routing and row loads are
// issued before the current unit's atomics, so a wave waits only for its own
// loads, never for its earlier atomics (both retire in issue order).
template <int K, bool EVEN>
__global__ __launch_bounds__(1024) void reduce_scatter_kernel(const u32x4* __restrict__ y, float* __restrict__ acc,
                                                              const int32_t* __restrict__ src_token,
                                                              const int32_t* __restrict__ dest_row,
                                                              const float* __restrict__ w, int T, int k_rt,
                                                              int row_vec, int nslab, int units) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  const int H = row_vec * 8;
  float* slice = reinterpret_cast<float*>(lds + wave * kRedSliceBytes);
  int u = blockIdx.x * wpg + wave;
  if (u >= units) return;
  u32x4 va[kRedVpl], vb[kRedVpl];
  RedUnit ca = red_route<K>(u, nslab, row_vec, lane, src_token, dest_row, w, T, k);
  load_slab_fixed<kRedVpl, true>(va, y + (ca.ok ? ca.r : 0) * row_vec, ca.un, row_vec);
  for (;;) {
    // the unit after the last one re-reads the last one, unused: unconditional
    // loads keep the waits exact
    int un = u + stride;
    bool more = un < units;
    const RedUnit cb = red_route<K>(more ? un : u, nslab, row_vec, lane, src_token, dest_row, w, T, k);
    load_slab_fixed<kRedVpl, true>(vb, y + (cb.ok ? cb.r : 0) * row_vec, cb.un, row_vec);
    red_process<EVEN>(ca, va, slice, acc, lane, H);
    if (!more) break;
    u = un;
    un = u + stride;
    more = un < units;
    ca = red_route<K>(more ? un : u, nslab, row_vec, lane, src_token, dest_row, w, T, k);
    load_slab_fixed<kRedVpl, true>(va, y + (ca.ok ? ca.r : 0) * row_vec, ca.un, row_vec);
    red_process<EVEN>(cb, vb, slice, acc, lane, H);
    if (!more) break;
    u = un;
  }
}

using ScatterFn = void (*)(const u32x4*, float*, const int32_t*, const int32_t*, const float*, int, int, int, int,
                           int);

template <bool EVEN>
ScatterFn pick_scatter(int k) {
  switch (k) {
    case 2: return reduce_scatter_kernel<2, EVEN>;
    case 4: return reduce_scatter_kernel<4, EVEN>;
    case 6: return reduce_scatter_kernel<6, EVEN>;
    case 8: return reduce_scatter_kernel<8, EVEN>;
    default: return reduce_scatter_kernel<0, EVEN>;
  }
}

// Geometry of the two streaming passes: on a CU budget, one workgroup of 16
// waves per CU of the budget (holding more than half a CU's LDS, so no two
// share a CU); otherwise workgroups of 4 waves over the whole device.
struct StreamLaunch {
  int grid, threads;
  size_t lds;
};

StreamLaunch stream_launch(const Budget& b, int64_t nvec) {
  StreamLaunch s;
  if (b.num_cus > 0) {
    s.grid = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    s.threads = 1024;
    s.lds = kExclusiveLds;
    return s;
  }
  int64_t g = (nvec + 255) / 256;
  const int64_t cap = (int64_t)b.device_cus * 8;
  if (g > cap) g = cap;
  s.grid = g < 1 ? 1 : (int)g;
  s.threads = 256;
  s.lds = 0;
  return s;
}

}  // namespace

size_t combine_reduce_workspace_bytes(int T, int H) { return (size_t)T * (size_t)H * sizeof(float); }

hipError_t launch_combine_reduce(const Budget& b, const void* y, int64_t recv_rows, int H, const int32_t* src_token,
                                 const int32_t* dest_row, const float* w, int T, int k, void* out, void* acc,
                                 hipStream_t stream) {
  const int row_vec = H / 8;
  const int64_t out_vec = (int64_t)T * row_vec;

  // 1. zero the accumulator (a fill kernel, not a memset node, so the call
  //    can be captured in a graph)
  const StreamLaunch zl = stream_launch(b, 2 * out_vec);
  hipError_t e = hipSuccess;
  if (zl.lds > 64 * 1024) {
    e = allow_dynamic_lds((const void*)reduce_zero_kernel, zl.lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reduce_zero_kernel, dim3(zl.grid), dim3(zl.threads), zl.lds, stream, static_cast<u32x4*>(acc),
                     2 * out_vec);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 2. scatter-add every receive row into its token's accumulator row
  if (recv_rows > 0) {
    const int nslab = (row_vec + kRedVpl * kWave - 1) / (kRedVpl * kWave);
    if (recv_rows * nslab > INT32_MAX) return hipErrorInvalidValue;
    const int units = (int)(recv_rows * nslab);
    const bool even = row_vec % kWave == 0;
    ScatterFn fn = even ? pick_scatter<true>(k) : pick_scatter<false>(k);
    int wpg, grid;
    size_t lds_bytes;
    if (b.num_cus > 0) {
      wpg = 16;
      grid = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
      lds_bytes = (size_t)wpg * kRedSliceBytes;
      if (lds_bytes < kExclusiveLds) lds_bytes = kExclusiveLds;
    } else {
      wpg = 4;
      grid = (units + wpg - 1) / wpg;
      if (grid > b.device_cus * 8) grid = b.device_cus * 8;
      lds_bytes = (size_t)wpg * kRedSliceBytes;
    }
    if (grid < 1) grid = 1;
    if (lds_bytes > 64 * 1024) {
      e = allow_dynamic_lds((const void*)fn, lds_bytes);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(y),
                       static_cast<float*>(acc), src_token, dest_row, w, T, k, row_vec, nslab, units);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // 3. round the accumulator to bf16
  const StreamLaunch cl = stream_launch(b, out_vec);
  if (cl.lds > 64 * 1024) {
    e = allow_dynamic_lds((const void*)reduce_convert_kernel, cl.lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reduce_convert_kernel, dim3(cl.grid), dim3(cl.threads), cl.lds, stream,
                     static_cast<const u32x4*>(acc), static_cast<u32x4*>(out), out_vec);
  return hipGetLastError();
}

}  // namespace ep
