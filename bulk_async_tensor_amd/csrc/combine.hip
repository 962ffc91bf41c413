// ep_combine: out[t, :] = bf16_rne( sum_{j<k} w[t, j] * f32(y[dest_row[t, j], :]) )
//
// The way back from the expert-grouped layout.  The pages show only the
// dispatch direction; the combine here is its inverse gather, weighted by the
// gate weights that the dispatch call of [DeepEP-TMA] ("High-Level DeepEP API
// Usage") takes alongside the expert ids.  Accumulation is fp32 from +0.0 in
// slot order with every product and sum rounded separately (contraction into
// fused multiply-add is switched off), then one round-to-nearest-even to
// bf16 with the hardware pack instruction.
//
// A work unit is (token, slab); the k source rows of the slab are gathered
// with 16-byte loads.  Variants mirror the dispatch kernels:
//   vgpr   all k x VPL loads of a unit issued together into registers;
//   vgpr2  two register sets: the next unit's k rows load while the current
//          one is summed and stored;
//   lds1   k rows land in a per-wave LDS slice by direct-to-LDS loads, one
//          stage;
//   lds2   two stages: the next unit's direct-to-LDS loads are in flight while
//          the current stage is read, summed and stored.
//   phase  each wave holds up to 16 finished output vectors per lane (a
//          whole row at H = 7168) in registers and stores them only after
//          it has read all of their source rows.  With at most one such unit
//          per wave, the grid reads first and writes last: HBM sees almost
//          no read/write turnaround, which a steady 8:1 mix pays on every
//          channel.
// The k destination rows and weights of a unit are fetched with scalar loads
// before its first row load.  EVEN = the row is a whole number of KiB, so no
// per-lane row-end masks are needed.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "row_io.hpp"

namespace ep {

namespace {

__device__ __forceinline__ bool row_ok(int64_t d, int64_t rows) { return (uint64_t)d < (uint64_t)rows; }

// Routing of one token: destination rows and gate weights of its k slots.
template <int K>
struct Slots {
  int32_t d[K];
  float w[K];
};

template <int K>
__device__ __forceinline__ void fetch_slots(Slots<K>& s, const int32_t* __restrict__ dr, const float* __restrict__ wr) {
#pragma unroll
  for (int j = 0; j < K; ++j) s.d[j] = dr[j];
#pragma unroll
  for (int j = 0; j < K; ++j) s.w[j] = wr[j];
}

// acc += w * f32(v) for the 8 bf16 of each vector; no contraction.
template <int VPL>
__device__ __forceinline__ void accumulate(float (&acc)[VPL][8], const u32x4 (&v)[VPL], float w, int nvec) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i < nvec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p0 = w * bf16_lo(v[i][q]);
        const float p1 = w * bf16_hi(v[i][q]);
        acc[i][2 * q] = acc[i][2 * q] + p0;
        acc[i][2 * q + 1] = acc[i][2 * q + 1] + p1;
      }
    }
  }
}

template <int VPL>
__device__ __forceinline__ void zero(float (&acc)[VPL][8]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
}

// Writes the slab; returns the number of store instructions issued (lane 0
// is inside the row for every vector < nvec, so none is skipped).
template <int VPL, bool EVEN, bool NT>
__device__ __forceinline__ int store_out(u32x4* __restrict__ dst, const float (&acc)[VPL][8], const Unit& un,
                                         int row_vec) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i < un.nvec) {
      const int c = un.c0 + i * kWave;
      if (EVEN || c < row_vec) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
        st16<NT>(dst + c, o);
      }
    }
  }
  return un.nvec;
}

template <int VPL, int K, bool EVEN, bool NT>
__device__ __forceinline__ void load_unit(u32x4 (&v)[K][VPL], const Slots<K>& s, const u32x4* __restrict__ y,
                                          int64_t recv_rows, const Unit& un, int row_vec) {
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (row_ok(s.d[j], recv_rows)) load_slab<VPL, EVEN, NT>(v[j], y + (int64_t)s.d[j] * row_vec, un, row_vec);
}

template <int VPL, int K>
__device__ __forceinline__ void sum_unit(float (&acc)[VPL][8], const u32x4 (&v)[K][VPL], const Slots<K>& s,
                                         int64_t recv_rows, int nvec) {
  zero<VPL>(acc);
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (row_ok(s.d[j], recv_rows)) accumulate<VPL>(acc, v[j], s.w[j], nvec);
}

#define EP_COMBINE_ARGS                                                                                        \
  const u32x4 *__restrict__ y, u32x4 *__restrict__ out, const int32_t *__restrict__ dest_row,                 \
      const float *__restrict__ w, int64_t recv_rows, int row_vec, int nslab, int k_rt, int units

// Threads per workgroup the register budget allows: k x VPL in-flight
// vectors plus 8 VPL accumulators per lane.
template <int VPL>
constexpr int combine_max_threads() {
  return VPL >= 4 ? 512 : 1024;
}

// Compile-time k: all k x VPL loads of a unit in flight together.
template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(combine_max_threads<VPL>()) void combine_vgpr_kernel(EP_COMBINE_ARGS) {
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  for (int u = blockIdx.x * wpg + wave_in_group(); u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    Slots<K> s;
    fetch_slots<K>(s, dest_row + un.t * K, w + un.t * K);
    u32x4 v[K][VPL];
    load_unit<VPL, K, EVEN, NT>(v, s, y, recv_rows, un, row_vec);
    float acc[VPL][8];
    sum_unit<VPL, K>(acc, v, s, recv_rows, un.nvec);
    store_out<VPL, EVEN, NT>(out + un.t * row_vec, acc, un, row_vec);
  }
}

// Any k: slots in batches of 8 whose loads are in flight together.
template <int VPL, bool EVEN, bool NT>
__global__ __launch_bounds__(combine_max_threads<VPL>()) void combine_vgpr_any_kernel(EP_COMBINE_ARGS) {
  constexpr int KB = 8;
  const int k = k_rt;
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  for (int u = blockIdx.x * wpg + wave_in_group(); u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    const int32_t* dr = dest_row + un.t * k;
    const float* wr = w + un.t * k;
    float acc[VPL][8];
    zero<VPL>(acc);
    for (int jb = 0; jb < k; jb += KB) {
      u32x4 v[KB][VPL];
      int64_t d[KB];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) d[jj] = (jb + jj < k) ? (int64_t)dr[jb + jj] : -1;
#pragma unroll
      for (int jj = 0; jj < KB; ++jj)
        if (row_ok(d[jj], recv_rows)) load_slab<VPL, EVEN, NT>(v[jj], y + d[jj] * row_vec, un, row_vec);
#pragma unroll
      for (int jj = 0; jj < KB; ++jj)
        if (row_ok(d[jj], recv_rows)) accumulate<VPL>(acc, v[jj], wr[jb + jj], un.nvec);
    }
    store_out<VPL, EVEN, NT>(out + un.t * row_vec, acc, un, row_vec);
  }
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void combine_vgpr2_kernel(EP_COMBINE_ARGS) {
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  int u = blockIdx.x * wpg + wave_in_group();
  if (u >= units) return;
  Unit cur = unit_of<VPL>(u, nslab, row_vec, lane);
  Slots<K> sa, sb;
  fetch_slots<K>(sa, dest_row + cur.t * K, w + cur.t * K);
  u32x4 a[K][VPL], b[K][VPL];
  float acc[VPL][8];
  load_unit<VPL, K, EVEN, NT>(a, sa, y, recv_rows, cur, row_vec);
  for (;;) {
    // two units per trip so that the register sets swap roles without moves
    int un = u + stride;
    Unit nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (un < units) {
      fetch_slots<K>(sb, dest_row + nxt.t * K, w + nxt.t * K);
      load_unit<VPL, K, EVEN, NT>(b, sb, y, recv_rows, nxt, row_vec);
    }
    sum_unit<VPL, K>(acc, a, sa, recv_rows, cur.nvec);
    store_out<VPL, EVEN, NT>(out + cur.t * row_vec, acc, cur, row_vec);
    if (un >= units) break;
    u = un;
    cur = nxt;
    un = u + stride;
    nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (un < units) {
      fetch_slots<K>(sa, dest_row + nxt.t * K, w + nxt.t * K);
      load_unit<VPL, K, EVEN, NT>(a, sa, y, recv_rows, nxt, row_vec);
    }
    sum_unit<VPL, K>(acc, b, sb, recv_rows, cur.nvec);
    store_out<VPL, EVEN, NT>(out + cur.t * row_vec, acc, cur, row_vec);
    if (un >= units) break;
    u = un;
    cur = nxt;
  }
}

// Stage layout: slot j, vector i at stage + (j * VPL + i) KiB, lane L at +16 L.
template <int VPL, int K, bool EVEN>
__device__ __forceinline__ void dma_unit(char* stage, const Slots<K>& s, const u32x4* __restrict__ y,
                                         int64_t recv_rows, const Unit& un, int row_vec) {
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (row_ok(s.d[j], recv_rows)) {
      const u32x4* src = y + (int64_t)s.d[j] * row_vec;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        if (i < un.nvec) {
          const int c = un.c0 + i * kWave;
          if (EVEN || c < row_vec) dma16(src + c, (lds_void_t*)(stage + (j * VPL + i) * kWaveVecBytes));
        }
      }
    }
  }
}

// Reads the whole stage (slots that were not filled hold stale bytes of this
// wave's own slice and are never summed): unconditional reads keep the
// register allocation simple.
template <int VPL, int K>
__device__ __forceinline__ void read_unit(u32x4 (&v)[K][VPL], const char* stage, int lane) {
  const uint32_t base = lds_addr_of(stage) + lane * kVecBytes;
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < VPL; ++i) lds_read16_async(v[j][i], base + (j * VPL + i) * kWaveVecBytes);
  lds_wait_all();
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < VPL; ++i) lds_fence_value(v[j][i]);
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void combine_lds1_kernel(EP_COMBINE_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  char* stage = lds + wave * (K * VPL * kWaveVecBytes);
  for (int u = blockIdx.x * wpg + wave; u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    Slots<K> s;
    fetch_slots<K>(s, dest_row + un.t * K, w + un.t * K);
    dma_unit<VPL, K, EVEN>(stage, s, y, recv_rows, un, row_vec);
    wait_vmcnt<0>();
    u32x4 v[K][VPL];
    read_unit<VPL, K>(v, stage, lane);
    float acc[VPL][8];
    sum_unit<VPL, K>(acc, v, s, recv_rows, un.nvec);
    store_out<VPL, EVEN, NT>(out + un.t * row_vec, acc, un, row_vec);
  }
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void combine_lds2_kernel(EP_COMBINE_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kStageBytes = K * VPL * kWaveVecBytes;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  char* ring = lds + wave * (2 * kStageBytes);
  int u = blockIdx.x * wpg + wave;
  if (u >= units) return;
  Unit cur = unit_of<VPL>(u, nslab, row_vec, lane);
  Slots<K> scur, snxt;
  fetch_slots<K>(scur, dest_row + cur.t * K, w + cur.t * K);
  dma_unit<VPL, K, EVEN>(ring, scur, y, recv_rows, cur, row_vec);
  int stage = 0;
  int issued_after = 0;  // vector-memory instructions issued after the pending fill of `stage`
  for (;;) {
    // vmcnt retires in issue order: letting at most `issued_after` newer
    // operations (the previous unit's output stores) stay outstanding is exact
    if (issued_after >= VPL) wait_vmcnt<VPL>();
    else wait_vmcnt<0>();
    u32x4 v[K][VPL];
    read_unit<VPL, K>(v, ring + stage * kStageBytes, lane);  // stage is free again
    const int un = u + stride;
    const bool more = un < units;
    const Unit nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (more) {
      fetch_slots<K>(snxt, dest_row + nxt.t * K, w + nxt.t * K);
      dma_unit<VPL, K, EVEN>(ring + (stage ^ 1) * kStageBytes, snxt, y, recv_rows, nxt, row_vec);
    }
    float acc[VPL][8];
    sum_unit<VPL, K>(acc, v, scur, recv_rows, cur.nvec);
    issued_after = store_out<VPL, EVEN, NT>(out + cur.t * row_vec, acc, cur, row_vec);
    if (!more) break;
    u = un;
    cur = nxt;
    scur = snxt;
    stage ^= 1;
  }
}

// Loads slot j's SEG vectors at the given columns (row 0 when the slot's row
// is out of range: those values are never summed).
template <int K, int SEG>
__device__ __forceinline__ void phase_load(u32x4 (&v)[SEG], const Slots<K>& s, int j, const u32x4* __restrict__ y,
                                           int64_t recv_rows, int row_vec, const int (&col)[SEG]) {
  const bool ok = row_ok(s.d[j], recv_rows);
  const u32x4* src = y + (ok ? (int64_t)s.d[j] : 0) * row_vec;
#pragma unroll
  for (int e = 0; e < SEG; ++e) v[e] = ld16<true>(src + col[e]);
}

// acc += w_j * f32(v) when slot j's row is in range (a select, not a branch,
// so no load waits on it); products and sums rounded separately.
template <int K, int SEG>
__device__ __forceinline__ void phase_sum(float (&acc)[SEG][8], const u32x4 (&v)[SEG], const Slots<K>& s, int j,
                                          int64_t recv_rows) {
#pragma clang fp contract(off)
  const bool ok = row_ok(s.d[j], recv_rows);
#pragma unroll
  for (int e = 0; e < SEG; ++e) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s0 = acc[e][2 * q] + s.w[j] * bf16_lo(v[e][q]);
      const float s1 = acc[e][2 * q + 1] + s.w[j] * bf16_hi(v[e][q]);
      acc[e][2 * q] = ok ? s0 : acc[e][2 * q];
      acc[e][2 * q + 1] = ok ? s1 : acc[e][2 * q + 1];
    }
  }
}

// Slots j0 .. j0 + G - 1 (those below K) of a register set.
template <int K, int SEG, int G>
__device__ __forceinline__ void phase_load_set(u32x4 (&v)[G][SEG], const Slots<K>& s, int j0,
                                               const u32x4* __restrict__ y, int64_t recv_rows, int row_vec,
                                               const int (&col)[SEG]) {
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (j0 + g < K) phase_load<K, SEG>(v[g], s, j0 + g, y, recv_rows, row_vec, col);
}

template <int K, int SEG, int G>
__device__ __forceinline__ void phase_sum_set(float (&acc)[SEG][8], const u32x4 (&v)[G][SEG], const Slots<K>& s,
                                              int j0, int64_t recv_rows) {
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (j0 + g < K) phase_sum<K, SEG>(acc, v[g], s, j0 + g, recv_rows);
}

// HELD output vectors held per wave; SEG vectors of a row are read per
// source row and step (SEG KiB contiguous per row), G slots per register
// set.  With several tokens per unit, SEG divides nv so that a step never
// spans two tokens.  MAXT: threads per workgroup at most (16 waves for the
// 16-vector hold; 8 for the 28-vector one, which needs about 175 VGPRs).
template <int K, int SEG, int G, int HELD, bool EVEN, int MAXT>
__global__ __launch_bounds__(MAXT) void combine_phase_kernel(const u32x4* __restrict__ y, u32x4* __restrict__ out,
                                                             const int32_t* __restrict__ dest_row,
                                                             const float* __restrict__ w, int64_t recv_rows,
                                                             int row_vec, int nv, int T, int tpu, int nseg, int seg,
                                                             int units) {
  constexpr int kSteps = (HELD + SEG - 1) / SEG;
  const int lane = lane_id();
  const int stride = gridDim.x * (blockDim.x >> 6);
  // Every wave makes its workgroup's trip count (waves past the last unit
  // work on the workgroup's first unit and store nothing), so each barrier
  // below is met by all of them.
  const int wfirst = blockIdx.x * (blockDim.x >> 6);
  const int trips = wfirst < units ? (units - wfirst + stride - 1) / stride : 0;
  for (int r = 0; r < trips; ++r) {
    const int u_raw = wfirst + r * stride + wave_in_group();
    const bool live = u_raw < units;
    const int u = live ? u_raw : wfirst;
    int t0, c0, n_in;
    if (nseg == 1) {
      t0 = u * tpu;
      c0 = 0;
      n_in = (T - t0 < tpu ? T - t0 : tpu) * nv;
    } else {
      t0 = u / nseg;
      c0 = (u - t0 * nseg) * seg;
      n_in = nv - c0 < seg ? nv - c0 : seg;
    }
    // Each token's vectors are visited from a rotated start, so that waves
    // that run in step do not all read the same offset of their rows at once
    // (with power-of-two rows that would load a few HBM channels at a time).
    const int span = nseg == 1 ? nv : n_in;
    const int rot = u % span;
    u32x4 held[HELD];
    int t = t0, p = 0, c = c0 + rot;
    Slots<K> s;
    fetch_slots<K>(s, dest_row + (int64_t)t * K, w + (int64_t)t * K);
#pragma unroll
    for (int g = 0; g < kSteps; ++g) {
      const int i0 = g * SEG;
      if (i0 < n_in) {
        if (i0 > 0 && p == 0) fetch_slots<K>(s, dest_row + (int64_t)t * K, w + (int64_t)t * K);
        // Straight-line loads (no branch between a load and its use lets the
        // compiler keep them all in flight): vectors past the unit and lanes
        // past a ragged row end read a valid column and are never stored;
        // slots whose row is out of range read row 0 and add nothing.
        int col[SEG];
#pragma unroll
        for (int e = 0; e < SEG; ++e) {
          col[e] = c * kWave + lane;
          if (!EVEN && col[e] >= row_vec) col[e] = row_vec - 1;
          if (i0 + e < HELD && i0 + e < n_in) {
            if (++c == c0 + span) c = c0;
            ++p;
          }
        }
        float acc[SEG][8];
        zero<SEG>(acc);
        // Two register sets of G slots each: the next set's loads are issued
        // before the current set is summed, so G to 2G slots (G SEG to 2G SEG
        // KiB per wave) stay in flight.  The scheduling barriers keep the
        // compiler from trading that depth for fewer registers.  (Carrying
        // the prefetch across steps as well spilled heavily.)
        u32x4 va[G][SEG], vb[G][SEG];
        phase_load_set<K, SEG, G>(va, s, 0, y, recv_rows, row_vec, col);
#pragma unroll
        for (int j = 0; j < K; j += 2 * G) {
          if (j + G < K) phase_load_set<K, SEG, G>(vb, s, j + G, y, recv_rows, row_vec, col);
          __builtin_amdgcn_sched_barrier(0);
          phase_sum_set<K, SEG, G>(acc, va, s, j, recv_rows);
          if (j + 2 * G < K) phase_load_set<K, SEG, G>(va, s, j + 2 * G, y, recv_rows, row_vec, col);
          __builtin_amdgcn_sched_barrier(0);
          if (j + G < K) phase_sum_set<K, SEG, G>(acc, vb, s, j + G, recv_rows);
        }
#pragma unroll
        for (int e = 0; e < SEG; ++e)
          if (i0 + e < HELD)
#pragma unroll
            for (int q = 0; q < 4; ++q) held[i0 + e][q] = pack_bf16x2(acc[e][2 * q], acc[e][2 * q + 1]);
        if (p == span) {
          p = 0;
          ++t;
        }
      }
    }
    // The workgroup meets before any of its waves stores: a CU's stores then
    // start only once all of its reads have returned, and do not queue
    // ahead of its waves' last reads in the CU's memory pipeline (prefill,
    // T = 16384: 265.5 against 271.5 us; train, T = 4096: 83.3 against
    // 85.7 us, x evicted).  The empty asm statements keep the finished
    // rows' computation, and so every load, above the barrier.
#pragma unroll
    for (int i = 0; i < HELD; ++i) asm volatile("" : "+v"(held[i]));
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    t = t0;
    p = 0;
    c = c0 + rot;
#pragma unroll
    for (int i = 0; i < HELD; ++i) {
      if (live && i < n_in) {
        const int col = c * kWave + lane;
        if (EVEN || col < row_vec) st16<true>(out + (int64_t)t * row_vec + col, held[i]);
        if (++c == c0 + span) c = c0;
        if (++p == span) {
          p = 0;
          ++t;
        }
      }
    }
  }
}

using PhaseFn = void (*)(const u32x4*, u32x4*, const int32_t*, const float*, int64_t, int, int, int, int, int, int,
                         int);

// Slots per register set: with single-vector runs, two sets of (k + 1) / 2
// (at odd k the second one is a slot short)
// (k = 6 in sets of 4 and 2 ran 3-10% slower than in two sets of 3 at
// H = 7168, T = 8192: 139.5 against 135.0 us and 139.9 against 129.3 us in
// two runs); with 2-vector runs, sets of 2 slots (4 KiB per wave).  (Runs of 4 vectors do not fit: two sets plus 32
// accumulators and the held output spill at k >= 6.)
constexpr int phase_set_slots(int k, int seg) { return seg == 1 ? (k + 1) / 2 : 2; }

template <int SEG, int HELD, bool EVEN, int MAXT = kPhaseWpg * kWave>
PhaseFn pick_phase_k(int k) {
  switch (k) {
    case 1: return combine_phase_kernel<1, SEG, phase_set_slots(1, SEG), HELD, EVEN, MAXT>;
    case 2: return combine_phase_kernel<2, SEG, phase_set_slots(2, SEG), HELD, EVEN, MAXT>;
    case 3: return combine_phase_kernel<3, SEG, phase_set_slots(3, SEG), HELD, EVEN, MAXT>;
    case 4: return combine_phase_kernel<4, SEG, phase_set_slots(4, SEG), HELD, EVEN, MAXT>;
    case 5: return combine_phase_kernel<5, SEG, phase_set_slots(5, SEG), HELD, EVEN, MAXT>;
    case 6: return combine_phase_kernel<6, SEG, phase_set_slots(6, SEG), HELD, EVEN, MAXT>;
    case 7: return combine_phase_kernel<7, SEG, phase_set_slots(7, SEG), HELD, EVEN, MAXT>;
    case 8: return combine_phase_kernel<8, SEG, phase_set_slots(8, SEG), HELD, EVEN, MAXT>;
    default: return nullptr;
  }
}

template <bool EVEN>
PhaseFn pick_phase(int seg_vec, int held, int k) {
  if (held == kPhaseWideHeld) return pick_phase_k<1, kPhaseWideHeld, EVEN, kPhaseWideWpg * kWave>(k);
  if (seg_vec == 2) return held == 14 ? pick_phase_k<2, 14, EVEN>(k) : pick_phase_k<2, 16, EVEN>(k);
  return held == 14 ? pick_phase_k<1, 14, EVEN>(k) : pick_phase_k<1, 16, EVEN>(k);
}

// Vectors per contiguous read of the phased combine, where a step can take
// runs of 2 (one row per unit, or an even row length): by default 1 at
// k >= 6 (runs of 2 measured 5% slower at the train shape: fewer slots in
// flight) and 2 at k <= 4, where a step of single vectors has too few loads
// to keep in flight (H = 7168, T k = 32 Ki: 5.82 against 4.91 TB/s at
// k = 4, 5.73 against 4.87 at k = 2); a requested slab of 1 or of 2 and
// more takes 1 or 2.
// Rows of 5 or 7 vectors per lane, which hold two tokens per unit, take
// 2-vector runs over the row padded by one vector: a token then spans an
// even number of vectors, so no run straddles two tokens, and k <= 4 takes
// the phased kernel instead of the register one.  The padding vector is
// loaded as the row's last one and never stored.  Cold, same-run A/B, k = 2,
// 3, 4, T = 8192 and 16384: H = 2304 / 2560 / 3584 4-14% faster (3584,
// k = 4, T = 16384: 113.0 against 99.5 us), T = 2048 and 4096 within 1%
// but for one 7% loss (2304, k = 3, T = 4096).  At 3 vectors the padding
// adds a third more loads: H = 1152, T = 8192 lost 14-19%.
bool phase_pad(int row_vec) {
  const int nv = (row_vec + kWave - 1) / kWave;
  return nv == 5 || nv == 7;
}

int combine_phase_seg(const Budget& b, int row_vec, int k) {
  const PhaseShape p16 = phase_shape(row_vec);
  const bool can2 = p16.tpu == 1 || p16.nv % 2 == 0 || phase_pad(row_vec);
  const bool want2 = b.slab_vpl >= 2 || (b.slab_vpl == 0 && k <= 4);
  return want2 && can2 ? 2 : 1;
}

// With every CU of the device, rows of 9 to 14 vectors per lane (H from
// 4104 to 7168) hold two or three whole rows per wave in workgroups of 8
// waves instead of one row in workgroups of 16: as many rows per CU (or
// more, at 9 vectors), written as one burst of two or three adjacent output
// rows per wave.  At the training shape this took the combine from 84.2 to
// 82.5 us (E = 256) and from 88.6 to 80.8 us (E = 128), bit-identical.  On
// fewer CUs the per-CU read rate is the bound and half the waves keep half
// the reads in flight: 4.2 against 5.1 TB/s on 128 CUs, 4.3 against 5.8 on
// 192, so there the 16-wave shape stays.  Larger rows would drop to one row
// per wave and smaller ones to fewer rows per CU.
//
// At 9 vectors a wave could hold three rows.  It takes two when that needs
// fewer passes over the grid (launches times rows per wave): at T = 8192 on
// 256 CUs three rows give 2731 units, two launches at two-thirds fill, and
// two rows give two full launches.  Cold, H = 4608, k = 8: T = 4096 65.2
// against 56.2 us, T = 8192 128.6 against 111.6; H = 4160, k = 6, 7, 8 at
// T = 4096 and 8192 6 to 13% faster (k = 8 had taken vgpr, whose fill rule
// the two-thirds fill failed); k = 5 and T = 2048 or 16384 within 2%.
//
// The 16-wave shape keeps its packing: the same rule there (at least two
// tokens per wave) measured within +-5% of it on rows of 2 to 8 KiB, k = 4,
// 6, 8, T = 2048 to 16384, a mean of +0.5%, with as many losses as gains.
PhaseShape combine_phase_shape(int row_vec, int seg_vec, int cus, int all_cus, int64_t T) {
  const int nv = (row_vec + kWave - 1) / kWave;
  if (seg_vec == 1 && nv >= 9 && nv <= 14 && cus >= all_cus) {
    PhaseShape p = phase_shape(row_vec, kPhaseWideHeld, kPhaseWideWpg);
    if (p.tpu > 2 && T > 0) {
      const int64_t slots = (int64_t)cus * p.wpg;
      auto passes = [&](int t) { return (T + slots * t - 1) / (slots * t) * t; };
      if (passes(2) < passes(p.tpu)) p.tpu = 2;
    }
    return p;
  }
  // (a padded row reads as one vector longer; the launch then takes the
  // kernel instance that clamps and skips columns past the row)
  if (seg_vec == 2 && phase_pad(row_vec)) return phase_shape(row_vec + kWave);
  return phase_shape(row_vec);
}


hipError_t launch_phase(const Budget& b, const void* y, int64_t recv_rows, int row_vec, const int32_t* dest_row,
                        const float* w, int T, int k, void* out, hipStream_t stream) {
  // 14 held vectors when a unit never needs more (whole tokens at H = 7168
  // in the 16-wave shape), which frees registers for the reads
  const int seg_vec = combine_phase_seg(b, row_vec, k);
  const int cus = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  const PhaseShape ps = combine_phase_shape(row_vec, seg_vec, cus, b.all_cus, T);
  const bool even = row_vec % kWave == 0 && (int64_t)ps.nv * kWave <= row_vec;  // no padded column
  const int unit_vec = ps.nseg == 1 ? ps.tpu * ps.nv : ps.seg;
  const int held = ps.held == kPhaseWideHeld ? kPhaseWideHeld : unit_vec <= 14 ? 14 : 16;
  PhaseFn fn = even ? pick_phase<true>(seg_vec, held, k) : pick_phase<false>(seg_vec, held, k);
  if (!fn) return hipErrorInvalidValue;
  const size_t lds_bytes = b.num_cus > 0 ? kExclusiveLds : 0;
  if (lds_bytes > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds_bytes);
    if (e != hipSuccess) return e;
  }
  // One launch per batch of tokens that gives every wave of the grid one
  // unit: the launch boundary keeps the read and write phases of the
  // batches apart, which waves that loop over several units would not.
  // Batches are of equal size, and a batch spreads over every CU with as
  // few waves per workgroup as it needs (a small last batch on a few full
  // CUs measured 7% slower at 192 CUs).
  const int64_t batch = phase_batch(ps, T, cus);
  for (int64_t t0 = 0; t0 < T;) {
    const int tb = (int)(T - t0 < batch ? T - t0 : batch);
    const int units = (int)phase_units(ps, tb);
    int grid = units < cus ? units : cus;
    if (grid < 1) grid = 1;
    const int wpg = (units + grid - 1) / grid;  // <= ps.wpg
    hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(y),
                       static_cast<u32x4*>(out) + t0 * row_vec, dest_row + t0 * k, w + t0 * k, recv_rows, row_vec,
                       ps.nv, tb, ps.tpu, ps.nseg, ps.seg, units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    t0 += tb;
  }
  return hipSuccess;
}

// The phase kernel is the default on at least half the device when each
// of its launches gives enough of the waves of a full grid a unit: it reads
// all rows of its unit before its first store, so a wave with little work
// gains nothing (decode batches stay on the register kernel), and on fewer
// CUs the per-CU read rate, not the read/write turnaround, is the bound.
// Cold single calls against the register kernel, every CU, two runs each:
//  - two or three rows per wave in 8-wave workgroups (k >= 6 at H = 4104
//    .. 7168): two thirds at k = 6, seven tenths at k = 8.  H = 4608,
//    5120, 6144, 7168: k = 6 at 67% 5-9% faster, at 60% 1-5% slower; k = 8
//    at 67% 2-6% slower, at 70-73% between 3% faster and 3% slower (slower
//    only at H = 5120), from 80% 4-12% faster;
//  - the 16-wave shape at k >= 4: nine twentieths.  H = 2048, 3072, 4096
//    and k = 4, 6, 8 at 45-65%: 3-11% faster in every case; at 37.5%, k = 4
//    3-6% slower (H = 1024, 2048, 7168);
//  - the 16-wave shape at k = 2: three fifths.  At 55% 0.4% faster to 3.5%
//    slower, at 60% 1% slower (H = 3072) to 4% faster, from 62.5% 2-5%
//    faster (H = 1024 .. 7168).
// Odd k: at a full launch the phased kernel is 3-16% faster than the any-k
// register kernel at k = 1, 3, 5, 7 (H = 4096 and 7168; k = 7, H = 7168,
// T = 16384: 293.0 against 347.1 us).  In the 16-wave shape odd k takes the
// rule of the even k above it (k = 1 that of k = 2; k = 1 wins from 50%,
// k = 3 from 47%, k = 5 and 7 from 40-47%).  In the two-row shape, whose
// register sets split unevenly at odd k: k = 5 from 23/25 (H = 5120 and
// 7168: 0-1.5% slower at 90%, 4% faster at 95%, 10-16% slower at 67-75%),
// k = 7 from three quarters (4-8% slower at 67-72%, 3% faster at 80%).  On part of the device (128-192 CUs) the rule
// stays at two thirds.  At k <= 4 the kernel needs runs of 2 vectors per
// read (see combine_phase_seg): with single vectors the register kernel was
// 11-20% faster at k = 2 and 4.
bool phase_preferred(const Budget& b, int row_vec, int T, int k) {
  if (k < 1 || k > 8) return false;
  const int cus = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  if (2 * cus < b.all_cus) return false;
  const int seg_vec = combine_phase_seg(b, row_vec, k);
  if (k <= 4 && seg_vec != 2) return false;
  const PhaseShape ps = combine_phase_shape(row_vec, seg_vec, cus, b.all_cus, T);
  const int64_t units = phase_units(ps, phase_batch(ps, T, cus));  // the largest launch's
  const int64_t slots = (int64_t)cus * ps.wpg;
  if (cus >= b.all_cus && ps.held != kPhaseWideHeld) return k <= 2 ? units * 5 >= slots * 3 : units * 20 >= slots * 9;
  if (ps.held == kPhaseWideHeld) {
    if (k == 5) return units * 25 >= slots * 23;
    if (k == 7) return units * 4 >= slots * 3;
    if (k == 8) return units * 10 >= slots * 7;
  }
  return units * 3 >= slots * 2;
}

using CombineFn = void (*)(const u32x4*, u32x4*, const int32_t*, const float*, int64_t, int, int, int, int);

template <int VPL, int K, bool EVEN>
CombineFn pick_kind(Variant v) {
  switch (v) {
    case Variant::Vgpr: return combine_vgpr_kernel<VPL, K, EVEN, true>;
    case Variant::VgprCached: return combine_vgpr_kernel<VPL, K, EVEN, false>;
    default: break;
  }
  if constexpr (VPL == 1) {
    switch (v) {
      case Variant::Vgpr2: return combine_vgpr2_kernel<VPL, K, EVEN, true>;
      case Variant::Lds1: return combine_lds1_kernel<VPL, K, EVEN, true>;
      case Variant::Lds2: return combine_lds2_kernel<VPL, K, EVEN, true>;
      default: break;
    }
  }
  return nullptr;
}

template <int VPL, bool EVEN>
CombineFn pick_k(Variant v, int k) {
  switch (k) {
    case 2: return pick_kind<VPL, 2, EVEN>(v);
    case 4: return pick_kind<VPL, 4, EVEN>(v);
    case 6: return pick_kind<VPL, 6, EVEN>(v);
    case 8: return pick_kind<VPL, 8, EVEN>(v);
    default: return combine_vgpr_any_kernel<VPL, EVEN, true>;
  }
}

template <bool EVEN>
CombineFn pick_vpl(Variant v, int vpl, int k) {
  switch (vpl) {
    case 1: return pick_k<1, EVEN>(v, k);
    case 2: return pick_k<2, EVEN>(v, k);
    default: return pick_k<4, EVEN>(v, k);
  }
}

// An empty receive buffer leaves every slot of every token out of range, and
// the sum of no terms is +0.0: out is filled with zeros and y, which may then
// be NULL, is never read.  (The phased kernel's loads are unconditional and
// read row 0 for out-of-range slots, so it must not run on an empty buffer.)
__global__ __launch_bounds__(1024) void combine_zero_kernel(u32x4* __restrict__ out, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) st16<true>(out + i, z);
}

hipError_t launch_combine_zero(const Budget& b, void* out, int64_t nvec, hipStream_t stream) {
  int grid;
  size_t lds_bytes = 0;
  if (b.num_cus > 0) {
    // the budget's persistent grid: one workgroup per CU
    grid = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    lds_bytes = kExclusiveLds;
    hipError_t e = allow_dynamic_lds((const void*)combine_zero_kernel, lds_bytes);
    if (e != hipSuccess) return e;
  } else {
    const int64_t want = (nvec + 1023) / 1024;
    grid = (int)(want < (int64_t)b.device_cus * 4 ? want : (int64_t)b.device_cus * 4);
  }
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(combine_zero_kernel, dim3(grid), dim3(1024), lds_bytes, stream, static_cast<u32x4*>(out), nvec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(Variant v, const Budget& b, const void* y, int64_t recv_rows, int H,
                          const int32_t* dest_row, const float* w, int T, int k, void* out, hipStream_t stream) {
  const int row_vec = H / 8;
  if (recv_rows == 0) return launch_combine_zero(b, out, (int64_t)T * row_vec, stream);
  if (v == Variant::Lds3 || v == Variant::Pc || v == Variant::VgprWg) v = Variant::Auto;  // dispatch-only variants
  if (v == Variant::Auto) v = phase_preferred(b, row_vec, T, k) ? Variant::Phase : Variant::Vgpr;
  if (v == Variant::Phase && k >= 1 && k <= 8)
    return launch_phase(b, y, recv_rows, row_vec, dest_row, w, T, k, out, stream);
  const bool known_k = (k == 2 || k == 4 || k == 6 || k == 8);
  if (!known_k) v = Variant::Vgpr;  // the any-k kernel
  const bool even = row_vec % kWave == 0;
  // in-flight registers grow as k x VPL: two vectors per lane per slot for
  // the single-set kernel, one for the double-buffered and LDS ones
  const bool single = (v == Variant::Vgpr || v == Variant::VgprCached);
  int vpl = single ? 2 : 1;
  if (single && b.slab_vpl > 0) vpl = b.slab_vpl >= 4 ? 4 : b.slab_vpl >= 2 ? 2 : 1;
  // A batch too small to give every CU of an ordinary grid four waves at 2
  // vectors per lane (decode) takes 1-vector slabs: twice the waves, each
  // with half the work (T = 128, H = 7168, k = 8: 4.08 against 3.71 TB/s;
  // at T = 1024 the 2-vector slabs stay ahead, 6.02 against 5.81).
  if (single && b.slab_vpl == 0 && b.num_cus == 0 &&
      (int64_t)T * ((row_vec + 2 * kWave - 1) / (2 * kWave)) < 4 * (int64_t)b.device_cus)
    vpl = 1;
  // On a CU budget, k = 2..7 read 4 vectors per lane per slot (8 waves per
  // CU): H = 7168, k = 3 and 5 on 24 CUs 1.25 and 1.30 against 1.14 and
  // 1.17 TB/s, k = 4 on 64 CUs 3.15 against 3.00; k = 1 and 8 keep 2
  // (4-vector slabs cost them 3-10%).
  if (single && b.slab_vpl == 0 && b.num_cus > 0 && k >= 2 && k <= 7) vpl = 4;
  // On a budget, batches of up to 32 tokens per CU take 1-vector slabs: more
  // units for the budget's 16 waves per CU.  Cold, us, against the slabs
  // above, 24 and 64 CUs, 0.5 to 64 tokens per CU: H = 7168, k = 8 7.8
  // against 11.0 (24 CUs, T = 24), 24.4 against 28.1 (T = 192), equal from
  // 32 per CU; k = 4 6.6 against 8.2 (T = 24), 1-6% faster up to 64 per CU;
  // H = 4096, k = 6 9.5 against 10.6 (T = 96), 38.7 against 40.5 (T = 768),
  // 1.5% slower at 64 per CU (64 CUs, T = 4096).
  if (single && b.slab_vpl == 0 && b.num_cus > 0 &&
      (int64_t)T <= 32LL * (b.num_cus < b.device_cus ? b.num_cus : b.device_cus))
    vpl = 1;
  if (row_vec <= kWave) vpl = 1;
  const int max_wpg = (single && vpl >= 4) ? 8 : 16;
  const int nslab = (row_vec + vpl * kWave - 1) / (vpl * kWave);
  if ((int64_t)T * nslab > INT32_MAX) return hipErrorInvalidValue;
  const int units = T * nslab;
  CombineFn fn = even ? pick_vpl<true>(v, vpl, k) : pick_vpl<false>(v, vpl, k);
  if (!fn) return hipErrorInvalidValue;

  const bool lds = (v == Variant::Lds1 || v == Variant::Lds2);
  const size_t per_wave = lds ? (size_t)(v == Variant::Lds2 ? 2 : 1) * k * vpl * kWaveVecBytes : 0;
  int wpg, grid;
  size_t lds_bytes;
  if (b.num_cus > 0) {
    wpg = max_wpg;
    if (per_wave && (int)(kLdsPerCu / per_wave) < wpg) wpg = (int)(kLdsPerCu / per_wave);
    grid = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    lds_bytes = per_wave * wpg;
    if (lds_bytes < kExclusiveLds) lds_bytes = kExclusiveLds;
  } else {
    wpg = 4;
    int per_cu = per_wave ? (int)(kLdsPerCu / (per_wave * wpg)) : 8;
    if (per_cu > 8) per_cu = 8;
    if (per_cu < 1) per_cu = 1;
    grid = (units + wpg - 1) / wpg;
    if (grid > b.device_cus * per_cu) grid = b.device_cus * per_cu;
    lds_bytes = per_wave * wpg;
  }
  if (grid < 1) grid = 1;
  if (lds_bytes > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(y),
                     static_cast<u32x4*>(out), dest_row, w, recv_rows, row_vec, nslab, k, units);
  return hipGetLastError();
}

}  // namespace ep
