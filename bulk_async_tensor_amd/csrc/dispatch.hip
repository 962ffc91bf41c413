// ep_dispatch: recv[dest_row[t, j], :] = x[t, :] -- every token row is read
// from HBM once and written to its k destinations.
//
// This is the receive-side row copy of [DeepEP-TMA] section "Asynchronous
// Copy Primitives" re-thought for CDNA4.  There, one elected lane per warp
// hands a half row to the bulk-copy engine, waits on a transaction barrier
// and hands the shared-memory slice back for the store.  gfx950 has no
// bulk-copy engine: the wave itself is the issuing unit, and one wave
// instruction moves 1 KiB (64 lanes x 16 bytes).  The kernels differ in where
// a row waits between its load and its k stores:
//
//   vgpr   registers: VPL dwordx4 loads, then k x VPL dwordx4 stores;
//   vgpr2  registers, two sets: the next unit's loads are issued before the
//          current unit's stores;
//   lds1   a per-wave LDS slice filled by direct-to-LDS loads
//          (global_load_lds_dwordx4, no VGPR staging), one stage: load, wait,
//          read the slice, store -- the single-slice loop of the pages;
//   lds2   the same slice doubled: the next unit's direct-to-LDS load is in
//          flight while the current one is read out and stored.
//
// A work unit is (token, slab), a slab being up to VPL x 64 16-byte vectors
// of the row (VPL KiB).  Waves take units round-robin; wave-uniform values
// (unit, token, destination rows) live in SGPRs, and the k destination rows
// of a unit are fetched with one scalar load before its first store.
// EVEN = the row is a whole number of KiB, so no lane ever falls off the row
// end and no per-lane masks are needed.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "row_io.hpp"

namespace ep {

namespace {

template <int K>
struct Dests {
  int32_t d[K > 0 ? K : 1];
};

template <int K>
__device__ __forceinline__ void fetch_dests(Dests<K>& ds, const int32_t* __restrict__ dr) {
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) ds.d[j] = dr[j];
  }
}

// Stores of one slab to its destinations.  Returns the number of store
// instructions issued (valid destinations x vectors; lane 0 is inside the
// row for every vector < nvec, so none is skipped), which bounds the
// completion wait of the two-stage ring.
template <int VPL, int K, bool EVEN, bool NT>
__device__ __forceinline__ int store_slab(const u32x4 (&v)[VPL], u32x4* __restrict__ recv, const Dests<K>& ds,
                                          const int32_t* __restrict__ dr, int k, int64_t recv_rows, const Unit& un,
                                          int row_vec) {
  int ndest = 0;
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t d = ds.d[j];
      if ((uint64_t)d < (uint64_t)recv_rows) {
        ++ndest;
        store_one<VPL, EVEN, NT>(v, recv + d * row_vec, un, row_vec);
      }
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int64_t d = dr[j];
      if ((uint64_t)d < (uint64_t)recv_rows) {
        ++ndest;
        store_one<VPL, EVEN, NT>(v, recv + d * row_vec, un, row_vec);
      }
    }
  }
  return ndest * un.nvec;
}

#define EP_DISPATCH_ARGS                                                                                     \
  const u32x4 *__restrict__ x, u32x4 *__restrict__ recv, const int32_t *__restrict__ dest_row, int64_t recv_rows, \
      int row_vec, int nslab, int k_rt, int units

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_vgpr_kernel(EP_DISPATCH_ARGS) {
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  for (int u = blockIdx.x * wpg + wave_in_group(); u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    const int32_t* dr = dest_row + un.t * k;
    Dests<K> ds;
    fetch_dests<K>(ds, dr);
    u32x4 v[VPL];
    load_slab<VPL, EVEN, NT>(v, x + un.t * row_vec, un, row_vec);
    store_slab<VPL, K, EVEN, NT>(v, recv, ds, dr, k, recv_rows, un, row_vec);
  }
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_vgpr2_kernel(EP_DISPATCH_ARGS) {
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  int u = blockIdx.x * wpg + wave_in_group();
  if (u >= units) return;
  Unit cur = unit_of<VPL>(u, nslab, row_vec, lane);
  Dests<K> dcur, dnxt;
  fetch_dests<K>(dcur, dest_row + cur.t * k);
  u32x4 a[VPL], b[VPL];
  load_slab<VPL, EVEN, NT>(a, x + cur.t * row_vec, cur, row_vec);
  for (;;) {
    // two units per trip so that the register sets swap roles without moves
    int un = u + stride;
    Unit nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (un < units) {
      fetch_dests<K>(dnxt, dest_row + nxt.t * k);
      load_slab<VPL, EVEN, NT>(b, x + nxt.t * row_vec, nxt, row_vec);
    }
    store_slab<VPL, K, EVEN, NT>(a, recv, dcur, dest_row + cur.t * k, k, recv_rows, cur, row_vec);
    if (un >= units) break;
    u = un;
    cur = nxt;
    un = u + stride;
    nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (un < units) {
      fetch_dests<K>(dcur, dest_row + nxt.t * k);
      load_slab<VPL, EVEN, NT>(a, x + nxt.t * row_vec, nxt, row_vec);
    }
    store_slab<VPL, K, EVEN, NT>(b, recv, dnxt, dest_row + cur.t * k, k, recv_rows, cur, row_vec);
    if (un >= units) break;
    u = un;
    cur = nxt;
  }
}

// The register kernel with each workgroup reading in step: every wave loads
// wg_units<VPL>() units and waits for them (and for their destination rows),
// then the workgroup meets at a barrier before any wave stores.  A CU's loads
// queue behind its own stores in its memory pipeline; the barrier keeps a
// CU's reads out of that queue, and a few long read and write bursts per CU
// (four whole rows per wave in workgroups of four waves) beat many short
// ones.  Every wave makes the workgroup's trip count, so each barrier is met
// by all of its waves.
template <int VPL>
constexpr int wg_units() {
  return wg_units_of(VPL);
}

// Loads of one slab for the workgroup-phased kernel, every one issued.  A row
// that is a whole number of KiB needs no per-lane clamp: vectors past the
// slab re-read the slab's last vector (a uniform offset), so one base address
// per wave serves every load.  Other rows clamp per lane as load_slab_fixed.
template <int VPL, bool EVEN, bool NT>
__device__ __forceinline__ void load_slab_wg(u32x4 (&v)[VPL], const u32x4* __restrict__ src, const Unit& un,
                                             int row_vec) {
  if constexpr (EVEN) {
    const u32x4* p = src + un.c0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int ii = i < un.nvec ? i : un.nvec - 1;
      v[i] = ld16<NT>(p + ii * kWave);
    }
  } else {
    load_slab_fixed<VPL, NT>(v, src, un, row_vec);
  }
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(kWgWaves * kWave) void dispatch_wg_kernel(EP_DISPATCH_ARGS) {
  constexpr int U = wg_units<VPL>();
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  const int first = blockIdx.x * wpg;
  if (first >= units) return;  // the same for every wave of the workgroup
  const int per_trip = stride * U;
  const int trips = (units - first + per_trip - 1) / per_trip;
  for (int r = 0; r < trips; ++r) {
    Unit un[U];
    bool live[U];
    Dests<K> ds[U];
    u32x4 v[U][VPL];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int u = first + (r * U + q) * stride + wave_in_group();
      live[q] = u < units;
      un[q] = unit_of<VPL>(live[q] ? u : first, nslab, row_vec, lane);
      load_slab_wg<VPL, EVEN, NT>(v[q], x + un[q].t * row_vec, un[q], row_vec);
      fetch_dests<K>(ds[q], dest_row + un[q].t * k);
    }
    // The barrier and wait builtins do not stop the compiler from sinking
    // loads below them, towards their first use: tying every loaded register
    // and destination row to this point keeps all of them above the barrier
    // (a destination fetched after it would delay the first store by a
    // memory round trip).
#pragma unroll
    for (int q = 0; q < U; ++q) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) asm volatile("" : "+v"(v[q][i]));
      if constexpr (K > 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) asm volatile("" : "+s"(ds[q].d[j]));
      }
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < U; ++q)
      if (live[q]) store_slab<VPL, K, EVEN, NT>(v[q], recv, ds[q], dest_row + un[q].t * k, k, recv_rows, un[q], row_vec);
  }
}


template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_lds1_kernel(EP_DISPATCH_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  char* slice = lds + wave * (VPL * kWaveVecBytes);
  for (int u = blockIdx.x * wpg + wave; u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);
    const int32_t* dr = dest_row + un.t * k;
    Dests<K> ds;
    fetch_dests<K>(ds, dr);
    dma_slab<VPL, EVEN>(x + un.t * row_vec, slice, un, row_vec);
    wait_vmcnt<0>();  // slice filled (this also drains the previous unit's stores)
    u32x4 v[VPL];
    read_slab<VPL>(v, slice, lane);
    store_slab<VPL, K, EVEN, NT>(v, recv, ds, dr, k, recv_rows, un, row_vec);
  }
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_lds2_kernel(EP_DISPATCH_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  static_assert(K > 0, "the two-stage ring needs a compile-time k for its wait counts");
  // stores issued after a stage's fill when the previous unit was complete
  constexpr int kFullStores = (K * VPL) < 63 ? (K * VPL) : 63;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  char* ring = lds + wave * (2 * VPL * kWaveVecBytes);
  int u = blockIdx.x * wpg + wave;
  if (u >= units) return;
  Unit cur = unit_of<VPL>(u, nslab, row_vec, lane);
  Dests<K> dcur, dnxt;
  fetch_dests<K>(dcur, dest_row + cur.t * K);
  dma_slab<VPL, EVEN>(x + cur.t * row_vec, ring, cur, row_vec);
  int stage = 0;
  int issued_after = 0;  // vector-memory instructions issued after the pending fill of `stage`
  for (;;) {
    // wait for the fill of `stage`: vmcnt retires in issue order, so letting
    // at most `issued_after` newer operations stay outstanding is exact
    if (issued_after >= kFullStores) wait_vmcnt<kFullStores>();
    else wait_vmcnt<0>();
    u32x4 v[VPL];
    read_slab<VPL>(v, ring + stage * (VPL * kWaveVecBytes), lane);  // stage is free again
    const int un = u + stride;
    const bool more = un < units;
    const Unit nxt = unit_of<VPL>(un, nslab, row_vec, lane);
    if (more) {
      fetch_dests<K>(dnxt, dest_row + nxt.t * K);
      dma_slab<VPL, EVEN>(x + nxt.t * row_vec, ring + (stage ^ 1) * (VPL * kWaveVecBytes), nxt, row_vec);
    }
    issued_after = store_slab<VPL, K, EVEN, NT>(v, recv, dcur, nullptr, K, recv_rows, cur, row_vec);
    if (!more) break;
    u = un;
    cur = nxt;
    dcur = dnxt;
    stage ^= 1;
  }
}

// Three stages per wave: the fills of the next two units are in flight while
// the current one is read out and stored.  A deeper ring costs LDS, so fewer
// waves fit a CU (3 x 7 KiB per wave at H = 7168: 7 waves).  The wait for a
// stage's fill lets the operations issued after it stay outstanding, up to
// vmcnt's limit of 63 (past it the wait also retires the oldest stores,
// which is still correct).  The ring is unrolled by three so that every stage
// index is a compile-time constant and the per-stage state stays in
// registers.
template <int VPL, int K>
struct Ring3 {
  Unit un[3];
  Dests<K> ds[3];
  int after[3];  // vector-memory operations issued since the pending fill of each stage
};

template <int S, int VPL, int K, bool EVEN, bool NT>
__device__ __forceinline__ bool lds3_step(Ring3<VPL, K>& r, int& u, char* ring, const u32x4* __restrict__ x,
                                          u32x4* __restrict__ recv, const int32_t* __restrict__ dest_row,
                                          int64_t recv_rows, int row_vec, int nslab, int units, int stride,
                                          int lane) {
  constexpr int kStage = VPL * kWaveVecBytes;
  // steady state after a stage's fill: the stores of the two units before it
  // and the fill of the unit after it
  constexpr int kSteady = 2 * K * VPL + VPL;
  constexpr int kCap = kSteady < 63 ? kSteady : 63;
  constexpr int S1 = (S + 1) % 3, S2 = (S + 2) % 3;
  if (r.after[S] >= kCap) wait_vmcnt<kCap>();
  else wait_vmcnt<0>();
  u32x4 v[VPL];
  read_slab<VPL>(v, ring + S * kStage, lane);  // stage S is free again
  const int u2 = u + 2 * stride;
  const bool fill = u2 < units;
  if (fill) {
    r.un[S2] = unit_of<VPL>(u2, nslab, row_vec, lane);
    fetch_dests<K>(r.ds[S2], dest_row + r.un[S2].t * K);
    dma_slab<VPL, EVEN>(x + r.un[S2].t * row_vec, ring + S2 * kStage, r.un[S2], row_vec);
    r.after[S1] += r.un[S2].nvec;  // the next stage's fill is older than this one
    r.after[S2] = 0;
  }
  const int st = store_slab<VPL, K, EVEN, NT>(v, recv, r.ds[S], nullptr, K, recv_rows, r.un[S], row_vec);
  r.after[S1] += st;
  if (fill) r.after[S2] += st;
  u += stride;
  return u < units;
}

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_lds3_kernel(EP_DISPATCH_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  static_assert(K > 0, "the three-stage ring needs a compile-time k for its wait counts");
  constexpr int kStage = VPL * kWaveVecBytes;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  char* ring = lds + wave * (3 * kStage);
  int u = blockIdx.x * wpg + wave;
  if (u >= units) return;
  Ring3<VPL, K> r;
  r.after[0] = r.after[1] = r.after[2] = 0;
  r.un[0] = unit_of<VPL>(u, nslab, row_vec, lane);
  fetch_dests<K>(r.ds[0], dest_row + r.un[0].t * K);
  dma_slab<VPL, EVEN>(x + r.un[0].t * row_vec, ring, r.un[0], row_vec);
  if (u + stride < units) {
    r.un[1] = unit_of<VPL>(u + stride, nslab, row_vec, lane);
    fetch_dests<K>(r.ds[1], dest_row + r.un[1].t * K);
    dma_slab<VPL, EVEN>(x + r.un[1].t * row_vec, ring + kStage, r.un[1], row_vec);
    r.after[0] = r.un[1].nvec;
  }
  for (;;) {
    if (!lds3_step<0, VPL, K, EVEN, NT>(r, u, ring, x, recv, dest_row, recv_rows, row_vec, nslab, units, stride,
                                        lane))
      break;
    if (!lds3_step<1, VPL, K, EVEN, NT>(r, u, ring, x, recv, dest_row, recv_rows, row_vec, nslab, units, stride,
                                        lane))
      break;
    if (!lds3_step<2, VPL, K, EVEN, NT>(r, u, ring, x, recv, dest_row, recv_rows, row_vec, nslab, units, stride,
                                        lane))
      break;
  }
}

// Producer/consumer specialisation: wave 0 of each workgroup only issues the
// direct-to-LDS fills for the W consumer waves (the "elected" issuer of
// [DeepEP-TMA] "Asynchronous Copy Primitives", made a whole wave because a
// wave instruction is the unit of issue here); consumers only read their
// slab out and store it k times.  Two slots of W slabs: the producer fills
// slot (i + 1) & 1 while the consumers store round i.  Synchronisation is two
// workgroup barriers per round and no polling: barrier A follows the
// producer's wait for the round's fill, barrier B the consumers' reads of the
// slot.  Every fill issues exactly W x VPL loads (units past the end re-read
// unit 0, lanes past a ragged row end its last vector), so the producer's
// wait for the older fill is exact.
template <int VPL>
constexpr int pc_consumers() {
  return 63 / VPL < 8 ? 63 / VPL : 8;
}

inline int pc_consumers_host(int vpl) { return 63 / vpl < 8 ? 63 / vpl : 8; }

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int VPL, int K, bool EVEN, bool NT>
__global__ __launch_bounds__(1024) void dispatch_pc_kernel(EP_DISPATCH_ARGS) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int W = pc_consumers<VPL>();
  constexpr int kSlot = W * VPL * kWaveVecBytes;
  const int k = K > 0 ? K : k_rt;
  const int lane = lane_id();
  const int wave = wave_in_group();
  const int G = gridDim.x;
  const int per_round = G * W;
  const int rounds = (units + per_round - 1) / per_round;
  if (wave == 0) {
    // producer
    auto fill = [&](int i) {
      char* slot = lds + (i & 1) * kSlot;
#pragma unroll
      for (int c = 0; c < W; ++c) {
        const int uc = (i * G + (int)blockIdx.x) * W + c;
        const Unit un = unit_of<VPL>(uc < units ? uc : 0, nslab, row_vec, lane);
        const u32x4* src = x + un.t * row_vec;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          int col = un.c0 + v * kWave;
          if (col >= row_vec) col = row_vec - 1;
          dma16(src + col, (lds_void_t*)(slot + (c * VPL + v) * kWaveVecBytes));
        }
      }
    };
    if (rounds > 0) fill(0);
    for (int i = 0; i < rounds; ++i) {
      if (i + 1 < rounds) {
        fill(i + 1);
        wait_vmcnt<W * VPL>();  // fill i done; fill i + 1 stays in flight
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier();  // A: slot i & 1 is full
      wg_barrier();  // B: the consumers have read it
    }
    return;
  }
  // consumer c
  const int c = wave - 1;
  for (int i = 0; i < rounds; ++i) {
    const int u = (i * G + (int)blockIdx.x) * W + c;
    const bool ok = u < units;
    const Unit un = unit_of<VPL>(ok ? u : 0, nslab, row_vec, lane);
    const int32_t* dr = dest_row + un.t * k;
    Dests<K> ds;
    fetch_dests<K>(ds, dr);
    wg_barrier();  // A
    u32x4 v[VPL];
    read_slab<VPL>(v, lds + (i & 1) * kSlot + c * VPL * kWaveVecBytes, lane);
    wg_barrier();  // B
    if (ok) store_slab<VPL, K, EVEN, NT>(v, recv, ds, dr, k, recv_rows, un, row_vec);
  }
}

using DispatchFn = void (*)(const u32x4*, u32x4*, const int32_t*, int64_t, int, int, int, int);

template <int VPL, int K, bool EVEN>
DispatchFn pick_kind(Variant v) {
  switch (v) {
    case Variant::Vgpr: return dispatch_vgpr_kernel<VPL, K, EVEN, true>;
    case Variant::VgprCached: return dispatch_vgpr_kernel<VPL, K, EVEN, false>;
    case Variant::Lds1: return dispatch_lds1_kernel<VPL, K, EVEN, true>;
    case Variant::Pc: return dispatch_pc_kernel<VPL, K, EVEN, true>;
    case Variant::VgprWg: return dispatch_wg_kernel<VPL, K, EVEN, true>;
    default: break;
  }
  // the register double buffer holds two slabs: compiled up to 14 vectors
  // per lane (124 VGPRs at k = 8, no spills; 16 spill)
  if constexpr (VPL <= 14) {
    if (v == Variant::Vgpr2) return dispatch_vgpr2_kernel<VPL, K, EVEN, true>;
  }
  // the LDS rings hold two or three slabs: compiled up to 8 vectors per lane
  if constexpr (VPL <= 8) {
    if constexpr (K > 0) {
      if (v == Variant::Lds2) return dispatch_lds2_kernel<VPL, K, EVEN, true>;
      if (v == Variant::Lds3) return dispatch_lds3_kernel<VPL, K, EVEN, true>;
    }
  }
  return nullptr;
}

template <int VPL, bool EVEN>
DispatchFn pick_k(Variant v, int k) {
  switch (k) {
    case 2: return pick_kind<VPL, 2, EVEN>(v);
    case 4: return pick_kind<VPL, 4, EVEN>(v);
    case 6: return pick_kind<VPL, 6, EVEN>(v);
    case 8: return pick_kind<VPL, 8, EVEN>(v);
    default: return pick_kind<VPL, 0, EVEN>(v);
  }
}

template <bool EVEN>
DispatchFn pick_vpl(Variant v, int vpl, int k) {
  switch (vpl) {
    case 2: return pick_k<2, EVEN>(v, k);
    case 4: return pick_k<4, EVEN>(v, k);
    case 7: return pick_k<7, EVEN>(v, k);
    case 8: return pick_k<8, EVEN>(v, k);
    case 14: return pick_k<14, EVEN>(v, k);
    default: return pick_k<16, EVEN>(v, k);
  }
}

constexpr int kSlabChoices[] = {2, 4, 7, 8, 14, 16};

// Vectors per lane per slab.  Default: the whole row when it is at most
// `cap` vectors per lane (rows then leave a wave as one contiguous burst per
// destination), else the largest choice that splits the row evenly, else
// `cap` with a ragged last slab.  A requested size is rounded down to a
// compiled choice.
int choose_vpl(int row_vec, int cap, int requested) {
  const int vpr = (row_vec + kWave - 1) / kWave;
  if (requested > 0) {
    int best = 2;
    for (int c : kSlabChoices)
      if (c <= requested && c <= cap) best = c;
    return best;
  }
  for (int c : kSlabChoices)
    if (c >= vpr && c <= cap) return c;
  for (int i = (int)(sizeof(kSlabChoices) / sizeof(int)) - 1; i >= 0; --i)
    if (kSlabChoices[i] <= cap && vpr % kSlabChoices[i] == 0) return kSlabChoices[i];
  return cap;
}

// Gather form of the same copy: recv[r, :] = x[src_token[r], :].  Waves take
// (receive row, slab) units in order, so the receive buffer is written as
// one sequential stream; each token row is read k times, mostly from the
// caches (x is 58.7 MB at the training shape, below the 256 MB Infinity
// Cache).  CL = true keeps the x loads cacheable.
template <int VPL, bool EVEN, bool CL>
__global__ __launch_bounds__(1024) void dispatch_rows_kernel(const u32x4* __restrict__ x, u32x4* __restrict__ recv,
                                                            const int32_t* __restrict__ src_token, int T,
                                                            int row_vec, int nslab, int units) {
  const int lane = lane_id();
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  for (int u = blockIdx.x * wpg + wave_in_group(); u < units; u += stride) {
    const Unit un = unit_of<VPL>(u, nslab, row_vec, lane);  // un.t is the receive row here
    const int t = src_token[un.t];
    if ((unsigned)t >= (unsigned)T) continue;
    u32x4 v[VPL];
    load_slab<VPL, EVEN, !CL>(v, x + (int64_t)t * row_vec, un, row_vec);
    store_one<VPL, EVEN, true>(v, recv + un.t * row_vec, un, row_vec);
  }
}

using RowsFn = void (*)(const u32x4*, u32x4*, const int32_t*, int, int, int, int);

template <bool EVEN, bool CL>
RowsFn rows_pick(int vpl) {
  switch (vpl) {
    case 2: return dispatch_rows_kernel<2, EVEN, CL>;
    case 4: return dispatch_rows_kernel<4, EVEN, CL>;
    case 7: return dispatch_rows_kernel<7, EVEN, CL>;
    case 8: return dispatch_rows_kernel<8, EVEN, CL>;
    case 14: return dispatch_rows_kernel<14, EVEN, CL>;
    default: return dispatch_rows_kernel<16, EVEN, CL>;
  }
}

// The phased dispatch: a wave's unit is up to 16 KiB of source rows (one
// token at H = 7168).  It reads them all into registers first, with every
// load in flight together, and then writes the k copies.  With one unit per
// wave on every CU, the whole grid reads x first and writes last, so the
// reads never queue behind the writes: the dispatch costs the same whether
// x is still in the caches or not (the staged kernels wait on each unit's
// read under full write traffic and are twice as slow when x is not).
template <int K, bool EVEN>
__global__ __launch_bounds__(1024) void dispatch_phase_kernel(const u32x4* __restrict__ x, u32x4* __restrict__ recv,
                                                              const int32_t* __restrict__ dest_row,
                                                              int64_t recv_rows, int row_vec, int nv, int T, int tpu,
                                                              int nseg, int seg, int units) {
  constexpr int HELD = kPhaseHeld;
  const int lane = lane_id();
  const int stride = gridDim.x * (blockDim.x >> 6);
  for (int u = blockIdx.x * (blockDim.x >> 6) + wave_in_group(); u < units; u += stride) {
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
    const int span = nseg == 1 ? nv : n_in;
    // rotated start per unit, as in the phased combine
    const int rot = u % span;
    // Straight-line loads: vectors past the unit re-read the unit's first
    // vector, lanes past a ragged row end its last; neither is stored.
    u32x4 held[HELD];
    {
      int t = t0, p = 0, c = c0 + rot;
#pragma unroll
      for (int i = 0; i < HELD; ++i) {
        const bool in = i < n_in;
        int col = (in ? c : c0 + rot) * kWave + lane;
        if (!EVEN && col >= row_vec) col = row_vec - 1;
        held[i] = ld16<false>(x + (int64_t)(in ? t : t0) * row_vec + col);
        if (in) {
          if (++c == c0 + span) c = c0;
          if (++p == span) {
            p = 0;
            ++t;
          }
        }
      }
    }
    int t = t0, p = 0, c = c0 + rot;
    Dests<K> ds;
    fetch_dests<K>(ds, dest_row + (int64_t)t * K);
#pragma unroll
    for (int i = 0; i < HELD; ++i) {
      if (i < n_in) {
        if (i > 0 && p == 0) fetch_dests<K>(ds, dest_row + (int64_t)t * K);
        const int col = c * kWave + lane;
        if (EVEN || col < row_vec) {
#pragma unroll
          for (int j = 0; j < K; ++j) {
            const int64_t d = ds.d[j];
            if ((uint64_t)d < (uint64_t)recv_rows) st16<true>(recv + d * row_vec + col, held[i]);
          }
        }
        if (++c == c0 + span) c = c0;
        if (++p == span) {
          p = 0;
          ++t;
        }
      }
    }
  }
}

using PhaseDispatchFn = void (*)(const u32x4*, u32x4*, const int32_t*, int64_t, int, int, int, int, int, int, int);

template <bool EVEN>
PhaseDispatchFn pick_phase_dispatch(int k) {
  switch (k) {
    case 2: return dispatch_phase_kernel<2, EVEN>;
    case 4: return dispatch_phase_kernel<4, EVEN>;
    case 6: return dispatch_phase_kernel<6, EVEN>;
    case 8: return dispatch_phase_kernel<8, EVEN>;
    default: return nullptr;
  }
}

hipError_t launch_dispatch_phase(const Budget& b, const void* x, int T, int row_vec, const int32_t* dest_row, int k,
                                 void* recv, int64_t recv_rows, hipStream_t stream) {
  const bool even = row_vec % kWave == 0;
  const PhaseShape ps = phase_shape(row_vec);
  PhaseDispatchFn fn = even ? pick_phase_dispatch<true>(k) : pick_phase_dispatch<false>(k);
  if (!fn) return hipErrorInvalidValue;
  const int cus = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  const size_t lds_bytes = b.num_cus > 0 ? kExclusiveLds : 0;
  if (lds_bytes > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t batch = phase_batch(ps, T, cus);
  for (int64_t t0 = 0; t0 < T;) {
    const int tb = (int)(T - t0 < batch ? T - t0 : batch);
    const int units = (int)phase_units(ps, tb);
    int grid = units < cus ? units : cus;
    if (grid < 1) grid = 1;
    const int wpg = (units + grid - 1) / grid;  // <= kPhaseWpg
    hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(x) + t0 * row_vec,
                       static_cast<u32x4*>(recv), dest_row + t0 * k, recv_rows, row_vec, ps.nv, tb, ps.tpu, ps.nseg,
                       ps.seg, units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    t0 += tb;
  }
  return hipSuccess;
}

}  // namespace

int dispatch_slab_vpl(int row_vec, int cap, int requested) { return choose_vpl(row_vec, cap, requested); }

bool dispatch_auto_large(const Budget& b, int64_t T) {
  const int cus = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  return T >= 8LL * cus;
}

// The default for a batch of at least 8 tokens per CU of its launch: a
// persistent grid on every CU it may use (the budget, the stream's mask or
// the device) running the workgroup-phased register kernel (vgpr_wg) with
// whole-row slabs and streaming loads of x.  Its time hardly depends on
// whether x is in the Infinity Cache.  The LDS-staged kernels (lds1, pc)
// load x with cacheable direct-to-LDS loads: faster while x is cached, up to
// 2.5x slower when it is not (each miss then fills the Infinity Cache).
// Measured at H = 7168, single launches after a 1 GiB write that evicts x
// (cold), and without it (warm), in us, for T = 4096, k = 8 and
// T = 16384, k = 6, E = 64:
//   all CUs: vgpr_wg 105.1 / 101.9 and 334.2 / 332.7; vgpr2 107.5 / 104.7
//     and 344.4 / 339.7; lds1 on 64 CUs 193.6 / 87.9 and 647.3 / 258.2;
//   24 CUs: vgpr_wg 209.3 / 207.7 and 661.8 / 661.2; pc 288.5 / 201.0 and
//     973.8 / 645.4; vgpr2 321.7 / 319.1 and 1068.4 / 1069.4;
//   64 CUs: vgpr_wg 122.5 / 122.1 and 366.1 / 365.5; pc 149.7 / 94.9 and
//     537.6 / 270.0.
// Callers whose x is cache-resident can ask for "lds1" or "pc".
//
// Smaller batches on every CU, from 2 tokens per CU (4 for rows of at most
// 8 KiB) up: the register double buffer (vgpr2) on the ordinary grid, which
// also streams x.  lds1 there goes persistent on dispatch_write_cus(k) CUs
// once it has that many units, and cold those CUs' reads are the bound.
// Cold, us, H = 7168, k = 8: T = 512 15.9 against 16.6 for lds1, T = 1024
// 28.0 against 44.1, T = 1536 41.0 against 66.1; k = 6, T = 1536 32.3
// against 59.6; H = 4096, k = 2, T = 1024 9.1 against 10.1.  Below that,
// lds1 on the ordinary grid: H = 7168, k = 8, T = 256 10.6 against 13.6;
// H = 2048, k = 8, T = 512 7.7 against 9.6, T = 1024 10.9 against 11.2;
// H = 4096, T = 512 (2 per CU), k = 3, 4, 5: 8.2 / 8.8 / 10.0 against
// 9.1 / 10.4 / 11.4, and from T = 1024 vgpr2 is as fast or faster.
// On a CU budget below the device every batch size takes vgpr_wg on the
// budget's CUs, whose reads are the bound there: cold, 1 to 6 tokens per CU
// on 24, 64 and 128 CUs, 7-59% faster than lds1 persistent on the same CUs
// (H = 7168, k = 8, 128 CUs, T = 256: 12.4 against 18.8 us; 24 CUs,
// T = 96: 11.4 against 15.4, T = 144: 15.4 against 16.6; H = 4096, k = 2,
// 64 CUs, T = 256: 7.5 against 10.9) and 15-49% faster than vgpr2 there.
// A CU-masked stream without a budget keeps lds1 on an ordinary grid sized
// to the mask below 8 tokens per CU: with several workgroups per CU it is
// the faster of the two there (decode, T = 128, cold dispatch: 1279 against
// 1054 GB/s on 24 masked CUs, 1570 against 1341 on 64).
//
// Rows of more than 8 KiB that are not a whole number of KiB, at k = 6 or
// 8, take the whole-row workgroup-phased kernel on the ordinary grid instead
// of vgpr2 in that range: vgpr2 runs them in 14-vector slabs that spill
// registers to scratch (9 to 14 vectors per lane) or in 1 KiB slabs (15
// and 16).  Cold, us, every CU, same-run A/B, H = 4104 / 5000 / 6000 /
// 7176, k = 8: T = 512 12.8 / 14.2 / 15.8 / 18.6 against 16.7 / 18.4 /
// 19.8 / 21.4, T = 2000 36.4 / 43.1 / 51.4 / 63.4 against 40.4 / 47.6 /
// 53.6 / 68.1; k = 6 up to 24% faster (one point 2% slower).  k = 7 lost
// 1-9% and k = 5 was even, and at k = 2 and 4 vgpr2 was ahead from
// T = 1536 (up to 22%), so they keep vgpr2.  Whole-KiB rows stay on vgpr2
// (H = 7168, k = 8: 16.0 / 28.0 / 40.2 against 17.1 / 29.1 / 43.0 us at
// T = 512 / 1024 / 1536).
Variant dispatch_auto(const Budget& b, int64_t T, int row_vec, int k, int* persistent_cus) {
  const int cus = b.num_cus > 0 && b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
  if (dispatch_auto_large(b, T) || (b.num_cus > 0 && cus < b.all_cus)) {
    *persistent_cus = cus;
    return Variant::VgprWg;
  }
  const int64_t per_cu = row_vec <= 8 * kWave ? 4 : 2;
  if (cus >= b.all_cus && T >= per_cu * cus) {
    const bool ragged_wide = row_vec > 8 * kWave && row_vec <= 16 * kWave && row_vec % kWave != 0;
    return ragged_wide && (k == 6 || k == 8) ? Variant::VgprWg : Variant::Vgpr2;
  }
  return Variant::Lds1;
}

hipError_t launch_dispatch(Variant v, const Budget& b, const void* x, int T, int H, const int32_t* dest_row, int k,
                           void* recv, int64_t recv_rows, hipStream_t stream) {
  const int row_vec = H / 8;
  int auto_cus = 0;  // the persistent grid the default chose (0: none)
  const bool chosen = v == Variant::Auto;
  if (chosen) v = dispatch_auto(b, T, row_vec, k, &auto_cus);
  const bool known_k = (k == 2 || k == 4 || k == 6 || k == 8);
  if ((v == Variant::Lds2 || v == Variant::Lds3 || v == Variant::Phase) && !known_k) v = Variant::Lds1;
  if (v == Variant::Phase) return launch_dispatch_phase(b, x, T, row_vec, dest_row, k, recv, recv_rows, stream);
  const bool even = row_vec % kWave == 0;
  // Slabs: the register double buffer, the workgroup-phased register kernel
  // and the producer/consumer split take whole rows of up to 14 KiB (T = 4096, H = 7168, x evicted: vgpr2 on all
  // CUs 105.7 against 106.7 us with half rows; pc on 24 CUs 286.7 against
  // 311.8 us).  The other staged kernels take at most 8 KiB (half rows at
  // H = 7168; whole 14 KiB rows measured no faster), the LDS rings holding
  // two or three slabs.  A requested size may go to 16 for the single-set
  // kernels.
  const bool ring = v == Variant::Lds2 || v == Variant::Lds3;
  const int cap = v == Variant::VgprWg ? 16
                : v == Variant::Vgpr2 ? 14
                : v == Variant::Pc ? (b.slab_vpl > 0 ? 16 : 14)
                : (ring || b.slab_vpl == 0) ? 8 : 16;
  int vpl = choose_vpl(row_vec, cap, b.slab_vpl);
  // Rows of more than 16 vectors per lane that no compiled slab divides
  // would get the largest slab that does (2 vectors at 18, 22, 26 and 30):
  // the workgroup-phased kernel takes 14-vector slabs there, the last one
  // partial.  Cold, us, every CU, T = 4096, k = 8: H = 9216 138.7 against
  // 148.2, H = 11264 165.2 against 178.0, H = 13312 197.3 against 211.7,
  // H = 15360 233.9 against 244.1; k = 2 3-7% faster; H = 12288 (24
  // vectors, 8-vector slabs) 1.6% faster.
  const int vpr = (row_vec + kWave - 1) / kWave;
  if (v == Variant::VgprWg && b.slab_vpl == 0 && vpr > 16 && vpr % 16 != 0) vpl = 14;
  const int nslab = (row_vec + vpl * kWave - 1) / (vpl * kWave);
  if ((int64_t)T * nslab > INT32_MAX) return hipErrorInvalidValue;
  const int units = T * nslab;
  // the workgroup-phased kernel's common case: one slab per row of at most
  // 16 vectors per lane (rows_vpl), k <= 8: the straight-line kernel
  const int rows_vpl = (v == Variant::VgprWg && nslab == 1) ? (row_vec + kWave - 1) / kWave : 0;
  const void* rows_fn = rows_vpl > 0 ? wg_rows_kernel(row_vec, k) : nullptr;
  DispatchFn fn = even ? pick_vpl<true>(v, vpl, k) : pick_vpl<false>(v, vpl, k);
  if (!fn) return hipErrorInvalidValue;

  const bool lds = (v == Variant::Lds1 || v == Variant::Lds2 || v == Variant::Lds3);
  const int stages = v == Variant::Lds3 ? 3 : v == Variant::Lds2 ? 2 : 1;
  const size_t per_wave = lds ? (size_t)stages * vpl * kWaveVecBytes : 0;
  int wpg, grid;
  size_t lds_bytes;
  // With no budget set, a large dispatch by a named variant still runs as a
  // persistent grid on dispatch_write_cus(k) CUs: at k = 8 its traffic is
  // 8/9 writes, and HBM write throughput was measured highest with about a
  // quarter of the CUs issuing them (more add contention, not bandwidth);
  // smaller k carry more reads and take more CUs.  Small batches keep the
  // ordinary grid, whose start-up is cheaper.  The default's own choices
  // never take this grid: it picks its persistent grid itself from 8 tokens
  // per CU and keeps the ordinary grid below that.  lds1 persistent on 64
  // CUs, where its many 1-2 KiB slabs of rows with a partial last KiB, or
  // the slabs of rows over 16 KiB, reached the unit count, ran up to 1.9x
  // slower cold (H = 9000, k = 6, T = 256: 20.6 against 11.0 us; H = 32768,
  // k = 8, T = 511: 106.1 against 70.1; H = 5000, k = 8, T = 511: 23.8
  // against 14.1), and no point measured gained from it.
  int budget = b.num_cus;
  const int write_cus = dispatch_write_cus(k);
  if (auto_cus > 0) budget = auto_cus;
  else if (budget == 0 && !chosen && units >= write_cus * 16 * 2) budget = write_cus;
  if (v == Variant::Pc) {
    // one producer and W consumer waves per workgroup, a two-slot ring of W
    // slabs each; always a persistent grid (one workgroup per CU)
    const int W = pc_consumers_host(vpl);
    wpg = W + 1;
    const int want = (units + W - 1) / W;
    grid = budget > 0 ? (budget < b.device_cus ? budget : b.device_cus) : (want < b.device_cus ? want : b.device_cus);
    lds_bytes = (size_t)2 * W * vpl * kWaveVecBytes;
    if (lds_bytes < kExclusiveLds) lds_bytes = kExclusiveLds;
  } else if (budget > 0) {
    // persistent: one workgroup per CU, as many waves as the LDS ring allows
    // (the workgroup-phased kernel: its own workgroup size)
    wpg = v == Variant::VgprWg ? kWgWaves : 16;
    if (per_wave && (int)(kLdsPerCu / per_wave) < wpg) wpg = (int)(kLdsPerCu / per_wave);
    grid = budget < b.device_cus ? budget : b.device_cus;
    lds_bytes = per_wave * wpg;
    if (lds_bytes < kExclusiveLds) lds_bytes = kExclusiveLds;
  } else {
    wpg = 4;
    int per_cu = per_wave ? (int)(kLdsPerCu / (per_wave * wpg)) : 8;
    if (per_cu > 8) per_cu = 8;
    if (per_cu < 1) {
      per_cu = 1;
      wpg = (int)(kLdsPerCu / per_wave);
    }
    grid = (units + wpg - 1) / wpg;
    if (grid > b.device_cus * per_cu) grid = b.device_cus * per_cu;
    lds_bytes = per_wave * wpg;
  }
  if (grid < 1) grid = 1;
  if (rows_fn) {
    if (lds_bytes > 64 * 1024) {
      hipError_t e = allow_dynamic_lds(rows_fn, lds_bytes);
      if (e != hipSuccess) return e;
    }
    const int64_t per_trip = (int64_t)grid * wpg * wg_units_of(rows_vpl);
    // On at least half the device, where HBM is the bound, one launch per
    // trip: the kernel boundary starts every CU's read burst together, which
    // the per-workgroup barrier alone does not (T = 16384, k = 6 on 256 CUs,
    // x evicted: 314.6 us in four launches against 337.4 in one).  On fewer
    // CUs each CU's reads are the bound and a launch per trip only adds
    // ramps (24 CUs: 743 against 666 us), so the grid stays persistent.
    // A trip that moves less than 32 MB (small rows at small k) does not pay
    // for its launch: H = 896 / 1024, k = 2 (22 and 25 MB per trip on 256
    // CUs), T = 8192 to 32768, one launch 7-13% faster (47.1 against 42.0
    // us at H = 1024, T = 32768); at 51 to 113 MB per trip the launch per
    // trip was even or up to 4% ahead.
    const int64_t trip_bytes = per_trip * (int64_t)row_vec * kVecBytes * (1 + k);
    const bool per_trip_launch = 2 * (int64_t)grid >= b.all_cus && trip_bytes >= (32ll << 20);
    const int64_t batch = per_trip_launch ? per_trip : (int64_t)T;
    for (int64_t t0 = 0; t0 < T; t0 += batch) {
      const int tb = (int)(T - t0 < batch ? T - t0 : batch);
      const int trips = (int)((tb + per_trip - 1) / per_trip);
      hipError_t e = launch_wg_rows(rows_fn, grid, wpg, lds_bytes, stream, static_cast<const u32x4*>(x) + t0 * row_vec,
                                    recv, dest_row + t0 * k, recv_rows, tb, trips, row_vec);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (lds_bytes > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(x),
                     static_cast<u32x4*>(recv), dest_row, recv_rows, row_vec, nslab, k, units);
  return hipGetLastError();
}

}  // namespace ep

namespace ep {

hipError_t launch_dispatch_rows(Variant v, const Budget& b, const void* x, int T, int H, const int32_t* src_token,
                                void* recv, int64_t recv_rows, hipStream_t stream) {
  const int row_vec = H / 8;
  const bool even = row_vec % kWave == 0;
  const int vpl = choose_vpl(row_vec, b.slab_vpl > 0 ? 16 : 8, b.slab_vpl);
  const int nslab = (row_vec + vpl * kWave - 1) / (vpl * kWave);
  if (recv_rows * nslab > INT32_MAX) return hipErrorInvalidValue;
  const int units = (int)recv_rows * nslab;
  // "vgpr_cached" selects streaming (nt) loads of x; every other variant keeps them cacheable
  const bool cl = v != Variant::VgprCached;
  RowsFn fn = even ? (cl ? rows_pick<true, true>(vpl) : rows_pick<true, false>(vpl))
                   : (cl ? rows_pick<false, true>(vpl) : rows_pick<false, false>(vpl));
  int wpg, grid;
  size_t lds_bytes = 0;
  if (b.num_cus > 0) {
    wpg = 16;
    grid = b.num_cus < b.device_cus ? b.num_cus : b.device_cus;
    lds_bytes = kExclusiveLds;
  } else {
    wpg = 4;
    grid = (units + wpg - 1) / wpg;
    if (grid > b.device_cus * 8) grid = b.device_cus * 8;
  }
  if (grid < 1) grid = 1;
  if (lds_bytes > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)fn, lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(x),
                     static_cast<u32x4*>(recv), src_token, T, row_vec, nslab, units);
  return hipGetLastError();
}

}  // namespace ep
