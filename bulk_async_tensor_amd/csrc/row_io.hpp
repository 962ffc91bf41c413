// Row-slab work units and their 16-byte vector loads and stores, shared by
// the dispatch, combine and fused decode kernels.
//
// A work unit is (row, slab): slab s of a row covers vectors
// [s * VPL * 64, (s + 1) * VPL * 64) of its row_vec 16-byte vectors; lane L
// of a wave handles vectors c0 + i * 64 for i < nvec.  EVEN = row_vec is a
// multiple of 64, so no lane ever falls off the row end.
#pragma once

#include "ep_device.hpp"

namespace ep {

struct Unit {
  int64_t t;  // the row (token, or receive row) of the unit
  int c0;     // this lane's first vector of the slab
  int nvec;   // vectors of the slab inside the row (uniform, >= 1)
};

template <int VPL>
__device__ __forceinline__ Unit unit_of(int u, int nslab, int row_vec, int lane) {
  Unit r;
  const int t = u / nslab;
  const int s = u - t * nslab;
  const int first = s * (VPL * kWave);
  r.t = t;
  r.c0 = first + lane;
  const int left = (row_vec - first + kWave - 1) / kWave;
  r.nvec = left < VPL ? left : VPL;
  return r;
}

template <int VPL, bool EVEN, bool NT>
__device__ __forceinline__ void load_slab(u32x4 (&v)[VPL], const u32x4* __restrict__ src, const Unit& un,
                                          int row_vec) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i < un.nvec) {
      const int c = un.c0 + i * kWave;
      if (EVEN || c < row_vec) v[i] = ld16<NT>(src + c);
    }
  }
}

// Exactly VPL loads, none skipped: vectors past the row end (and every
// vector of an idle unit, given row 0) are clamped to the row's last vector
// and never used.  A fixed count lets the compiler wait for these loads
// precisely instead of draining every outstanding memory operation.
template <int VPL, bool NT>
__device__ __forceinline__ void load_slab_fixed(u32x4 (&v)[VPL], const u32x4* __restrict__ src, const Unit& un,
                                                int row_vec) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = un.c0 + i * kWave;
    v[i] = ld16<NT>(src + (c < row_vec ? c : row_vec - 1));
  }
}

// Stores one slab; every store with i < nvec is issued (lane 0 is inside
// the row), which the two-stage kernels rely on when counting operations.
template <int VPL, bool EVEN, bool NT>
__device__ __forceinline__ void store_one(const u32x4 (&v)[VPL], u32x4* __restrict__ dst, const Unit& un,
                                          int row_vec) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i < un.nvec) {
      const int c = un.c0 + i * kWave;
      if (EVEN || c < row_vec) st16<NT>(dst + c, v[i]);
    }
  }
}

// Direct-to-LDS fill of one slab: instruction i moves vector i of every lane
// into slice + i KiB.  Every instruction with i < nvec is issued.
template <int VPL, bool EVEN>
__device__ __forceinline__ void dma_slab(const u32x4* __restrict__ src, char* slice, const Unit& un, int row_vec) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (i < un.nvec) {
      const int c = un.c0 + i * kWave;
      if (EVEN || c < row_vec) dma16(src + c, (lds_void_t*)(slice + i * kWaveVecBytes));
    }
  }
}

// Reads the whole slice (vectors past the slab hold stale bytes of this wave's
// own slice and are never stored): unconditional reads keep the register
// allocation simple.
template <int VPL>
__device__ __forceinline__ void read_slab(u32x4 (&v)[VPL], const char* slice, int lane) {
  const uint32_t base = lds_addr_of(slice) + lane * kVecBytes;
#pragma unroll
  for (int i = 0; i < VPL; ++i) lds_read16_async(v[i], base + i * kWaveVecBytes);
  lds_wait_all();
#pragma unroll
  for (int i = 0; i < VPL; ++i) lds_fence_value(v[i]);
}

// ---- phased units: a wave holds up to `held` vectors per lane of rows in
// registers between reading and writing them: kPhaseHeld (16 KiB) in
// workgroups of kPhaseWpg waves, or kPhaseWideHeld (28 KiB) in workgroups of
// kPhaseWideWpg waves, which leaves each wave the registers for it.  A unit
// is tpu whole rows when a row has at most `held` vectors per lane
// (nseg == 1), else one of nseg segments of seg vectors of one row.
// Host-side geometry.
constexpr int kPhaseHeld = 16;
constexpr int kPhaseWpg = 16;  // waves per workgroup; one such workgroup fits a CU
constexpr int kPhaseWideHeld = 28;
constexpr int kPhaseWideWpg = 8;

struct PhaseShape {
  int nv, tpu, nseg, seg;
  int held = kPhaseHeld, wpg = kPhaseWpg;
};

inline PhaseShape phase_shape(int row_vec, int held = kPhaseHeld, int wpg = kPhaseWpg) {
  PhaseShape p;
  p.held = held;
  p.wpg = wpg;
  p.nv = (row_vec + kWave - 1) / kWave;
  p.tpu = 1;
  p.nseg = 1;
  p.seg = p.nv;
  if (p.nv <= held) {
    p.tpu = held / p.nv;
  } else {
    p.nseg = (p.nv + held - 1) / held;
    p.seg = (p.nv + p.nseg - 1) / p.nseg;
  }
  return p;
}

inline int64_t phase_units(const PhaseShape& p, int64_t T) {
  return p.nseg == 1 ? (T + p.tpu - 1) / p.tpu : T * p.nseg;
}

// Rows per launch so that every launch gives each wave of a grid of `cus`
// workgroups at most one unit, in launches of equal size (whole units).
inline int64_t phase_batch(const PhaseShape& p, int64_t T, int cus) {
  const int64_t wave_slots = (int64_t)cus * p.wpg;
  const int64_t max_batch = p.nseg == 1 ? wave_slots * p.tpu : (wave_slots / p.nseg > 0 ? wave_slots / p.nseg : 1);
  const int64_t nbatch = (T + max_batch - 1) / max_batch;
  int64_t batch = (T + nbatch - 1) / nbatch;
  if (p.nseg == 1) batch = (batch + p.tpu - 1) / p.tpu * p.tpu;
  return batch;
}

}  // namespace ep
