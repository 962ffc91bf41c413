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

}  // namespace ep
