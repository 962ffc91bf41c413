// The workgroup-phased dispatch (vgpr_wg) for its common case: one slab per
// row, with the row's own length in vectors per lane compiled in (1 .. 16
// KiB) and k known at compile time (1 .. 8).  A unit is a token; its loads
// and stores are straight-line, with no per-vector row-end checks (one wave
// runs per SIMD, so every extra instruction between the memory operations
// costs issue time), and every workgroup makes the same `trips`, so every
// barrier is met by all of its waves.
//
// RAGGED: the row is not a whole number of KiB.  Its first VPL - 1 KiB are
// whole; lanes past the tail of the last KiB load the row's last vector and
// store nothing there, and rows are row_vec vectors apart.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

namespace {

template <int VPL, int K, bool RAGGED>
__global__ __launch_bounds__(kWgWaves * kWave) void dispatch_wg_rows_kernel(const u32x4* __restrict__ x,
                                                                            u32x4* __restrict__ recv,
                                                                            const int32_t* __restrict__ dest_row,
                                                                            int64_t recv_rows, int T, int trips,
                                                                            int row_vec) {
  constexpr int U = wg_units_of(VPL);
  const int64_t rv = RAGGED ? row_vec : VPL * kWave;
  const int lane = lane_id();
  const int tail = RAGGED ? row_vec - (VPL - 1) * kWave : kWave;  // lanes of the last KiB inside the row
  const bool in_tail = lane < tail;
  const int last = (VPL - 1) * kWave + (in_tail ? lane : tail - 1);
  const int wpg = blockDim.x >> 6;
  const int stride = gridDim.x * wpg;
  const int first = blockIdx.x * wpg + wave_in_group();
  for (int r = 0; r < trips; ++r) {
    u32x4 v[U][VPL];
    int32_t d[U][K];
    bool live[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int t = first + (r * U + q) * stride;
      live[q] = t < T;
      const int64_t tc = live[q] ? t : 0;
      const u32x4* src = x + tc * rv;
#pragma unroll
      for (int i = 0; i < VPL - 1; ++i) v[q][i] = ld16<true>(src + i * kWave + lane);
      v[q][VPL - 1] = ld16<true>(src + last);
#pragma unroll
      for (int j = 0; j < K; ++j) d[q][j] = dest_row[tc * K + j];
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
#pragma unroll
      for (int j = 0; j < K; ++j) asm volatile("" : "+s"(d[q][j]));
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (!live[q]) continue;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if ((uint64_t)(int64_t)d[q][j] >= (uint64_t)recv_rows) continue;
        u32x4* p = recv + (int64_t)d[q][j] * rv + lane;
#pragma unroll
        for (int i = 0; i < VPL - 1; ++i) st16<true>(p + i * kWave, v[q][i]);
        if (!RAGGED || in_tail) st16<true>(p + (VPL - 1) * kWave, v[q][VPL - 1]);
      }
    }
  }
}

using RowsFn = void (*)(const u32x4*, u32x4*, const int32_t*, int64_t, int, int, int);

template <int VPL, bool RAGGED>
RowsFn pick_k(int k) {
  switch (k) {
    case 1: return dispatch_wg_rows_kernel<VPL, 1, RAGGED>;
    case 2: return dispatch_wg_rows_kernel<VPL, 2, RAGGED>;
    case 3: return dispatch_wg_rows_kernel<VPL, 3, RAGGED>;
    case 4: return dispatch_wg_rows_kernel<VPL, 4, RAGGED>;
    case 5: return dispatch_wg_rows_kernel<VPL, 5, RAGGED>;
    case 6: return dispatch_wg_rows_kernel<VPL, 6, RAGGED>;
    case 7: return dispatch_wg_rows_kernel<VPL, 7, RAGGED>;
    case 8: return dispatch_wg_rows_kernel<VPL, 8, RAGGED>;
    default: return nullptr;
  }
}

template <bool RAGGED>
RowsFn pick_vpl(int vpl, int k) {
  switch (vpl) {
    case 1: return pick_k<1, RAGGED>(k);
    case 2: return pick_k<2, RAGGED>(k);
    case 3: return pick_k<3, RAGGED>(k);
    case 4: return pick_k<4, RAGGED>(k);
    case 5: return pick_k<5, RAGGED>(k);
    case 6: return pick_k<6, RAGGED>(k);
    case 7: return pick_k<7, RAGGED>(k);
    case 8: return pick_k<8, RAGGED>(k);
    case 9: return pick_k<9, RAGGED>(k);
    case 10: return pick_k<10, RAGGED>(k);
    case 11: return pick_k<11, RAGGED>(k);
    case 12: return pick_k<12, RAGGED>(k);
    case 13: return pick_k<13, RAGGED>(k);
    case 14: return pick_k<14, RAGGED>(k);
    case 15: return pick_k<15, RAGGED>(k);
    case 16: return pick_k<16, RAGGED>(k);
    default: return nullptr;
  }
}

}  // namespace

const void* wg_rows_kernel(int row_vec, int k) {
  const int vpl = (row_vec + kWave - 1) / kWave;
  const bool ragged = row_vec % kWave != 0;
  RowsFn fn = ragged ? pick_vpl<true>(vpl, k) : pick_vpl<false>(vpl, k);
  return reinterpret_cast<const void*>(fn);
}

hipError_t launch_wg_rows(const void* kernel, int grid, int wpg, size_t lds_bytes, hipStream_t stream, const void* x,
                          void* recv, const int32_t* dest_row, int64_t recv_rows, int T, int trips, int row_vec) {
  RowsFn fn = reinterpret_cast<RowsFn>(const_cast<void*>(kernel));
  hipLaunchKernelGGL(fn, dim3(grid), dim3(wpg * kWave), lds_bytes, stream, static_cast<const u32x4*>(x),
                     static_cast<u32x4*>(recv), dest_row, recv_rows, T, trips, row_vec);
  return hipGetLastError();
}

}  // namespace ep
