// Device primitives for gfx950 (CDNA4, wave64) shared by the row-movement
// kernels: 16-byte vector loads/stores with cache-policy control, the
// direct-to-LDS load and its explicit completion waits, wave ballot/prefix
// helpers, and bf16 <-> f32 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr int kVecBytes = 16;              // one dwordx4 per lane
constexpr int kWaveVecBytes = kWave * 16;  // 1 KiB moved by one wave instruction

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Wave index inside the workgroup, made scalar so that everything derived
// from it (work-unit ids, row addresses, dest_row reads) stays in SGPRs.
__device__ __forceinline__ int wave_in_group() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int mask_rank(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Mask of the lanes that hold the same value v as the calling lane, among
// the lanes with ok set (v < 2^nbits): the intersection of one ballot per bit.
__device__ __forceinline__ uint64_t same_value_lanes(bool ok, int v, int nbits) {
  uint64_t m = ballot(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t bal = ballot(ok && bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Workgroup barrier that orders LDS accesses only: global loads and stores
// issued before it stay in flight (__syncthreads would wait for them).
// Valid wherever threads exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive scan of one value per thread over a block of NWAVES waves;
// *total receives the sum.  s_wave holds NWAVES + 1 ints of LDS.  Every
// thread of the block must call it (it contains two LDS-only barriers).
template <int NWAVES>
__device__ __forceinline__ int block_excl_scan(int v, int32_t* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  lds_barrier();
  if (wave == 0) {
    const int wt = lane < NWAVES ? s_wave[lane] : 0;
    const int ws = wave_incl_scan(wt, lane);
    if (lane < NWAVES) s_wave[lane] = ws - wt;
    if (lane == NWAVES - 1) s_wave[NWAVES] = ws;
  }
  lds_barrier();
  *total = s_wave[NWAVES];
  return incl - v + s_wave[wave];
}

// ---------------------------------------------------------------- global I/O
// NT = true marks the access as streaming (the "nt" cache-policy bit): the
// line is not kept for reuse.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ------------------------------------------------------------ direct-to-LDS
// One wave instruction: every lane fetches 16 bytes from its own global
// address and the data lands in LDS at lds_base + 16 * lane, without passing
// through VGPRs (global_load_lds_dwordx4).  lds_base must be wave-uniform.
// Completion is tracked by the wave's vmcnt counter only.  The load keeps
// the default cache policy: marked streaming (nt) it cut dispatch from 6.1
// to 2.95 TB/s.
__device__ __forceinline__ void dma16(const void* gptr, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}

// Explicit completion waits.  The compiler's own tracking of direct-to-LDS
// loads waits for *all* outstanding vector memory operations before any LDS
// read it can see, which would serialise a two-stage ring; the staged kernels
// therefore read their slices with inline-asm ds_read_b128 (invisible to that
// tracking) and wait with exact counts.  Vector-memory operations of one wave
// retire from vmcnt in issue order, so vmcnt(N) means "everything except the
// N most recently issued vector-memory operations has completed".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
  // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  constexpr int imm = (N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// ds_read_b128 from an LDS byte address, result valid only after
// lds_wait_and_fence() on the same registers.
__device__ __forceinline__ void lds_read16_async(u32x4& v, uint32_t lds_addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr) : "memory");
}
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Ties v to the point after lds_wait_all(): later uses of v cannot be
// scheduled above the wait (volatile asm statements keep their order).
__device__ __forceinline__ void lds_fence_value(u32x4& v) { asm volatile("" : "+v"(v)); }

// LDS byte address of a __shared__ / dynamic-LDS pointer.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even, NaN
// stays NaN: the hardware conversion v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// -------------------------------------------------------------- placement
__device__ __forceinline__ uint32_t hw_id_reg() {
  // HW_REG_HW_ID (id 4), 32 bits
  return __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
}
__device__ __forceinline__ uint32_t xcc_id_reg() {
  // HW_REG_XCC_ID (id 20), 32 bits
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));
}

}  // namespace ep
