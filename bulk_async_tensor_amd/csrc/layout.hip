// ep_layout: per-expert counts, prefix-sum offsets and stable destination
// rows of the (token, slot) entries -- the routing handle that the dispatch
// call of [DeepEP-TMA] ("High-Level DeepEP API Usage") returns for the way
// back.  Entries of one expert are placed in row-major (token, slot) order;
// no atomic operation decides a row, so the result is deterministic.
//
// Fused path (one launch; used while the per-chunk histogram fits in LDS):
// workgroup c owns entries [1024 c, 1024 c + 1024), one 64-entry step per
// wave.  Every workgroup reads all T*k ids (a few hundred KiB at most) and
// builds the full (chunk, expert) histogram in LDS, so it knows each
// expert's total and the part that precedes its chunk without any
// inter-workgroup communication; a block scan over experts gives the
// offsets.  Inside the chunk, lanes holding the same expert find each other
// with log2(E) ballots, rank themselves with mbcnt, and the per-step group
// sizes (written to LDS by the highest lane of each group) give each wave
// the rows taken by the steps before it.
//
// Large path (three launches): count (LDS histogram per chunk of tokens),
// scan (one workgroup: totals, offsets and the base row of every (chunk,
// expert)), place (one wave per chunk walking its entries 64 at a time,
// advancing per-expert cursors in LDS).
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

namespace {

constexpr int kChunkEntries = 1024;   // entries per chunk (tokens * k), at most
constexpr int kMaxSteps = kChunkEntries / kWave;  // 64-entry steps of one chunk
constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kStatusOutOfRange = 1;
constexpr int kStatusDuplicate = 2;

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(const int32_t* __restrict__ idx, int T,
                                                                     int k, int E, int chunk_tokens,
                                                                     int32_t* __restrict__ chunk_counts,
                                                                     int32_t* __restrict__ chunk_status) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;      // [E]
  int32_t* ent = lds + E;   // [chunk_tokens * k]
  __shared__ int32_t s_status;

  const int c = blockIdx.x;
  const int t0 = c * chunk_tokens;
  const int nt = min(chunk_tokens, T - t0);
  const int n = nt * k;
  const int32_t* src = idx + (int64_t)t0 * k;

  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (threadIdx.x == 0) s_status = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ent[i] = src[i];
  __syncthreads();

  int bad = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ent[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    else bad |= kStatusOutOfRange;
  }
  // repeated expert inside one token: thread per token, pairwise
  for (int tt = threadIdx.x; tt < nt; tt += blockDim.x) {
    const int32_t* r = ent + tt * k;
    for (int j = 1; j < k; ++j) {
      const int e = r[j];
      if ((unsigned)e >= (unsigned)E) continue;
      for (int j2 = 0; j2 < j; ++j2)
        if (r[j2] == e) bad |= kStatusDuplicate;
    }
  }
  if (bad) atomicOr(&s_status, bad);
  __syncthreads();

  int32_t* out = chunk_counts + (int64_t)c * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
  if (threadIdx.x == 0) chunk_status[c] = s_status;
}

// Single workgroup.  Threads form G = 1024 / Epad groups of Epad lanes
// (Epad = E rounded up to a power of two, at least 64); group g owns a
// contiguous range of chunks and lane e an expert.  chunk_counts is
// overwritten in place with the first receive row of each (chunk, expert).
__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(int32_t* __restrict__ chunk_counts,
                                                                   const int32_t* __restrict__ chunk_status,
                                                                   int nchunks, int E, int epad,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  const int G = kScanThreads / epad;
  int32_t* part = lds;                 // [G][epad]
  int32_t* scan = lds + G * epad;      // [2][epad] ping-pong
  __shared__ int32_t s_status;

  const int tid = threadIdx.x;
  const int g = tid / epad;
  const int e = tid - g * epad;
  const int cpg = (nchunks + G - 1) / G;
  const int c0 = min(nchunks, g * cpg);
  const int c1 = min(nchunks, c0 + cpg);

  if (tid == 0) s_status = 0;

  int sum = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += chunk_counts[(int64_t)c * E + e];
  }
  part[g * epad + e] = sum;
  int st = 0;
  for (int c = tid; c < nchunks; c += kScanThreads) st |= chunk_status[c];
  __syncthreads();
  if (st) atomicOr(&s_status, st);

  int pre = 0, tot = 0;
  for (int g2 = 0; g2 < G; ++g2) {
    const int v = part[g2 * epad + e];
    pre += (g2 < g) ? v : 0;
    tot += v;
  }
  // inclusive scan of tot over e (Hillis-Steele, ping-pong buffers)
  if (g == 0) scan[e] = tot;
  __syncthreads();
  int src = 0;
  for (int d = 1; d < epad; d <<= 1) {
    if (g == 0) {
      const int v = scan[src * epad + e] + ((e >= d) ? scan[src * epad + e - d] : 0);
      scan[(src ^ 1) * epad + e] = v;
    }
    src ^= 1;
    __syncthreads();
  }
  const int incl = scan[src * epad + e];
  const int excl = incl - tot;
  if (g == 0 && e < E) {
    counts[e] = tot;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = incl;
  }
  if (e < E) {
    int run = excl + pre;
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int64_t at = (int64_t)c * E + e;
      const int v = chunk_counts[at];
      chunk_counts[at] = run;
      run += v;
    }
  }
  __syncthreads();
  if (tid == 0 && status) status[0] = s_status;
}

// One wave per chunk.  run[e] (LDS) is the next free receive row of expert e
// for this chunk.
__global__ __launch_bounds__(kWave) void layout_place_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                            int nbits, int chunk_tokens,
                                                            const int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ dest_row,
                                                            int32_t* __restrict__ src_token) {
  extern __shared__ int32_t run[];  // [E]
  const int lane = lane_id();
  const int c = blockIdx.x;
  const int t0 = c * chunk_tokens;
  const int nt = min(chunk_tokens, T - t0);
  const int n = nt * k;
  const int64_t i0 = (int64_t)t0 * k;

  for (int e = lane; e < E; e += kWave) run[e] = chunk_base[(int64_t)c * E + e];

  // fetch the whole chunk up front: one memory latency instead of one per step
  int ent[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    const int i = s * kWave + lane;
    ent[s] = (i < n) ? idx[i0 + i] : -1;
  }
  __syncthreads();

  const int nsteps = (n + kWave - 1) / kWave;
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    if (s >= nsteps) continue;  // uniform; keeps the loop fully unrolled so ent[] stays in VGPRs
    const int i = s * kWave + lane;
    const bool in_chunk = i < n;
    const int e = ent[s];
    const bool ok = in_chunk && (unsigned)e < (unsigned)E;
    const uint64_t m = same_value_lanes(ok, e, nbits);
    const int rank = mask_rank(m);
    int r = -1;
    if (ok) r = run[e] + rank;
    // the highest lane of each group moves the expert's cursor past the group
    if (ok && (m >> lane) == 1ull) run[e] = r + 1;
    // one wave: its LDS operations complete in program order, so the next
    // step's reads see these writes; no barrier (a barrier would also wait
    // for the global stores below)
    __builtin_amdgcn_wave_barrier();
    if (in_chunk) {
      dest_row[i0 + i] = r;
      if (ok && src_token) src_token[r] = t0 + i / k;
    }
  }
}

constexpr int kFusedChunk = 1024;   // entries per workgroup: 16 waves x 64
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;

// Reads the k ids of token t, checks them and adds them to the (chunk,
// expert) histogram.  KT > 0: k known at compile time, so the loads of a
// token are independent and issued together.
template <int KT>
__device__ __forceinline__ void count_token(const int32_t* __restrict__ idx, int t, int k, int E, int32_t* cnt,
                                            int& bad) {
  constexpr int KA = KT > 0 ? KT : 1;
  if constexpr (KT > 0) {
    int e[KA];
#pragma unroll
    for (int j = 0; j < KA; ++j) e[j] = idx[(int64_t)t * KA + j];
#pragma unroll
    for (int j = 0; j < KA; ++j) {
      const int i = t * KA + j;
      if ((unsigned)e[j] < (unsigned)E) {
        atomicAdd(&cnt[(i >> 10) * E + e[j]], 1);
#pragma unroll
        for (int j2 = 0; j2 < j; ++j2)
          if (e[j2] == e[j]) bad |= kStatusDuplicate;
      } else {
        bad |= kStatusOutOfRange;
      }
    }
  } else {
    const int32_t* r = idx + (int64_t)t * k;
    for (int j = 0; j < k; ++j) {
      const int e = r[j];
      const int i = t * k + j;
      if ((unsigned)e < (unsigned)E) {
        atomicAdd(&cnt[(i >> 10) * E + e], 1);
        for (int j2 = 0; j2 < j; ++j2)
          if (r[j2] == e) bad |= kStatusDuplicate;
      } else {
        bad |= kStatusOutOfRange;
      }
    }
  }
}

template <int KT>
__global__ __launch_bounds__(kFusedThreads) void layout_fused_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                     int E, int nbits, int nchunks,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ dest_row,
                                                                     int32_t* __restrict__ src_token,
                                                                     int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;                         // [nchunks][E] entries per (chunk, expert)
  int32_t* stepc = cnt + nchunks * E;         // [16][E] group sizes per step of this chunk
  int32_t* base = stepc + kFusedWaves * E;    // [E] first row of each expert for this chunk
  __shared__ int32_t s_wave[kFusedWaves + 1];
  __shared__ int32_t s_status;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int c = blockIdx.x;
  const int N = T * k;

  for (int i = tid; i < (nchunks + kFusedWaves) * E; i += kFusedThreads) cnt[i] = 0;
  if (tid == 0) s_status = 0;
  const int my_i = c * kFusedChunk + tid;
  const int my_e = my_i < N ? idx[my_i] : -1;
  __syncthreads();

  // Every workgroup histograms all tokens (thread per token) and validates
  // them, so each one knows the totals and the global status by itself.
  // Two tokens per trip keep 2k loads in flight per thread.
  int bad = 0;
  for (int t = tid; t < T; t += 2 * kFusedThreads) {
    count_token<KT>(idx, t, k, E, cnt, bad);
    if (t + kFusedThreads < T) count_token<KT>(idx, t + kFusedThreads, k, E, cnt, bad);
  }
  if (bad) atomicOr(&s_status, bad);
  __syncthreads();

  // expert totals, the part before this chunk, and the offsets
  int tot = 0, pre = 0;
  if (tid < E) {
    for (int cc = 0; cc < nchunks; ++cc) {
      const int v = cnt[cc * E + tid];
      tot += v;
      pre += (cc < c) ? v : 0;
    }
  }
  int all = 0;
  const int excl = block_excl_scan<kFusedWaves>(tot, s_wave, &all);
  if (tid < E) base[tid] = excl + pre;
  if (c == 0) {
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = excl;
    }
    if (tid == 0) {
      offsets[E] = all;
      if (status) status[0] = s_status;
    }
  }

  // ranks inside this wave's 64-entry step
  const bool in_range = my_i < N;
  const bool ok = in_range && (unsigned)my_e < (unsigned)E;
  const uint64_t m = same_value_lanes(ok, my_e, nbits);
  const int rank = mask_rank(m);
  if (ok && (m >> lane) == 1ull) stepc[wave * E + my_e] = __builtin_popcountll(m);
  __syncthreads();
  if (in_range) {
    int r = -1;
    if (ok) {
      r = base[my_e] + rank;
      for (int w = 0; w < wave; ++w) r += stepc[w * E + my_e];
      if (src_token) src_token[r] = my_i / k;
    }
    dest_row[my_i] = r;
  }
}

using FusedFn = void (*)(const int32_t*, int, int, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*);

FusedFn fused_for(int k) {
  switch (k) {
    case 1: return layout_fused_kernel<1>;
    case 2: return layout_fused_kernel<2>;
    case 4: return layout_fused_kernel<4>;
    case 6: return layout_fused_kernel<6>;
    case 8: return layout_fused_kernel<8>;
    default: return layout_fused_kernel<0>;
  }
}

size_t fused_lds_bytes(int T, int k, int E) {
  const int64_t N = (int64_t)T * k;
  const int64_t nchunks = (N + kFusedChunk - 1) / kFusedChunk;
  return (size_t)(nchunks + kFusedWaves + 1) * E * sizeof(int32_t);
}

bool use_fused(int T, int k, int E) {
  const int64_t N = (int64_t)T * k;
  const int64_t nchunks = (N + kFusedChunk - 1) / kFusedChunk;
  return nchunks <= 128 && fused_lds_bytes(T, k, E) <= 144 * 1024;
}

}  // namespace

int layout_chunk_tokens(int k) { return kChunkEntries / k; }

int layout_num_chunks(int T, int k) {
  const int ct = layout_chunk_tokens(k);
  return (T + ct - 1) / ct;
}

size_t layout_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || use_fused(T, k, E)) return 0;
  const size_t nch = (size_t)layout_num_chunks(T, k);
  size_t counts = nch * (size_t)E * sizeof(int32_t);
  counts = (counts + 255) & ~(size_t)255;
  return counts + nch * sizeof(int32_t);
}

hipError_t launch_layout(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                         int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
                         hipStream_t stream) {
  int epad = 64;
  while (epad < E) epad <<= 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (T == 0 || use_fused(T, k, E)) {
    const int N = T * k;
    const int nchunks = (N + kFusedChunk - 1) / kFusedChunk;
    const size_t lds = fused_lds_bytes(T, k, E);
    FusedFn fn = fused_for(k);
    if (lds > 64 * 1024) {
      hipError_t e = allow_dynamic_lds((const void*)fn, lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(nchunks > 0 ? nchunks : 1), dim3(kFusedThreads), lds, stream, idx, T, k, E, nbits,
                       nchunks, counts, offsets, dest_row, src_token, status);
    return hipGetLastError();
  }
  const int ct = layout_chunk_tokens(k);
  const int nch = T > 0 ? layout_num_chunks(T, k) : 0;

  int32_t* chunk_counts = static_cast<int32_t*>(workspace);
  int32_t* chunk_status = nullptr;
  if (nch > 0) {
    size_t cb = (size_t)nch * E * sizeof(int32_t);
    cb = (cb + 255) & ~(size_t)255;
    chunk_status = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cb);
    const size_t lds = (size_t)(E + ct * k) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_count_kernel, dim3(nch), dim3(kCountThreads), lds, stream, idx, T, k, E, ct,
                       chunk_counts, chunk_status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int G = kScanThreads / epad;
    const size_t lds = (size_t)(G * epad + 2 * epad) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), lds, stream, chunk_counts, chunk_status,
                       nch, E, epad, counts, offsets, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (nch > 0) {
    const size_t lds = (size_t)E * sizeof(int32_t);
    hipLaunchKernelGGL(layout_place_kernel, dim3(nch), dim3(kWave), lds, stream, idx, T, k, E, nbits, ct,
                       chunk_counts, dest_row, src_token);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace ep
