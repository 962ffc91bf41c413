// ep_layout: per-expert counts, prefix-sum offsets and stable destination
// rows of the (token, slot) entries -- the routing handle that the dispatch
// call of [DeepEP-TMA] ("High-Level DeepEP API Usage") returns for the way
// back.  Entries of one expert are placed in row-major (token, slot) order;
// no atomic operation decides a row, so the result is deterministic.
//
// One-launch path (a few 1024-entry chunks, or up to 64 when E > 64):
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
// Two-launch path (larger batches, or few experts): count (an LDS histogram per chunk
// of 1024 / k tokens, equal experts of a step aggregated into one atomic),
// then scan and rank in one launch, each workgroup summing the small
// (chunk, expert) table instead of all ids.
//
// Three-launch path (tables too large to read per workgroup): count, a scan
// of the table over chunks (one workgroup per 64 experts, running counts
// written in place), then the rank kernel of the two-launch path reading
// two table entries per expert instead of the whole table.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

namespace {

constexpr int kChunkEntries = 1024;   // entries per chunk (tokens * k), at most
constexpr int kCountThreads = 256;
constexpr int kStatusOutOfRange = 1;
constexpr int kStatusDuplicate = 2;

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(const int32_t* __restrict__ idx, int T,
                                                                     int k, int E, int nbits, int chunk_tokens,
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
  // a chunk holds at most kChunkEntries = 4 x kCountThreads ids: every load
  // is issued before the first LDS store waits on one
  static_assert(kChunkEntries == 4 * kCountThreads, "four ids per thread");
  int v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x + q * kCountThreads;
    v[q] = i < n ? src[i] : 0;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x + q * kCountThreads;
    if (i < n) ent[i] = v[q];
  }
  __syncthreads();

  // Lanes of one step that hold the same expert add their count with one
  // atomic (the highest lane of the group): with a few hot experts the
  // atomics of a step would otherwise serialise on one address.
  int bad = 0;
  const int lane = lane_id();
  for (int i0 = threadIdx.x - lane; i0 < n; i0 += blockDim.x) {  // uniform per wave
    const int i = i0 + lane;
    const int e = i < n ? ent[i] : -1;
    const bool ok = (unsigned)e < (unsigned)E;
    if (i < n && !ok) bad |= kStatusOutOfRange;
    const uint64_t m = same_value_lanes(ok, e, nbits);
    if (ok && (m >> lane) == 1ull) atomicAdd(&hist[e], __builtin_popcountll(m));
  }
  // repeated expert inside one token: every entry is compared with the
  // earlier entries of its token, entries spread over all threads (a thread
  // per token would leave most threads idle and walk k^2 / 2 pairs each)
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ent[i];
    if ((unsigned)e >= (unsigned)E) continue;
    for (int i2 = i - i % k; i2 < i; ++i2)
      if (ent[i2] == e) bad |= kStatusDuplicate;
  }
  if (bad) atomicOr(&s_status, bad);
  __syncthreads();

  int32_t* out = chunk_counts + (int64_t)c * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
  if (threadIdx.x == 0) chunk_status[c] = s_status;
}

// Middle launch of the three-launch path, for (chunk, expert) tables too
// large for every rank workgroup to read: one workgroup per 64 experts.  Its
// 16 waves take consecutive ranges of chunks and lane e of each wave an
// expert; the table is overwritten in place with each expert's running count
// up to and including each chunk.  The rank kernel then finds the rows of
// its expert before its chunk in the previous chunk's entry and the expert's
// total in the last chunk's.  Each entry is read and written by one thread
// only.
__global__ __launch_bounds__(1024) void layout_colscan_kernel(int32_t* __restrict__ chunk_counts, int nchunks,
                                                              int E) {
  constexpr int kWaves = 1024 / kWave;
  __shared__ int32_t part[kWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int e = blockIdx.x * kWave + lane;
  const int cpw = (nchunks + kWaves - 1) / kWaves;
  const int c0 = min(nchunks, wave * cpw);
  const int c1 = min(nchunks, c0 + cpw);
  int sum = 0;
  if (e < E) {
    for (int cb = c0; cb < c1; cb += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = cb + q < c1 ? chunk_counts[(int64_t)(cb + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) sum += v[q];
    }
  }
  part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += part[w][lane];
  if (e < E) {
    for (int cb = c0; cb < c1; cb += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = cb + q < c1 ? chunk_counts[(int64_t)(cb + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        run += v[q];
        if (cb + q < c1) chunk_counts[(int64_t)(cb + q) * E + e] = run;
      }
    }
  }
}

// Second launch of the two-launch path: scan and rank in one kernel, one
// workgroup of 1024 threads per chunk of the count kernel (chunk_tokens
// tokens, at most 1024 entries; thread j takes entry j of the chunk).  Each
// workgroup reads the whole (chunk, expert) table written by the count
// kernel -- nchunks x E counts, instead of the T*k ids that the one-launch
// path histograms -- and sums it in G = 1024 / Epad groups of Epad lanes
// (lane e an expert, group g a range of chunks): the totals give the
// offsets, the chunks before its own the start of each expert's rows in this
// chunk.  Ranks inside the chunk as in the one-launch path.  With
// `prefixed` (the three-launch path) the table already holds running counts
// (layout_colscan_kernel): it reads two entries per expert instead.
__global__ __launch_bounds__(1024) void layout_rank_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                           int nbits, int epad, int chunk_tokens, int nchunks,
                                                           int prefixed, const int32_t* __restrict__ chunk_counts,
                                                           const int32_t* __restrict__ chunk_status,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ dest_row,
                                                           int32_t* __restrict__ src_token,
                                                           int32_t* __restrict__ status) {
  constexpr int kWaves = 1024 / kWave;
  extern __shared__ int32_t lds[];
  const int G = 1024 / epad;
  int32_t* part_tot = lds;                  // [G][epad]
  int32_t* part_pre = part_tot + G * epad;  // [G][epad]
  int32_t* stepc = part_pre + G * epad;     // [16][E] group sizes per 64-entry step of this chunk
  int32_t* base = stepc + kWaves * E;       // [E] first row of each expert for this chunk
  __shared__ int32_t s_wave[kWaves + 1];
  __shared__ int32_t s_status;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int c = blockIdx.x;
  const int t0 = c * chunk_tokens;
  const int nt = min(chunk_tokens, T - t0);
  const int n = nt * k;
  const int64_t i = (int64_t)t0 * k + tid;
  const bool in_range = tid < n;
  const int my_e = in_range ? idx[i] : -1;
  if (tid == 0) s_status = 0;

  int st = 0;
  for (int cc = tid; cc < nchunks; cc += 1024) st |= chunk_status[cc];
  const int g = tid / epad;
  const int e = tid - g * epad;
  // expert totals and the part before this chunk; thread e of group 0 holds expert e
  int tot = 0, pre = 0;
  if (prefixed) {
    if (g == 0 && e < E) {
      tot = chunk_counts[(int64_t)(nchunks - 1) * E + e];
      pre = c > 0 ? chunk_counts[(int64_t)(c - 1) * E + e] : 0;
    }
    __syncthreads();
    if (st) atomicOr(&s_status, st);
  } else {
    const int cpg = (nchunks + G - 1) / G;
    const int c0 = min(nchunks, g * cpg);
    const int c1 = min(nchunks, c0 + cpg);
    // up to 8 counts per trip, all loads issued before the first is used
    int sum = 0, before = 0;
    if (e < E) {
      for (int cb = c0; cb < c1; cb += 8) {
        int v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = cb + q < c1 ? chunk_counts[(int64_t)(cb + q) * E + e] : 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          sum += v[q];
          before += cb + q < c ? v[q] : 0;
        }
      }
    }
    part_tot[g * epad + e] = sum;
    part_pre[g * epad + e] = before;
    __syncthreads();
    if (st) atomicOr(&s_status, st);
    if (g == 0 && e < E) {
      for (int g2 = 0; g2 < G; ++g2) {
        tot += part_tot[g2 * epad + e];
        pre += part_pre[g2 * epad + e];
      }
    }
  }
  int all = 0;
  const int excl = block_excl_scan<kWaves>(tot, s_wave, &all);  // threads past E add 0
  if (g == 0 && e < E) base[e] = excl + pre;
  for (int x = tid; x < kWaves * E; x += 1024) stepc[x] = 0;
  __syncthreads();
  if (c == 0) {
    if (g == 0 && e < E) {
      counts[e] = tot;
      offsets[e] = excl;
    }
    if (tid == 0) {
      offsets[E] = all;
      if (status) status[0] = s_status;
    }
  }

  // ranks inside this wave's 64-entry step
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
      if (src_token) src_token[r] = t0 + tid / k;
    }
    dest_row[i] = r;
  }
}

size_t rank_lds_bytes(int E, int epad) { return (size_t)(2 * 1024 + 16 * E + E) * sizeof(int32_t); }

constexpr int kFusedChunk = 1024;   // entries per workgroup: 16 waves x 64
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;

// Reads the KT ids of token t (KT known at compile time, so its loads are
// independent and issued together), keeps them in registers and adds them
// to the (chunk, expert) histogram.  check_dups: compare every id with the
// earlier ids of its token (only the workgroup that reports the status does).
template <int KT>
__device__ __forceinline__ void count_token(const int32_t* __restrict__ idx, int t, int E, int32_t* cnt, int& bad,
                                            bool check_dups) {
  int e[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) e[j] = idx[(int64_t)t * KT + j];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    const int i = t * KT + j;
    if ((unsigned)e[j] < (unsigned)E) {
      atomicAdd(&cnt[(i >> 10) * E + e[j]], 1);
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

  // Every workgroup histograms all tokens (thread per token), so each one
  // knows the totals by itself; workgroup 0, which reports the status, also
  // looks for repeated experts.  Two tokens per trip keep 2k loads in flight
  // per thread.
  int bad = 0;
  const bool dups = c == 0;
  for (int t = tid; t < T; t += 2 * kFusedThreads) {
    count_token<KT>(idx, t, E, cnt, bad, dups);
    if (t + kFusedThreads < T) count_token<KT>(idx, t + kFusedThreads, E, cnt, bad, dups);
  }
  if (bad) atomicOr(&s_status, bad);
  __syncthreads();

  // expert totals, the part before this chunk, and the offsets (a plain loop
  // per expert measured faster than spreading the sums over all threads)
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

// The one-launch kernel keeps a token's ids in registers, so k must be
// known at compile time: instances for k = 1 .. 8.  With k known only at run
// time it measured 30-40 us at 32 Ki entries (k = 3, 7, 16, 32) against
// 8.5 us for k = 8, so larger k take the count kernel, whose chunk of ids
// sits in LDS.  The odd-k instances against the two launches they replace,
// cold: E = 256, T = 128 .. 4096, 7.0-11.6 against 12.0-15.2 us; E = 64,
// T = 128 and 512, 6.8-7.7 against 11.7-13.8 us; bit-identical.
bool fused_k(int k) { return k >= 1 && k <= 8; }

FusedFn fused_for(int k) {
  switch (k) {
    case 1: return layout_fused_kernel<1>;
    case 2: return layout_fused_kernel<2>;
    case 3: return layout_fused_kernel<3>;
    case 4: return layout_fused_kernel<4>;
    case 5: return layout_fused_kernel<5>;
    case 7: return layout_fused_kernel<7>;
    case 6: return layout_fused_kernel<6>;
    case 8: return layout_fused_kernel<8>;
    default: return nullptr;
  }
}

size_t fused_lds_bytes(int T, int k, int E) {
  const int64_t N = (int64_t)T * k;
  const int64_t nchunks = (N + kFusedChunk - 1) / kFusedChunk;
  return (size_t)(nchunks + kFusedWaves + 1) * E * sizeof(int32_t);
}

// Path choice, from measurements on MI355X (one launch costs at least about
// 4.5 us here, whatever it does):
//  - the one-launch path, whose every workgroup histograms all T*k ids with
//    LDS atomics, costs 4.6 us at 1 chunk, 8.6 us at 32 and 12.9 us at 64
//    chunks of 1024 entries with E = 256, but 21.9 us at 96 chunks with
//    E = 64 and skewed routing, where the atomics of a 64-lane step collide
//    on a few addresses (with E <= 64 some always do);
//  - the two-launch path costs 10.4 to 12.4 us over the same range.
// So: one launch up to a few chunks, and up to 64 chunks when E > 64.
// Past 12288 tokens the one-launch kernel's cost grows with the tokens, not
// the entries, and the two launches win at any k (cold, E = 128 / 256:
// k = 2, T = 32768 19.7 / 20.0 against 14.3 / 15.4 us, T = 20000 15.0 /
// 15.4 against 14.2 / 15.1; k = 4, T = 16384 16.6 / 17.4 against 14.4 /
// 15.9), while up to it the one launch stays ahead (k = 4, T = 12288
// 14.2 / 14.8 against 14.5 / 15.6; k = 8, T = 6144 13.3 / 13.6 against
// 15.2 / 16.4).
#ifndef EP_LAYOUT_FUSED_MAX_CHUNKS
#define EP_LAYOUT_FUSED_MAX_CHUNKS 64
#endif
constexpr int64_t kFusedFewChunks = 4;
constexpr int kFusedMinExperts = 65;  // one launch past a few chunks only above this many experts
constexpr int kFusedMaxTokens = 12288;  // and for at most this many tokens
// The two-launch path reads the whole (chunk, expert) table in every
// workgroup; past this many counts the three-launch path scans it first.
// Cold, us, two against three launches: 64 Ki counts (E = 128 / 512 /
// 1024, k = 8, T = 65536 / 16384 / 8192) 28.2 / 21.3 / 21.2 against 25.1 /
// 19.7 / 19.4; 32 Ki counts (E = 256 / 1024 / 64, k = 8 / 2 / 8) 18.1 /
// 17.5 / 22.9 against 18.8 / 17.6 / 24.3.  At 128 Ki the three launches
// take 19-26 us.
constexpr int64_t kRankTableMax = 48 * 1024;

enum class Path { Fused, Two, Three };

Path layout_path(int T, int k, int E) {
  if (T <= 0) return Path::Fused;
  const int64_t N = (int64_t)T * k;
  const int64_t nf = (N + kFusedChunk - 1) / kFusedChunk;
  const bool fits = fused_lds_bytes(T, k, E) <= 144 * 1024;
  if (fused_k(k) && fits &&
      (nf <= kFusedFewChunks || (E >= kFusedMinExperts && nf <= EP_LAYOUT_FUSED_MAX_CHUNKS && T <= kFusedMaxTokens)))
    return Path::Fused;
  const int64_t ct = kChunkEntries / k;
  const int64_t nch = (T + ct - 1) / ct;
  if (nch * E <= kRankTableMax) return Path::Two;
  return Path::Three;
}

}  // namespace

int layout_chunk_tokens(int k) { return kChunkEntries / k; }

int layout_num_chunks(int T, int k) {
  const int ct = layout_chunk_tokens(k);
  return (T + ct - 1) / ct;
}

size_t layout_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || layout_path(T, k, E) == Path::Fused) return 0;
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
  const Path path = layout_path(T, k, E);
  if (path == Path::Fused) {
    const int N = T * k;
    const int nchunks = (N + kFusedChunk - 1) / kFusedChunk;
    const size_t lds = fused_lds_bytes(T, k, E);
    // an empty batch only writes zero counts and offsets: any instance does
    FusedFn fn = fused_for(T > 0 ? k : 1);
    if (!fn) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
      hipError_t e = allow_dynamic_lds((const void*)fn, lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(nchunks > 0 ? nchunks : 1), dim3(kFusedThreads), lds, stream, idx, T, k, E, nbits,
                       nchunks, counts, offsets, dest_row, src_token, status);
    return hipGetLastError();
  }
  const int ct = layout_chunk_tokens(k);
  const int nch = layout_num_chunks(T, k);  // T > 0 here

  int32_t* chunk_counts = static_cast<int32_t*>(workspace);
  size_t cb = (size_t)nch * E * sizeof(int32_t);
  cb = (cb + 255) & ~(size_t)255;
  int32_t* chunk_status = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cb);
  {
    const size_t lds = (size_t)(E + ct * k) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_count_kernel, dim3(nch), dim3(kCountThreads), lds, stream, idx, T, k, E, nbits, ct,
                       chunk_counts, chunk_status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (path == Path::Three) {
    hipLaunchKernelGGL(layout_colscan_kernel, dim3((E + kWave - 1) / kWave), dim3(1024), 0, stream, chunk_counts, nch,
                       E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const size_t lds = rank_lds_bytes(E, epad);
  if (lds > 64 * 1024) {
    hipError_t e = allow_dynamic_lds((const void*)layout_rank_kernel, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(layout_rank_kernel, dim3(nch), dim3(1024), lds, stream, idx, T, k, E, nbits, epad, ct, nch,
                     path == Path::Three ? 1 : 0, chunk_counts, chunk_status, counts, offsets, dest_row, src_token,
                     status);
  return hipGetLastError();
}

}  // namespace ep
