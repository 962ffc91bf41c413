/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE row-movement library, libep.so.
 *
 * The library moves bf16 hidden-state rows between token order and an
 * expert-grouped receive buffer on one GPU:
 *
 *   ep_layout   per-expert counts, their prefix sum, and the destination row
 *               of every (token, slot) entry;
 *   ep_dispatch copy each token's row to its k destination rows;
 *   ep_combine  gather each token's k expert-output rows back as a
 *               gate-weighted sum (fp32 accumulate, bf16 out).
 *
 * Sources.  "How DeepEP Utilizes TMA Instructions for Minimal SM Usage on
 * Hopper GPUs" (instagit.com DeepEP deep-dive; cited as [DeepEP-TMA]),
 * section "High-Level DeepEP API Usage", shows the dispatch call this ABI
 * splits into ep_layout (its handle) and ep_dispatch (its output); section
 * "Asynchronous Copy Primitives" shows the staged row copy; section
 * "Minimal SM Occupancy Configuration" the knob that caps the compute units
 * the copy kernels use.  The pages define neither the grouping order nor a
 * combine; the readings taken are stated at each entry point.
 *
 * Conventions shared by every entry point:
 *   - all tensor pointers are DEVICE pointers into memory the caller owns;
 *     the library never allocates, frees or retains them;
 *   - bf16 tensors are row-major with H elements per row, H % 8 == 0, and
 *     16-byte aligned base pointers (rows are moved as 16-byte vectors);
 *   - int32/float tensors are row-major and 4-byte aligned;
 *   - `stream` is a hipStream_t handle (NULL = the default stream); every
 *     call only enqueues work on it and returns without synchronising;
 *   - a negative return is a host-detected error: nothing was enqueued and
 *     ep_last_error() holds a message for the calling thread;
 *   - T == 0 enqueues nothing and returns EP_OK (after argument checks),
 *     except ep_layout, which still writes zero counts and offsets and a
 *     zero status word.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = -1, /* null pointer, negative or oversized count, k > E, H % 8 != 0 */
  EP_ERR_ALIGNMENT = -2,   /* a bf16 tensor not 16-byte aligned, an int/float one not 4-byte aligned */
  EP_ERR_UNSUPPORTED = -3, /* device is not gfx950, or an unknown variant name */
  EP_ERR_WORKSPACE = -4,   /* workspace missing or smaller than ep_layout_workspace_bytes() */
  EP_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
};

/* bits of the device status word written by ep_layout */
enum {
  EP_STATUS_EXPERT_OUT_OF_RANGE = 1, /* some topk_idx entry is outside [0, E) */
  EP_STATUS_DUPLICATE_EXPERT = 2     /* some token lists the same expert twice */
};

#define EP_MAX_TOPK 32
#define EP_MAX_EXPERTS 1024

/*
 * Largest count of (token, slot) entries (T*k), of receive rows, and of
 * 512-element row slabs (T*ceil(H/512) and recv_rows*ceil(H/512)) that a
 * call accepts: 2^31 - 1 - 2^22.  The kernels count their work in 32-bit
 * integers and may step one grid stride past the last unit before they
 * stop; the margin keeps that step from wrapping.  At H = 512 the slab
 * bound is a 2 TiB buffer, beyond any single device.
 */
#define EP_MAX_ENTRIES 2143289343

/*
 * Compute-unit budget of the copy kernels, after [DeepEP-TMA] section
 * "Minimal SM Occupancy Configuration" (a process-wide cap on the SMs the
 * communication kernels occupy).  n > 0: dispatch, combine and the probes
 * launch a persistent grid of n workgroups, each holding more than half a
 * CU's LDS so that no two share a CU (the hardware spreads consecutive
 * workgroups over the 8 XCDs); n is clamped to the device's CU count at
 * launch.  n == 0: no budget; the library picks the launch per kernel --
 * an ordinary grid over the whole device, except that a dispatch of at
 * least 8 tokens per CU (variant "auto"; any size on a budget)
 * runs the workgroup-phased register kernel ("vgpr_wg") with whole-row
 * slabs as a persistent grid on every CU it may use: its streaming loads of
 * x take the same time whether or not x is still in the Infinity Cache;
 * "auto" keeps its smaller batches on an ordinary grid.  With another
 * variant named, a dispatch of at least 32 work units per CU of its default
 * budget runs persistent on that budget: 64 CUs for k >= 5 (at k = 8 its
 * traffic is 8/9 writes, and HBM write throughput peaks with about a
 * quarter of the CUs issuing them), 96 for k = 2..4 and 128 for k = 1,
 * whose larger read share needs more CUs in flight.  The initial value comes from the environment variable
 * EP_NUM_CUS (default 0).
 * On a CU-masked stream (ep_stream_create_cu_masked, or any stream whose
 * mask hipExtStreamGetCUMask reports) every launch counts only the CUs of
 * the mask: n and the default dispatch budget are clamped to them, ordinary
 * grids are sized for them, and the kernel choices that depend on the CU
 * count (the phased combine needs at least half the device) use them.
 * Returns EP_OK, or EP_ERR_INVALID_ARG for n < 0 or n > 4096.
 */
int ep_set_num_cus(int n);
int ep_get_num_cus(void);

/*
 * Kernel variant for dispatch and combine (process-wide):
 *   "auto"  the default choice per shape.  A dispatch of at least 8 tokens
 *           per CU of its launch runs "vgpr_wg" as a persistent grid on
 *           every CU it may use, with whole-row slabs and streaming loads of
 *           x.  Its time hardly depends on whether x is still cached
 *           (T = 16384, H = 7168, k = 6: about 310 us on the whole device,
 *           about 670 us on 24 CUs, evicted or not).  "lds1" (64 CUs) and
 *           "pc" (the budget's CUs) load x with cacheable loads: faster
 *           while x is in the Infinity Cache (about 258 us on 64 CUs, 645 us
 *           on 24), much slower once it is not (about 650 and 975 us), so a
 *           caller that has just written x may prefer them.  Smaller
 *           batches on every CU take "vgpr2" on an ordinary grid from 2
 *           tokens per CU (4 for rows of at most 8 KiB), which also streams
 *           x; rows of 8 to 16 KiB that are not a whole number of KiB take
 *           "vgpr_wg" on that ordinary grid instead at k = 6 and 8.  The
 *           smallest batches take "lds1".  On a CU budget every batch
 *           size takes "vgpr_wg" on the budget's CUs; on a CU-masked stream
 *           without a budget, batches below 8 tokens per CU take "lds1" on
 *           an ordinary grid sized to the mask;
 *   "vgpr"  rows staged in registers, one load feeding k stores (dispatch)
 *           or k loads feeding one store (combine);
 *   "vgpr2" the same with the next work unit's loads issued before the
 *           current unit's stores (register double buffer);
 *   "lds1"  rows staged in a per-wave LDS slice by direct-to-LDS loads,
 *           one stage;
 *   "lds2"  the same with two stages per wave: the next unit's
 *           direct-to-LDS load is in flight while the current one is stored;
 *   "phase" reads before writes, per wave: for combine each wave sums up
 *           to 16 KiB of output rows (28 KiB in 8-wave workgroups) in
 *           registers and stores them only after all their source rows are
 *           read; for dispatch each wave loads up to 16 KiB of x rows into
 *           registers, then writes their k copies.  With one such unit per
 *           wave the whole grid reads first and writes last.  k must be
 *           at most 8 for combine (else the any-k register kernel runs) and
 *           2, 4, 6 or 8 for dispatch (else lds1).  "auto" picks it for
 *           combine on at least half the device when each launch fills two
 *           thirds of a full grid (with every CU and units of at most
 *           16 KiB per wave: 9/20 at k >= 3, 3/5 at k <= 2; with two rows
 *           per wave: 23/25 at k = 5, 3/4 at k = 7, 7/10 at k = 8), at
 *           k <= 4 reading runs of 2 vectors per source row where the row
 *           allows them;
 *   "lds3"  (dispatch; combine takes its default) three stages per wave:
 *           the next two units' direct-to-LDS loads are in flight while the
 *           current one is stored (fewer waves fit a CU);
 *   "pc"    (dispatch; combine takes its default) producer/consumer: one
 *           wave per workgroup issues every direct-to-LDS load into a
 *           two-slot ring and 3 to 8 consumer waves store the slabs, in
 *           step through workgroup barriers (the elected issuer of
 *           [DeepEP-TMA] "Asynchronous Copy Primitives" as a whole wave);
 *           always a persistent grid of one workgroup per CU;
 *   "vgpr_wg" (dispatch; combine takes its default) "vgpr" with each
 *           workgroup in step: every wave loads four slabs (two of 16 KiB)
 *           and waits for them, the workgroup (4 waves) meets at a barrier,
 *           then every wave stores.  A CU's loads then do not queue behind
 *           its own stores, and each CU alternates a few long read and
 *           write bursts.  On at least half the device a call is split into
 *           one launch per such trip (a launch boundary starts every CU's
 *           read burst together); on fewer CUs it is one persistent launch.
 * lds2, lds3 and phase need k in {2, 4, 6, 8}; for other k dispatch runs lds1.
 * Returns EP_OK or EP_ERR_UNSUPPORTED for an unknown name.
 */
int ep_set_variant(const char* name);
const char* ep_get_variant(void);

/*
 * Staging geometry (process-wide): the row slab a wave moves per work unit,
 * in 16-byte vectors per lane (one vector per lane = 1 KiB per wave).
 * 0 = each kernel's default (dispatch: "vgpr_wg" the whole row up to
 * 16 KiB, else 16 KiB slabs where they divide the row and 14 KiB slabs
 * otherwise, the last one partial; "vgpr2" and "pc" the whole row up
 * to 14 KiB; the LDS-staged kernels the whole row up to 8 KiB, else slabs
 * of at most 8 KiB -- half rows at H = 7168; combine: 2 KiB per source
 * row).  Accepted: 0, 1, 2, 4, 7, 8, 14, 16; a kernel
 * rounds a value down to the sizes it is compiled for (combine: 1, 2, 4).
 * The choice changes only speed, never results.  Returns EP_OK or
 * EP_ERR_UNSUPPORTED.
 */
int ep_set_slab(int vectors_per_lane);
int ep_get_slab(void);

/* Bytes of scratch ep_layout needs for (T, k, E); 0 for T == 0. */
size_t ep_layout_workspace_bytes(int T, int k, int E);

/*
 * ep_layout -- the routing handle of a dispatch ([DeepEP-TMA] "High-Level
 * DeepEP API Usage": dispatch takes topk_idx and num_experts and returns a
 * handle for the way back).
 *
 * Entries are the T*k (token, slot) pairs in row-major order.  Output:
 *   counts[e]       number of entries with topk_idx == e           [E]
 *   offsets[e]      sum of counts[0..e-1]; offsets[E] = total      [E+1]
 *   dest_row[t*k+j] offsets[e] + (number of earlier entries, in row-major
 *                   order, with the same expert e), i.e. a stable
 *                   counting sort: tokens ascend inside each expert
 *                   segment; -1 for an entry whose expert is out of range [T*k]
 *   src_token[r]    the token whose row lands in receive row r, for
 *                   r < offsets[E]; entries beyond are not written;
 *                   may be NULL                                      [T*k]
 *   status[0]       OR of EP_STATUS_* bits (0 when all ids are valid and
 *                   distinct per token); always written when non-NULL.
 * An out-of-range id is skipped (not counted, dest_row -1).  A repeated id
 * inside one token is flagged but still placed as its own entry.
 * workspace: device scratch of at least ep_layout_workspace_bytes(T, k, E)
 * bytes, 16-byte aligned, owned by the caller, clobbered by the call.
 * Limits: 1 <= k <= EP_MAX_TOPK, k <= E <= EP_MAX_EXPERTS, T*k <= EP_MAX_ENTRIES.
 */
int ep_layout(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
              int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * ep_layout_noalloc -- ep_layout for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (without the
 * workspace), outputs, limits and errors as ep_layout, with identical
 * results.  Where ep_layout needs scratch (ep_layout_workspace_bytes > 0:
 * the two- and three-launch paths for larger batches), this call uses a
 * static device array of EP_LAYOUT_NOALLOC_MAX_SCRATCH bytes inside the
 * library instead; each GPU the library runs on holds its own copy until
 * the process ends.  A batch whose scratch would exceed it returns
 * EP_ERR_WORKSPACE before anything is enqueued (ep_layout with a workspace
 * handles it).  The call allocates nothing, frees nothing and makes no
 * memset: the layout overwrites every scratch entry it later reads, so the
 * previous call's contents do not matter.  All calls on one GPU share its
 * array: calls that may overlap on one GPU (on different streams without
 * ordering between them, or from several threads) race and must be
 * serialised by the caller.
 */
#define EP_LAYOUT_NOALLOC_MAX_SCRATCH ((size_t)4 << 20)
int ep_layout_noalloc(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                      int32_t* dest_row, int32_t* src_token, int32_t* status, void* stream);

/*
 * ep_dispatch -- recv[dest_row[t*k+j], :] = x[t, :] for all t < T, j < k
 * (bit copy).  The row copy of [DeepEP-TMA] section "Asynchronous Copy
 * Primitives": each source row is read once into an on-chip slice and
 * written to each of its k destinations.
 *   x         bf16 [T, H]
 *   dest_row  int32 [T, k], normally from ep_layout
 *   recv      bf16 [recv_rows, H]; an entry whose dest_row is outside
 *             [0, recv_rows) is skipped; rows nobody targets are untouched.
 * With valid, distinct routing recv_rows = T*k covers every entry.
 * Limits: 1 <= k <= EP_MAX_TOPK, 0 <= recv_rows <= EP_MAX_ENTRIES,
 * T*k <= EP_MAX_ENTRIES, and T and recv_rows times ceil(H/512) at most
 * EP_MAX_ENTRIES.
 */
int ep_dispatch(const void* x, int T, int H, const int32_t* dest_row, int k, void* recv,
                int64_t recv_rows, void* stream);

/*
 * ep_layout_dispatch -- ep_layout followed by ep_dispatch, with identical
 * outputs, in one launch where that is faster (the low-latency kernel
 * family of [DeepEP-TMA], "TMA Implementation Across Kernel Types", and its
 * use for wide batches):
 *   - up to 64 Ki entries with k in {2, 4, 6, 8} and 65 <= E <= 256, while
 *     the dispatch variant is "auto" or "lds1": a persistent grid on the
 *     dispatch's compute units in which every workgroup histograms all ids
 *     and then ranks and copies its own range of tokens (decode batches
 *     included, where launches rather than bytes set the time);
 *   - other batches of T*k <= 1024 entries: a grid in which every
 *     workgroup lays out all the entries and copies its share.
 * Other batches run ep_layout and ep_dispatch in order on the stream.
 * Arguments as for ep_layout and ep_dispatch (x bf16 [T, H], recv bf16
 * [recv_rows, H]); the workspace must be given whenever ep_layout needs one
 * for these sizes (ep_layout_workspace_bytes), whichever path runs.
 */
int ep_layout_dispatch(const int32_t* topk_idx, int T, int k, int E, const void* x, int H, int32_t* counts,
                       int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* recv, int64_t recv_rows, void* stream);

/*
 * ep_dispatch_rows -- the same copy in gather form:
 *   recv[r, :] = x[src_token[r], :] for r < recv_rows
 * with src_token from ep_layout (then recv_rows = offsets[E]); rows whose
 * src_token is outside [0, T) are untouched.  With a layout of valid ids
 * the result equals ep_dispatch's.  The receive buffer is written as one
 * sequential stream and each token row is read k times (from the caches
 * when x fits in them); which form is faster depends on the shape.
 *   x          bf16 [T, H]
 *   src_token  int32 [recv_rows]
 *   recv       bf16 [recv_rows, H]
 * Limits: 0 <= recv_rows <= EP_MAX_ENTRIES, and T and recv_rows times
 * ceil(H/512) at most EP_MAX_ENTRIES.  The variant "vgpr_cached" selects
 * streaming (non-temporal) loads of x; every other keeps them cacheable.
 */
int ep_dispatch_rows(const void* x, int T, int H, const int32_t* src_token, void* recv, int64_t recv_rows,
                     void* stream);

/*
 * ep_combine -- the way back from the expert-grouped layout, which the
 * pages do not spell out; the plainest reading is used:
 *   out[t, :] = bf16_rne( sum_{j=0..k-1} w[t, j] * f32(y[dest_row[t*k+j], :]) )
 * accumulated in fp32 from +0.0, j ascending, each product and each sum
 * rounded separately (never fused), then rounded once to bf16 (round to
 * nearest even).  An entry whose dest_row is outside [0, recv_rows)
 * contributes nothing.  Weights are used as given (not renormalised).
 *   y         bf16 [recv_rows, H] expert outputs in the ep_layout order;
 *             may be NULL when recv_rows == 0
 *   dest_row  int32 [T, k]
 *   topk_w    float32 [T, k]
 *   out       bf16 [T, H]
 * With recv_rows == 0 (a receive buffer sized from offsets[E] when no id
 * was valid) every slot is out of range: out is filled with +0.0 and y is
 * never read.
 * Limits as ep_dispatch.
 */
int ep_combine(const void* y, int64_t recv_rows, int H, const int32_t* dest_row, const float* topk_w,
               int T, int k, void* out, void* stream);

/*
 * ep_combine_reduce -- the same combine computed from the expert side by
 * reduce-on-store: the bulk store that adds element-wise into its global
 * destination, described in "TMA study notes" (mkbk-pku.cn, cited as
 * [TMA-notes]), section "TMA 的其他特性（单卡 / Cluster 内）", item 3.  gfx950 has no
 * such store, so the addition is an fp32 atomic per element:
 *   acc[t, :] = 0;  for r < recv_rows with t = src_token[r] in [0, T) and a
 *   slot j with dest_row[t*k+j] == r:  acc[t, :] += w[t, j] * f32(y[r, :]);
 *   out[t, :] = bf16_rne(acc[t, :])
 * y is read once, as one sequential stream in receive-row order; each
 * accumulator element takes k atomic additions.  The order of those
 * additions is not fixed, so the result is the fp32 sum of the k products
 * in SOME order (each product rounded separately, never fused), rounded
 * once to bf16: within fp32 rounding of ep_combine's result, but not always
 * bit-identical to it and not bit-reproducible from call to call.  Rows
 * whose src_token is outside [0, T), or whose token does not list them in
 * dest_row (entries of src_token beyond offsets[E] that ep_layout left
 * unwritten), add nothing.
 *   y          bf16 [recv_rows, H] expert outputs in the ep_layout order
 *   src_token  int32 [recv_rows] from ep_layout
 *   dest_row   int32 [T, k] from ep_layout
 *   topk_w     float32 [T, k]
 *   out        bf16 [T, H]
 *   workspace  device scratch of at least ep_combine_reduce_workspace_bytes
 *              (T, H) = 4*T*H bytes (the fp32 accumulator), 16-byte
 *              aligned, owned by the caller, clobbered by the call
 * Three launches on `stream` (zero, scatter-add, convert).  Limits as
 * ep_combine; a missing or short workspace returns EP_ERR_WORKSPACE.
 */
size_t ep_combine_reduce_workspace_bytes(int T, int H);
int ep_combine_reduce(const void* y, int64_t recv_rows, int H, const int32_t* src_token, const int32_t* dest_row,
                      const float* topk_w, int T, int k, void* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Static text for a return code. */
const char* ep_status_string(int code);
/* Detail of the calling thread's last negative return ("" if none). */
const char* ep_last_error(void);

/*
 * Measurement helpers (not part of the routing path).
 *
 * ep_bw_probe: a plain streaming kernel under the same compute-unit budget
 * as dispatch/combine, giving the achievable HBM ceiling at that budget.
 * `mode` packs three fields:
 *   bits [2:0]  operation: 0 copy dst[i] = src[i] (reads and writes `bytes`);
 *               1 read src (dst must hold 16 bytes; written only for one
 *               improbable checksum, which keeps the reads alive);
 *               2 write a pattern to dst (src unused);
 *               3 read src into per-wave LDS slices with direct-to-LDS loads
 *               (dst as for 1);
 *               4 mixed 8:1 -- read `bytes` of src, write bytes/8 of dst
 *               (each wave: 8 KiB in, 1 KiB out);
 *               5 mixed 1:8 -- read bytes/8 of src, write `bytes` of dst
 *               (each wave: 1 KiB in, 8 KiB out);
 *               6 mixed 8:1 in bursts -- as 4, but each wave reads 64 KiB
 *               and then writes 8 KiB;
 *               7 mixed in phases, on one workgroup of 16 waves per CU
 *               whatever the budget: with depth field 0, 8:1 as 4, each
 *               wave reading 128 KiB and then writing 16 KiB; with depth
 *               field 1, 1:8 as 5, each wave reading 16 KiB and then
 *               writing it 8 times (copy r has r xor-ed into the first
 *               word of each 16-byte vector); with bytes = 128 KiB x waves
 *               each wave does this once, so the grid reads first and
 *               writes last; with depth field 2, the 8:1 form once per
 *               wave with a bounded wait (at most 20 us) for every
 *               workgroup's reads to finish before any writes (bytes above
 *               128 KiB x waves fail with EP_ERR_HIP);
 *               4 and 5 need bytes % 8192 == 0, 6 bytes % 65536 == 0,
 *               7 bytes % 131072 == 0; 4-6 ignore depth, 4-7 policy
 *   bits [5:4]  depth: 16-byte vectors in flight per lane, 0 -> 8, 1 -> 16,
 *               2 -> 32 (3 is invalid)
 *   bits [10:8] cache policy of the loads of operations 1 and 3: 0 nt,
 *               1 none, 2 sc0, 3 sc1, 4 sc0+sc1, 5 nt (policies 1-5 use
 *               buffer loads)
 * bytes % 16 == 0, pointers 16-byte aligned.
 */
int ep_bw_probe(int mode, const void* src, void* dst, int64_t bytes, void* stream);

/*
 * ep_inflight_probe: the per-CU read ceiling and the load latency behind it.
 * A persistent grid of one workgroup of waves_per_cu (1..16; 1..8 with 16
 * vectors per lane) waves per CU of
 * the budget (every CU when ep_get_num_cus() == 0) streams reads over
 * `bytes` of src (streaming nt loads; cacheable ones with cached = 1), each wave keeping vectors_per_lane (1, 2, 4, 8 or 16) to
 * twice that many 16-byte vectors per lane in flight (the next batch is
 * issued before the current one is consumed).  With hops > 0, wave 0 of
 * workgroup 0 does not stream: it follows `hops` links of `chain` (int64
 * element i holds the index of the next element; an index outside
 * [0, chain_len) restarts the walk at 0), one dependent vector load at a
 * time, and writes out[0] = elapsed 100 MHz real-time ticks, out[1] =
 * elapsed shader-clock cycles, out[2] = the last index, out[3] = HW_ID
 * (low 32 bits) and XCC id (bits 32..35) of its CU.  With bytes == 0 the
 * chase runs on an otherwise idle device (unloaded latency).  sink holds
 * 16 bytes and is written only for an improbable checksum.  Returns EP_OK,
 * EP_ERR_INVALID_ARG, EP_ERR_ALIGNMENT or EP_ERR_HIP.
 */
int ep_inflight_probe(int waves_per_cu, int vectors_per_lane, int cached, const void* src, int64_t bytes, void* sink,
                      const int64_t* chain, int64_t chain_len, int64_t hops, int64_t* out, void* stream);

/*
 * ep_probe_placement: launch min(n_groups, budget) workgroups that each
 * need more than half a CU's LDS (budget = the CU count when
 * ep_get_num_cus() > 0, else n_groups), each holding its CU for ~50 us, and
 * have workgroup g write {XCC id, SE id, (SH << 4) | CU id, raw HW_ID} as 4
 * int32 to out[4g .. 4g+3].  out holds 4 * n_groups int32 (device memory).
 * Returns the number of workgroups launched, or a negative code.
 */
int ep_probe_placement(int32_t* out, int n_groups, void* stream);

/*
 * ep_mfma_probe: a compute-bound kernel to run beside the copy kernels (the
 * computation that [DeepEP-TMA] "Minimal SM Occupancy Configuration" keeps
 * the remaining units free for).  n_groups workgroups of 4 waves; each wave
 * runs `iters` rounds of four 32x32x8 bf16 matrix-core products on register
 * operands, 4 x 16384 flop per round, with no memory traffic, so its
 * throughput follows the compute units it gets.  out is device memory of
 * 256 * n_groups floats that is written only if the products sum to an
 * impossible value (it keeps the work live).  Returns EP_OK,
 * EP_ERR_INVALID_ARG (null out, n_groups outside [1, 65536], iters < 0),
 * EP_ERR_ALIGNMENT or EP_ERR_HIP.
 */
int ep_mfma_probe(int n_groups, int iters, float* out, void* stream);

/*
 * CU-masked streams, for running the copy kernels on a chosen set of compute
 * units beside other work ([DeepEP-TMA] "Minimal SM Occupancy
 * Configuration": the communication kernels keep to a few units so that the
 * rest stay free for computation).
 *
 * ep_stream_create_cu_masked: a new default-priority HIP stream whose
 * kernels may only run on the compute units whose bits are set in
 * mask[0 .. mask_words-1] (bit i of word w = CU 32 w + i in the runtime's
 * CU numbering).  *stream receives the hipStream_t handle; the caller
 * releases it with ep_stream_destroy.  Returns EP_OK, EP_ERR_INVALID_ARG
 * (null pointers, mask_words outside [1, 64], an empty mask) or EP_ERR_HIP.
 * On MI355X (8 XCDs of 32 CUs) the runtime's numbering interleaves the
 * XCDs: bit i selects a CU of XCD i mod 8, so any 8 consecutive bits hold
 * one CU of every XCD and bits 32 apart land on the same XCD (placement
 * measured with ep_probe_placement).  A masked stream's queue runs on every
 * XCD, and the runtime refuses a mask that leaves some XCD without a CU
 * (hipExtStreamCreateWithCUMask reports "out of memory" for the 8-CU mask
 * {0, 32, ..., 224}, all on XCD 0, or for {0, 1, 2, 3}); this call checks
 * that first, with the XCD count the device reports, and returns
 * EP_ERR_INVALID_ARG for such a mask.  Masks built from consecutive bits
 * reach every XCD evenly once they hold 8 or more bits.
 */
int ep_stream_create_cu_masked(const uint32_t* mask, int mask_words, void** stream);
int ep_stream_destroy(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
