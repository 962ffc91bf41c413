/*
 * The C ABI used from C: plain device pointers from hipMalloc, the null
 * stream, no Python.  A small routing is laid out, dispatched and combined;
 * the results are checked through properties that hold at any size, with no
 * oracle:
 *   - layout: counts sum to T*k, offsets are their exclusive prefix sum,
 *     dest_row is a bijection onto [0, T*k), src_token[dest_row[t,j]] = t,
 *     and tokens ascend inside each expert segment;
 *   - dispatch: recv[dest_row[t,j]] equals x[t] bit for bit;
 *   - combine with the identity expert and weights summing to 1 (here 1/k
 *     for k = 4, exact in fp32): combine(dispatch(x)) == x bit for bit, since
 *     each bf16 row times 1/4, four times added, is exact;
 *   - ep_layout_dispatch with NULL src_token and status gives the same
 *     dest_row and receive rows as the two separate calls.
 * Prints "c_abi_roundtrip: ok" and exits 0 on success, prints the first
 * failure and exits 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define T 300
#define K 4
#define E 80 /* 65..256 experts and 1200 entries: ep_layout_dispatch runs as one wide launch */
#define H 1032 /* not a multiple of 512 elements: ragged slabs */

static int fail(const char* what) {
  printf("c_abi_roundtrip: FAILED: %s\n", what);
  return 1;
}

#define HIP_OK(x)                                                   \
  do {                                                              \
    if ((x) != hipSuccess) return fail("HIP call " #x);             \
  } while (0)

#define EP_CALL(x)                                                           \
  do {                                                                       \
    int rc_ = (x);                                                           \
    if (rc_ != EP_OK) {                                                      \
      printf("c_abi_roundtrip: %s -> %d (%s)\n", #x, rc_, ep_last_error()); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static uint32_t lcg(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return *s >> 8;
}

int main(void) {
  static int32_t idx[T * K], counts[E], offsets[E + 1], dest[T * K], src[T * K], status;
  static uint16_t x[T * H], recv[T * K * H], out[T * H], recv2[T * K * H];
  static int32_t dest2[T * K];
  static float w[T * K];
  uint32_t seed = 12345u;

  /* k distinct experts per token, weights 1/k */
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K; ++j) {
      int e, dup;
      do {
        e = (int)(lcg(&seed) % E);
        dup = 0;
        for (int j2 = 0; j2 < j; ++j2) dup |= idx[t * K + j2] == e;
      } while (dup);
      idx[t * K + j] = e;
      w[t * K + j] = 1.0f / K;
    }
  }
  /* bf16 with exponents 120..130 (magnitudes 2^-7 .. 2^4): x/4 and every
     partial sum j*x/4 stay normal and exact in fp32 */
  for (int i = 0; i < T * H; ++i) {
    const uint32_t sign = lcg(&seed) & 1u, ex = 120u + lcg(&seed) % 11u, man = lcg(&seed) & 0x7Fu;
    x[i] = (uint16_t)((sign << 15) | (ex << 7) | man);
  }

  int32_t *d_idx, *d_counts, *d_offsets, *d_dest, *d_src, *d_status;
  float* d_w;
  void *d_x, *d_recv, *d_out, *d_ws = NULL;
  HIP_OK(hipMalloc((void**)&d_idx, sizeof idx));
  HIP_OK(hipMalloc((void**)&d_counts, sizeof counts));
  HIP_OK(hipMalloc((void**)&d_offsets, sizeof offsets));
  HIP_OK(hipMalloc((void**)&d_dest, sizeof dest));
  HIP_OK(hipMalloc((void**)&d_src, sizeof src));
  HIP_OK(hipMalloc((void**)&d_status, sizeof status));
  HIP_OK(hipMalloc((void**)&d_w, sizeof w));
  HIP_OK(hipMalloc(&d_x, sizeof x));
  HIP_OK(hipMalloc(&d_recv, sizeof recv));
  HIP_OK(hipMalloc(&d_out, sizeof out));
  size_t ws = ep_layout_workspace_bytes(T, K, E);
  if (ws) HIP_OK(hipMalloc(&d_ws, ws));
  HIP_OK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

  EP_CALL(ep_layout(d_idx, T, K, E, d_counts, d_offsets, d_dest, d_src, d_status, d_ws, ws, NULL));
  EP_CALL(ep_dispatch(d_x, T, H, d_dest, K, d_recv, (int64_t)T * K, NULL));
  EP_CALL(ep_combine(d_recv, (int64_t)T * K, H, d_dest, d_w, T, K, d_out, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(offsets, d_offsets, sizeof offsets, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dest, d_dest, sizeof dest, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(src, d_src, sizeof src, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&status, d_status, sizeof status, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(recv, d_recv, sizeof recv, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

  if (status != 0) return fail("status word set for valid routing");
  int64_t sum = 0;
  for (int e = 0; e < E; ++e) {
    if (offsets[e] != sum) return fail("offsets are not the prefix sum of counts");
    sum += counts[e];
  }
  if (sum != T * K || offsets[E] != T * K) return fail("counts do not sum to T*k");
  static char seen[T * K];
  memset(seen, 0, sizeof seen);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K; ++j) {
      int r = dest[t * K + j], e = idx[t * K + j];
      if (r < offsets[e] || r >= offsets[e + 1]) return fail("dest_row outside its expert's segment");
      if (seen[r]++) return fail("dest_row is not a bijection");
      if (src[r] != t) return fail("src_token[dest_row] != token");
      if (memcmp(recv + (size_t)r * H, x + (size_t)t * H, H * sizeof(uint16_t)) != 0)
        return fail("dispatched row differs from its source row");
    }
  }
  for (int e = 0; e < E; ++e)
    for (int r = offsets[e] + 1; r < offsets[e + 1]; ++r)
      if (src[r] <= src[r - 1]) return fail("tokens do not ascend inside a segment");
  if (memcmp(out, x, sizeof out) != 0) return fail("combine(dispatch(x)) != x");

  /* the one-call form, without the optional outputs, on fresh buffers */
  HIP_OK(hipMemset(d_dest, 0xFF, sizeof dest));
  HIP_OK(hipMemset(d_recv, 0, sizeof recv));
  EP_CALL(ep_layout_dispatch(d_idx, T, K, E, d_x, H, d_counts, d_offsets, d_dest, NULL, NULL, d_ws, ws, d_recv,
                             (int64_t)T * K, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(dest2, d_dest, sizeof dest2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(recv2, d_recv, sizeof recv2, hipMemcpyDeviceToHost));
  if (memcmp(dest2, dest, sizeof dest) != 0) return fail("ep_layout_dispatch dest_row differs");
  if (memcmp(recv2, recv, sizeof recv) != 0) return fail("ep_layout_dispatch receive rows differ");

  hipFree(d_idx); hipFree(d_counts); hipFree(d_offsets); hipFree(d_dest); hipFree(d_src);
  hipFree(d_status); hipFree(d_w); hipFree(d_x); hipFree(d_recv); hipFree(d_out);
  if (d_ws) hipFree(d_ws);
  printf("c_abi_roundtrip: ok\n");
  return 0;
}
