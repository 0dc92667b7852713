/*
 * ep_c_example.c -- the C ABI of include/ep.h used from plain C, with no
 * Python and no torch: the caller owns every buffer (hipMalloc here), the
 * library allocates nothing.
 *
 * One layer's routing on one GPU: seeded top-k indices (repeats inside a
 * token allowed), ep_layout, BF16 ep_dispatch, then ep_combine with identity
 * "experts" (the combine reads the dispatched rows back) and weights 1/8, so
 * every output row must equal its input row bit for bit (8 exact halvings
 * summed in binary32; x has no -0, which a combine returns as +0).  The
 * handle's per-expert counts are checked against a host histogram.
 *
 * Build (done by combine_ep_layout_03_amd/build.py next to libep.so):
 *   gcc -std=c11 -D__HIP_PLATFORM_AMD__ -I include -I /opt/rocm/include \
 *       examples/ep_c_example.c -L combine_ep_layout_03_amd -lep \
 *       -L /opt/rocm/lib -lamdhip64 -o examples/ep_c_example
 * Exit status 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      return 2;                                                                        \
    }                                                                                  \
  } while (0)

#define EP_OK_(call)                                                                   \
  do {                                                                                 \
    ep_status s_ = (call);                                                             \
    if (s_ != EP_OK) {                                                                 \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call, ep_status_string(s_)); \
      return 3;                                                                        \
    }                                                                                  \
  } while (0)

/* 32-bit linear congruential generator (Numerical Recipes constants). */
static uint32_t lcg(uint32_t *s) {
  *s = *s * 1664525u + 1013904223u;
  return *s;
}

int main(void) {
  enum { T = 1000, H = 1024, K = 8, E = 64, R = 8 };
  const ep_config cfg = {T, H, K, E, R, EP_DTYPE_BF16, 0};

  if (ep_abi_version() != EP_ABI_VERSION) {
    fprintf(stderr, "ABI %u, header %u\n", ep_abi_version(), EP_ABI_VERSION);
    return 4;
  }
  const int64_t cap = ep_recv_capacity_rows(&cfg);
  const size_t ws_bytes = ep_layout_workspace_bytes(&cfg);
  if (cap != (int64_t)T * K || ws_bytes == 0) {
    fprintf(stderr, "size helpers: cap %lld, workspace %zu\n", (long long)cap, ws_bytes);
    return 4;
  }

  /* host inputs */
  int32_t *idx = malloc(sizeof(int32_t) * T * K);
  float *w = malloc(sizeof(float) * T * K);
  uint16_t *x = malloc(sizeof(uint16_t) * T * H);
  uint16_t *out = malloc(sizeof(uint16_t) * T * H);
  int32_t counts_ref[E], counts[E], rank_counts[R], err = -1;
  if (!idx || !w || !x || !out) return 5;
  uint32_t seed = 12345u;
  memset(counts_ref, 0, sizeof counts_ref);
  for (int p = 0; p < T * K; ++p) {
    idx[p] = (int32_t)(lcg(&seed) >> 8) % E;
    w[p] = 0.125f;
    ++counts_ref[idx[p]];
  }
  for (int i = 0; i < T * H; ++i) {
    /* a normal bf16 value: random sign and mantissa, exponent in [1, 254] */
    const uint32_t r = lcg(&seed);
    const uint32_t ex = 1u + (r >> 8) % 254u;
    x[i] = (uint16_t)(((r >> 31) << 15) | (ex << 7) | (r & 0x7Fu));
  }

  /* device buffers, all owned by the caller */
  int32_t *d_idx, *d_arr;
  float *d_w;
  void *d_x, *d_out, *d_ws, *recv[R];
  HIP_OK(hipMalloc((void **)&d_idx, sizeof(int32_t) * T * K));
  HIP_OK(hipMalloc((void **)&d_w, sizeof(float) * T * K));
  HIP_OK(hipMalloc(&d_x, sizeof(uint16_t) * T * H));
  HIP_OK(hipMalloc(&d_out, sizeof(uint16_t) * T * H));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  for (int r = 0; r < R; ++r) HIP_OK(hipMalloc(&recv[r], sizeof(uint16_t) * (size_t)cap * H));
  /* the handle's arrays in one allocation: E + (E+1) + R + (R+1) + 2*T*K + 1 ints */
  const size_t n_arr = (size_t)E + (E + 1) + R + (R + 1) + 2 * (size_t)T * K + 1;
  HIP_OK(hipMalloc((void **)&d_arr, sizeof(int32_t) * n_arr));
  ep_layout_t h;
  h.expert_counts = d_arr;
  h.expert_offsets = h.expert_counts + E;
  h.rank_counts = h.expert_offsets + E + 1;
  h.rank_offsets = h.rank_counts + R;
  h.slot_of = h.rank_offsets + R + 1;
  h.src_of = h.slot_of + T * K;
  h.error_flag = h.src_of + T * K;

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  HIP_OK(hipMemcpy(d_idx, idx, sizeof(int32_t) * T * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, sizeof(float) * T * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

  /* the path: layout -> dispatch -> (identity experts) -> combine, one stream */
  EP_OK_(ep_layout(&cfg, d_idx, &h, d_ws, stream));
  EP_OK_(ep_dispatch(&cfg, &h, d_idx, d_x, recv, NULL, cap, stream));
  EP_OK_(ep_combine(&cfg, &h, d_idx, (const void *const *)recv, d_w, d_out, cap, stream));
  HIP_OK(hipStreamSynchronize(stream));

  HIP_OK(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(counts, h.expert_counts, sizeof counts, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(rank_counts, h.rank_counts, sizeof rank_counts, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&err, h.error_flag, sizeof err, hipMemcpyDeviceToHost));

  int bad = 0;
  if (err != 0) {
    fprintf(stderr, "device error word %d\n", err);
    bad = 1;
  }
  int64_t rows = 0;
  for (int r = 0; r < R; ++r) rows += rank_counts[r];
  if (rows != (int64_t)T * K) {
    fprintf(stderr, "rank counts sum to %lld\n", (long long)rows);
    bad = 1;
  }
  for (int e = 0; e < E; ++e)
    if (counts[e] != counts_ref[e]) {
      fprintf(stderr, "expert %d: %d rows, expected %d\n", e, counts[e], counts_ref[e]);
      bad = 1;
      break;
    }
  int64_t mismatches = 0;
  for (int i = 0; i < T * H; ++i) mismatches += out[i] != x[i];
  if (mismatches) {
    fprintf(stderr, "%lld output elements differ from the input\n", (long long)mismatches);
    bad = 1;
  }

  HIP_OK(hipStreamDestroy(stream));
  for (int r = 0; r < R; ++r) HIP_OK(hipFree(recv[r]));
  HIP_OK(hipFree(d_arr));
  HIP_OK(hipFree(d_ws));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_x));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_idx));
  free(idx);
  free(w);
  free(x);
  free(out);
  printf("ep_c_example T=%d H=%d k=%d E=%d R=%d: %s\n", T, H, K, E, R, bad ? "FAILED" : "ok");
  return bad;
}
