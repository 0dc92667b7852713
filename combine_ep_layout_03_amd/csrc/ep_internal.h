// ep_internal.h -- launch plans and kernel launchers shared by the HIP
// sources of libep (host validation lives in ep_api.cpp).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "ep.h"

namespace ep {

// Per-rank buffer pointers travel as kernel arguments (by value).
struct RankPtrs {
  void *p[EP_MAX_RANKS];
};
struct RankCPtrs {
  const void *p[EP_MAX_RANKS];
};
struct ScalePtrs {
  float *p[EP_MAX_RANKS];
};

// Layout plan: the P = T*k pairs are cut into C chunks of S pairs; one
// wavefront owns one chunk in both layout kernels.
struct LayoutPlan {
  bool tiny;   // one single-wave workgroup per 64 pairs (P <= kFusedMaxPairs)
  bool small;  // single-workgroup path
  int64_t P;
  int32_t S;  // pairs per chunk (multiple of 64; k * tpc for the router-counted table)
  int32_t C;  // chunks (0: no such plan)
  int32_t tpc;  // router-counted table only: tokens per chunk (one router workgroup each)
  int32_t workgroups;  // launch grid: C (tiny, small) or ceil(C / kLayoutWaves) (two-launch)
  size_t workspace_bytes;  // two-launch: ceil(C/4)*4 * (E + 1) * 4, chunk histograms
                           // [C/4][E+1][4]; one-launch paths: 256 (unused)
};

constexpr int kWave = 64;
constexpr int kLayoutWaves = 4;  // wavefronts per layout workgroup
constexpr int kLayoutMaxChunks = kLayoutWaves * kWave;  // C <= threads of a layout workgroup
constexpr int kLayoutChunk = 512;  // pairs per chunk (= per wavefront) of the two-launch layout
constexpr int kRowWaves = 1;     // wavefronts per dispatch / combine workgroup
// Error-word bits that make a call write nothing: the layout's own findings
// (set before any call that reads the handle).  EP_DEVERR_ROW is checked per
// pair instead, so a row error found by one wave of a call does not change
// what the call's other waves write.
constexpr int32_t kLayoutErrBits = EP_DEVERR_INDEX | EP_DEVERR_INTERNAL;
constexpr int kSmallWaves = 16;  // wavefronts of the single-workgroup layout
constexpr int64_t kSmallMaxPairs = 8192;    // T*k limit of the single-launch layout
constexpr int kSmallMaxExperts = 384;       // E limit of the single-launch layout (LDS <= 64 KB)
constexpr int64_t kFusedMaxPairs = 2048;    // T*k limit of the one-launch layout + dispatch and
                                            // of the one-wave-per-64-pairs layout

LayoutPlan plan_layout(int64_t P, int E);

// The router can count the layout's chunk table itself when one router
// workgroup (kRouteCountWaves waves, four tokens each per step) routes exactly
// one chunk of tpc tokens; then only the scatter kernel follows.  The plan has
// C = 0 where the two-launch layout does not apply (decode and small sizes)
// or E > kRouteCountMaxExperts.  C <= kLayoutMaxChunks.
constexpr int kRouteCountWaves = 8;
constexpr int kRouteCountStep = kRouteCountWaves * 4;  // tokens a router workgroup routes per step
constexpr int kRouteCountMaxExperts = 512;
LayoutPlan plan_route_count(int64_t T, int k, int E);

// The layout's chunk table in a file-scope device array (ep_layout_noalloc):
// its size, and its address on the current device (resolved once per device).
constexpr size_t kLayoutScratchBytes = 288 * 1024;
constexpr int kMaxDevices = 64;
hipError_t layout_scratch(void **ptr);

// Launchers (no validation; the C ABI validates first).  Return hipError_t of
// the launch.
hipError_t launch_layout(const ep_config &c, const LayoutPlan &plan, const int32_t *topk_idx,
                         const ep_layout_t &h, void *workspace, hipStream_t s);

// The scatter kernel alone, for a table the router counted (plan_route_count).
hipError_t launch_layout_scatter(const ep_config &c, const LayoutPlan &plan,
                                 const int32_t *topk_idx, const ep_layout_t &h, void *workspace,
                                 hipStream_t s);

hipError_t launch_dispatch(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                           const void *x, const RankPtrs &rx, const ScalePtrs &rs,
                           int64_t capacity_rows, hipStream_t s);

// The gradient rows of combine's backward, bf16(RN32(w[p] * grad_out[t])) into
// each pair's row (w NULL: weights 1): the BF16 dispatch with one multiply
// per copy (ep_dispatch.hip).
hipError_t launch_combine_backward_rows(const ep_config &c, const ep_layout_t &h,
                                        const int32_t *topk_idx, const void *grad_out,
                                        const float *w, const RankPtrs &rg,
                                        int64_t capacity_rows, hipStream_t s);

hipError_t launch_combine(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                          const RankCPtrs &ry, const float *w, const void *shared, void *out,
                          int64_t capacity_rows, hipStream_t s);

hipError_t launch_combine_backward(const ep_config &c, const ep_layout_t &h,
                                   const int32_t *topk_idx, const void *grad_out, const float *w,
                                   const RankCPtrs &ry, const RankPtrs &rg, float *grad_w,
                                   int64_t capacity_rows, hipStream_t s);

hipError_t launch_silu_mul_quant(const ep_config &c, const ep_layout_t &h, int32_t I,
                                 const RankCPtrs &in, const RankPtrs &q, const ScalePtrs &s,
                                 int64_t capacity_rows, hipStream_t st);

bool fused_layout_dispatch_ok(const ep_config &c);
hipError_t launch_layout_dispatch_small(const ep_config &c, const int32_t *topk_idx,
                                        const ep_layout_t &h, const void *x, const RankPtrs &rx,
                                        const ScalePtrs &rs, int64_t capacity_rows, hipStream_t s);

hipError_t launch_route(const ep_config &c, const ep_router_t &rt, const float *logits,
                        const float *bias, const int32_t *rep_off, const int32_t *rep_slots,
                        int32_t *topk_idx, float *topk_w, hipStream_t s);

// ep_route_layout: the counting router + scatter where plan_route_count and
// the four-tokens-per-wave router apply (and num_workgroups is 0), else
// launch_route then launch_layout.
hipError_t launch_route_layout(const ep_config &c, const ep_router_t &rt, const float *logits,
                               const float *bias, const int32_t *rep_off,
                               const int32_t *rep_slots, int32_t *topk_idx, float *topk_w,
                               const ep_layout_t &h, void *workspace, hipStream_t s);

hipError_t launch_unpermute(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                            const RankCPtrs &ry, void *out, int64_t capacity_rows, hipStream_t s);

// Resident-workgroup cap of the large streaming launches (dispatch, combine,
// the backward's gradient rows): dynamic LDS that the kernel never touches,
// sized so a CU holds at most wg_per_cu of these single-wave workgroups
// (gfx950: 160 KiB of LDS per CU; rounded down to whole KiB, so an allocation
// granule of up to 1 KiB keeps the count exact).  Launches of fewer than
// kResidentCapMinUnits work units (about two rounds of the waves the GPU
// holds) are not capped: there a partly filled extra round can cost more
// than the cap gains.  Only timing depends on it.
constexpr int64_t kResidentCapMinUnits = 16384;
constexpr int kLdsPerCu = 160 * 1024;
inline size_t resident_cap_lds(int64_t units, int wg_per_cu) {
  if (units < kResidentCapMinUnits) return 0;
  return (size_t)(kLdsPerCu / wg_per_cu) / 1024 * 1024;
}

// Grid size of the per-row kernels: num_workgroups, else one single-wave
// workgroup per work unit (the kernels grid-stride over the rest, if any).
inline int row_grid(const ep_config &c, int64_t units) {
  if (c.num_workgroups > 0) return c.num_workgroups;
  int64_t g = (units + kRowWaves - 1) / kRowWaves;
  if (g > 0x7FFFFFFF) g = 0x7FFFFFFF;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace ep
