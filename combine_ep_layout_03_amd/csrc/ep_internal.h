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
  int64_t P;
  int32_t S;  // pairs per chunk (multiple of 64)
  int32_t C;  // chunks
  int32_t workgroups;  // ceil(C / kLayoutWaves)
  size_t workspace_bytes;  // C * (E + 1) * 4: per-chunk histograms + bad-index column
};

constexpr int kWave = 64;
constexpr int kLayoutWaves = 4;  // wavefronts per layout workgroup
constexpr int kRowWaves = 4;     // wavefronts per dispatch / combine workgroup

LayoutPlan plan_layout(int64_t P, int E);

// Launchers (no validation; the C ABI validates first).  Return hipError_t of
// the launch.
hipError_t launch_layout(const ep_config &c, const LayoutPlan &plan, const int32_t *topk_idx,
                         const ep_layout_t &h, void *workspace, hipStream_t s);

hipError_t launch_dispatch(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                           const void *x, const RankPtrs &rx, const ScalePtrs &rs,
                           int64_t capacity_rows, hipStream_t s);

hipError_t launch_combine(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                          const RankCPtrs &ry, const float *w, void *out, int64_t capacity_rows,
                          hipStream_t s);

hipError_t launch_unpermute(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                            const RankCPtrs &ry, void *out, int64_t capacity_rows, hipStream_t s);

// Grid size for the per-token kernels: num_workgroups or ceil(T / waves).
inline int row_grid(const ep_config &c, int64_t units) {
  if (c.num_workgroups > 0) return c.num_workgroups;
  int64_t g = (units + kRowWaves - 1) / kRowWaves;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace ep
