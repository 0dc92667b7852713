// ep_api.cpp -- the C ABI declared in include/ep.h: host-side validation,
// launch planning and status mapping.  Every check here is synchronous and
// enqueues nothing when it fails; the kernels are in the .hip files beside it
// (layout, dispatch, combine, the fused decode path, the expert activation and
// the router).
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ep_internal.h"

namespace {

// EP_DEBUG is read once, at the first call that asks (a getenv per call is a
// scan of the environment, a measurable share of a small call's host time).
bool debug_enabled() {
  static const bool on = [] {
    const char *v = std::getenv("EP_DEBUG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

bool config_ok(const ep_config *c) {
  if (!c) return false;
  if (c->num_tokens < 1 || c->num_topk < 1 || c->num_topk > EP_MAX_TOPK) return false;
  if (c->num_experts < 1 || c->num_experts > EP_MAX_EXPERTS) return false;
  if (c->num_ranks < 1 || c->num_ranks > EP_MAX_RANKS) return false;
  if (c->num_experts % c->num_ranks != 0) return false;
  if (c->hidden < 8 || c->hidden > EP_MAX_HIDDEN || c->hidden % 8 != 0) return false;
  if (c->dispatch_dtype != EP_DTYPE_BF16 && c->dispatch_dtype != EP_DTYPE_FP8_E4M3) return false;
  if (c->dispatch_dtype == EP_DTYPE_FP8_E4M3 && c->hidden % 128 != 0) return false;
  if (c->num_workgroups < 0) return false;
  if ((int64_t)c->num_tokens * c->num_topk > INT32_MAX) return false;
  return true;
}

bool handle_ok(const ep_layout_t *h) {
  return h && h->expert_counts && h->expert_offsets && h->rank_counts && h->rank_offsets &&
         h->slot_of && h->src_of && h->error_flag;
}

// 16-byte aligned: the row kernels move every row buffer (tokens, received
// rows, scales, outputs, gradients) with 16-byte vector loads and stores, and
// the layout reads its chunk table the same way.
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool workspace_ok(const void *ws) { return ws && aligned16(ws); }

ep_status from_hip(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// EP_DEBUG=1: one line per call on stderr.
void trace(const char *what, const ep_config *c) {
  if (!debug_enabled()) return;
  std::fprintf(stderr, "[ep] %s T=%d H=%d k=%d E=%d R=%d dtype=%d num_workgroups=%d\n", what,
               c->num_tokens, c->hidden, c->num_topk, c->num_experts, c->num_ranks,
               c->dispatch_dtype, c->num_workgroups);
}

// A non-NULL, 16-byte aligned row buffer.
bool row_buf_ok(const void *p) { return p && aligned16(p); }

// The R receive (and, for FP8, scale) buffers of a dispatch; false if one is
// NULL or not 16-byte aligned.
bool recv_ptrs(const ep_config *cfg, void *const *recv_x, float *const *recv_scales,
               ep::RankPtrs &rx, ep::ScalePtrs &rs) {
  const bool fp8 = cfg->dispatch_dtype == EP_DTYPE_FP8_E4M3;
  if (!recv_x || (fp8 && !recv_scales)) return false;
  for (int r = 0; r < cfg->num_ranks; ++r) {
    if (!row_buf_ok(recv_x[r]) || (fp8 && !row_buf_ok(recv_scales[r]))) return false;
    rx.p[r] = recv_x[r];
    rs.p[r] = fp8 ? recv_scales[r] : nullptr;
  }
  return true;
}

// R read-only row buffers; false if the array or one pointer is NULL or not
// 16-byte aligned.
bool const_ptrs(const ep_config *cfg, const void *const *bufs, ep::RankCPtrs &out) {
  if (!bufs) return false;
  for (int r = 0; r < cfg->num_ranks; ++r) {
    if (!row_buf_ok(bufs[r])) return false;
    out.p[r] = bufs[r];
  }
  return true;
}

// Shared checks of dispatch / combine / unpermute.
ep_status row_call_ok(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                      int64_t capacity_rows) {
  if (!config_ok(cfg) || !handle_ok(h) || !topk_idx) return EP_ERR_INVALID_ARG;
  if (capacity_rows < (int64_t)cfg->num_tokens * cfg->num_topk) return EP_ERR_CAPACITY;
  return EP_OK;
}

bool router_ok(const ep_config *c, const ep_router_t *r, bool replicas) {
  if (!r) return false;
  const int32_t El = r->num_logical;
  if (El < 1 || El > EP_MAX_EXPERTS) return false;
  if (r->gate != EP_GATE_SOFTMAX && r->gate != EP_GATE_SIGMOID) return false;
  if (r->num_groups < 1 || r->num_groups > EP_MAX_GROUPS || El % r->num_groups != 0) return false;
  if (r->topk_groups < 1 || r->topk_groups > r->num_groups) return false;
  if (r->group_topn != 1 && r->group_topn != 2) return false;
  if (c->num_topk > El) return false;
  if ((int64_t)c->num_topk > (int64_t)r->topk_groups * (El / r->num_groups)) return false;
  if (!replicas && c->num_experts != El) return false;
  return true;
}

ep_status route_call_ok(const ep_config *cfg, const ep_router_t *router, const float *logits,
                        const int32_t *rep_off, const int32_t *rep_slots, const int32_t *topk_idx,
                        const float *topk_w) {
  if (!config_ok(cfg) || !logits || !topk_idx || !topk_w) return EP_ERR_INVALID_ARG;
  if ((rep_off == nullptr) != (rep_slots == nullptr)) return EP_ERR_INVALID_ARG;
  if (!router_ok(cfg, router, rep_off != nullptr)) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

}  // namespace

extern "C" {

uint32_t ep_abi_version(void) { return EP_ABI_VERSION; }

const char *ep_status_string(ep_status status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_UNSUPPORTED: return "unsupported";
    case EP_ERR_CAPACITY: return "receive capacity below ep_recv_capacity_rows()";
    case EP_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int64_t ep_recv_capacity_rows(const ep_config *cfg) {
  if (!config_ok(cfg)) return -1;
  return (int64_t)cfg->num_tokens * cfg->num_topk;
}

size_t ep_layout_workspace_bytes(const ep_config *cfg) {
  if (!config_ok(cfg)) return 0;
  // the larger of ep_layout's chunk table and ep_route_layout's router-counted one
  const size_t a =
      ep::plan_layout((int64_t)cfg->num_tokens * cfg->num_topk, cfg->num_experts).workspace_bytes;
  const size_t b =
      ep::plan_route_count(cfg->num_tokens, cfg->num_topk, cfg->num_experts).workspace_bytes;
  return a > b ? a : b;
}

ep_status ep_layout(const ep_config *cfg, const int32_t *topk_idx, const ep_layout_t *h,
                    void *workspace, hipStream_t stream) {
  if (!config_ok(cfg) || !handle_ok(h) || !topk_idx || !workspace_ok(workspace))
    return EP_ERR_INVALID_ARG;
  const ep::LayoutPlan plan =
      ep::plan_layout((int64_t)cfg->num_tokens * cfg->num_topk, cfg->num_experts);
  if (debug_enabled())
    std::fprintf(stderr, "[ep] layout P=%lld chunks=%d x %d pairs, workgroups=%d\n",
                 (long long)plan.P, plan.C, plan.S, plan.workgroups);
  return from_hip(ep::launch_layout(*cfg, plan, topk_idx, *h, workspace, stream));
}

ep_status ep_layout_noalloc(const ep_config *cfg, const int32_t *topk_idx, const ep_layout_t *h,
                            hipStream_t stream) {
  if (!config_ok(cfg) || !handle_ok(h) || !topk_idx) return EP_ERR_INVALID_ARG;
  const ep::LayoutPlan plan =
      ep::plan_layout((int64_t)cfg->num_tokens * cfg->num_topk, cfg->num_experts);
  if (plan.workspace_bytes > ep::kLayoutScratchBytes) {
    if (debug_enabled())
      std::fprintf(stderr, "[ep] layout_noalloc: table of %zu bytes exceeds the %zu-byte array\n",
                   plan.workspace_bytes, ep::kLayoutScratchBytes);
    return EP_ERR_UNSUPPORTED;
  }
  void *scratch = nullptr;
  if (ep::layout_scratch(&scratch) != hipSuccess) return EP_ERR_HIP;
  trace("layout_noalloc", cfg);
  return from_hip(ep::launch_layout(*cfg, plan, topk_idx, *h, scratch, stream));
}

ep_status ep_dispatch(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                      const void *x, void *const *recv_x, float *const *recv_scales,
                      int64_t capacity_rows, hipStream_t stream) {
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  ep::RankPtrs rx{};
  ep::ScalePtrs rs{};
  if (!row_buf_ok(x) || !recv_ptrs(cfg, recv_x, recv_scales, rx, rs)) return EP_ERR_INVALID_ARG;
  trace("dispatch", cfg);
  return from_hip(ep::launch_dispatch(*cfg, *h, topk_idx, x, rx, rs, capacity_rows, stream));
}

ep_status ep_layout_dispatch(const ep_config *cfg, const int32_t *topk_idx, const ep_layout_t *h,
                             void *workspace, const void *x, void *const *recv_x,
                             float *const *recv_scales, int64_t capacity_rows,
                             hipStream_t stream) {
  if (!config_ok(cfg) || !handle_ok(h) || !topk_idx || !workspace_ok(workspace))
    return EP_ERR_INVALID_ARG;
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  ep::RankPtrs rx{};
  ep::ScalePtrs rs{};
  if (!row_buf_ok(x) || !recv_ptrs(cfg, recv_x, recv_scales, rx, rs)) return EP_ERR_INVALID_ARG;
  if (ep::fused_layout_dispatch_ok(*cfg)) {
    trace("layout_dispatch (one launch)", cfg);
    return from_hip(
        ep::launch_layout_dispatch_small(*cfg, topk_idx, *h, x, rx, rs, capacity_rows, stream));
  }
  const ep::LayoutPlan plan =
      ep::plan_layout((int64_t)cfg->num_tokens * cfg->num_topk, cfg->num_experts);
  hipError_t e = ep::launch_layout(*cfg, plan, topk_idx, *h, workspace, stream);
  if (e != hipSuccess) return EP_ERR_HIP;
  trace("layout_dispatch (layout, then dispatch)", cfg);
  return from_hip(ep::launch_dispatch(*cfg, *h, topk_idx, x, rx, rs, capacity_rows, stream));
}

ep_status ep_combine(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                     const void *const *recv_y, const float *topk_weights, void *out,
                     int64_t capacity_rows, hipStream_t stream) {
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  ep::RankCPtrs ry{};
  if (!row_buf_ok(out) || !const_ptrs(cfg, recv_y, ry)) return EP_ERR_INVALID_ARG;
  trace("combine", cfg);
  return from_hip(ep::launch_combine(*cfg, *h, topk_idx, ry, topk_weights, nullptr, out,
                                     capacity_rows, stream));
}

ep_status ep_combine_shared(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                            const void *const *recv_y, const float *topk_weights,
                            const void *shared, void *out, int64_t capacity_rows,
                            hipStream_t stream) {
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  ep::RankCPtrs ry{};
  if (!row_buf_ok(out) || !row_buf_ok(shared) || !const_ptrs(cfg, recv_y, ry))
    return EP_ERR_INVALID_ARG;
  trace("combine_shared", cfg);
  return from_hip(ep::launch_combine(*cfg, *h, topk_idx, ry, topk_weights, shared, out,
                                     capacity_rows, stream));
}

ep_status ep_combine_backward(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                              const void *grad_out, const float *topk_weights,
                              const void *const *recv_y, void *const *grad_recv,
                              float *grad_weights, int64_t capacity_rows, hipStream_t stream) {
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  if (!row_buf_ok(grad_out) || !grad_recv) return EP_ERR_INVALID_ARG;
  if ((recv_y == nullptr) != (grad_weights == nullptr)) return EP_ERR_INVALID_ARG;
  ep::RankCPtrs ry{};
  ep::RankPtrs rg{};
  if (recv_y && !const_ptrs(cfg, recv_y, ry)) return EP_ERR_INVALID_ARG;
  for (int r = 0; r < cfg->num_ranks; ++r) {
    if (!row_buf_ok(grad_recv[r])) return EP_ERR_INVALID_ARG;
    rg.p[r] = grad_recv[r];
  }
  trace("combine_backward", cfg);
  return from_hip(ep::launch_combine_backward(*cfg, *h, topk_idx, grad_out, topk_weights, ry, rg,
                                              grad_weights, capacity_rows, stream));
}

ep_status ep_silu_mul_quant(const ep_config *cfg, const ep_layout_t *h, int32_t intermediate,
                            const void *const *act_in, void *const *q_out,
                            float *const *scales_out, int64_t capacity_rows, hipStream_t stream) {
  if (!config_ok(cfg) || !handle_ok(h)) return EP_ERR_INVALID_ARG;
  if (intermediate < 128 || intermediate % 128 != 0 || intermediate > EP_MAX_HIDDEN)
    return EP_ERR_INVALID_ARG;
  if (capacity_rows < (int64_t)cfg->num_tokens * cfg->num_topk) return EP_ERR_CAPACITY;
  if (!act_in || !q_out || !scales_out) return EP_ERR_INVALID_ARG;
  ep::RankCPtrs in{};
  ep::RankPtrs q{};
  ep::ScalePtrs s{};
  for (int r = 0; r < cfg->num_ranks; ++r) {
    if (!row_buf_ok(act_in[r]) || !row_buf_ok(q_out[r]) || !row_buf_ok(scales_out[r]))
      return EP_ERR_INVALID_ARG;
    in.p[r] = act_in[r];
    q.p[r] = q_out[r];
    s.p[r] = scales_out[r];
  }
  trace("silu_mul_quant", cfg);
  return from_hip(ep::launch_silu_mul_quant(*cfg, *h, intermediate, in, q, s, capacity_rows,
                                            stream));
}

ep_status ep_unpermute(const ep_config *cfg, const ep_layout_t *h, const int32_t *topk_idx,
                       const void *const *recv_y, void *out, int64_t capacity_rows,
                       hipStream_t stream) {
  ep_status st = row_call_ok(cfg, h, topk_idx, capacity_rows);
  if (st != EP_OK) return st;
  ep::RankCPtrs ry{};
  if (!row_buf_ok(out) || !const_ptrs(cfg, recv_y, ry)) return EP_ERR_INVALID_ARG;
  trace("unpermute", cfg);
  return from_hip(ep::launch_unpermute(*cfg, *h, topk_idx, ry, out, capacity_rows, stream));
}

ep_status ep_route(const ep_config *cfg, const ep_router_t *router, const float *logits,
                   const float *bias, const int32_t *replica_offsets,
                   const int32_t *replica_slots, int32_t *topk_idx, float *topk_weights,
                   hipStream_t stream) {
  const ep_status st = route_call_ok(cfg, router, logits, replica_offsets, replica_slots,
                                     topk_idx, topk_weights);
  if (st != EP_OK) return st;
  trace("route", cfg);
  return from_hip(ep::launch_route(*cfg, *router, logits, bias, replica_offsets, replica_slots,
                                   topk_idx, topk_weights, stream));
}

ep_status ep_route_layout(const ep_config *cfg, const ep_router_t *router, const float *logits,
                          const float *bias, const int32_t *replica_offsets,
                          const int32_t *replica_slots, int32_t *topk_idx, float *topk_weights,
                          const ep_layout_t *h, void *workspace, hipStream_t stream) {
  ep_status st = route_call_ok(cfg, router, logits, replica_offsets, replica_slots, topk_idx,
                               topk_weights);
  if (st != EP_OK) return st;
  if (!handle_ok(h) || !workspace_ok(workspace)) return EP_ERR_INVALID_ARG;
  trace("route_layout", cfg);
  return from_hip(ep::launch_route_layout(*cfg, *router, logits, bias, replica_offsets,
                                          replica_slots, topk_idx, topk_weights, *h, workspace,
                                          stream));
}

}  // extern "C"
