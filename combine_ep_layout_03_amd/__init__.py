"""MI355X (gfx950) MoE token dispatch / combine: router, routing layout, dispatch
(BF16 or FP8 E4M3 with per-128-channel scales), un-permute and top-k weighted
BF16 combine, as hand-written HIP kernels behind the C ABI of include/ep.h.

This package is the binding: `libep.so` (built from csrc/) does all the work.
"""
from ._lib import (Config, EpError, EXPORTS, EP_DEVERR_INDEX, EP_DEVERR_ROW, EP_DTYPE_BF16,
                   EP_DTYPE_FP8_E4M3, EP_ERR_CAPACITY, EP_ERR_HIP, EP_ERR_INVALID_ARG,
                   EP_ERR_UNSUPPORTED, EP_OK, ep_abi_version, ep_combine, ep_combine_backward,
                   ep_combine_shared, ep_dispatch, ep_layout, ep_layout_dispatch, ep_layout_noalloc,
                   ep_silu_mul_quant, ep_layout_workspace_bytes, ep_recv_capacity_rows, ep_status_string,
                   ep_unpermute, ep_route, ep_route_layout, Router, EP_GATE_SOFTMAX,
                   EP_GATE_SIGMOID, load)

__all__ = ["Config", "EpError", "EXPORTS", "ep_abi_version", "ep_combine", "ep_combine_shared",
           "ep_combine_backward", "ep_dispatch", "ep_layout_dispatch", "ep_silu_mul_quant",
           "ep_layout", "ep_layout_noalloc", "ep_layout_workspace_bytes", "ep_recv_capacity_rows",
           "ep_status_string",
           "ep_unpermute", "ep_route", "ep_route_layout", "Router", "EP_GATE_SOFTMAX",
           "EP_GATE_SIGMOID", "load", "EP_OK", "EP_ERR_INVALID_ARG", "EP_ERR_UNSUPPORTED",
           "EP_ERR_CAPACITY", "EP_ERR_HIP", "EP_DEVERR_INDEX", "EP_DEVERR_ROW", "EP_DTYPE_BF16",
           "EP_DTYPE_FP8_E4M3"]
