"""ctypes binding of libep.so (include/ep.h).  Argument marshalling only: every
step of layout, dispatch, un-permute and combine runs in the library's HIP
kernels.  Torch tensors supply device memory and the stream.

The functions carry the C names (EXPORTS lists them): the router, layout,
dispatch, combine and their fused, backward and expert-side variants, plus
the size helpers.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libep.so")

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_CAPACITY, EP_ERR_HIP = 0, 1, 2, 3, 4
EP_DEVERR_INDEX, EP_DEVERR_ROW, EP_DEVERR_INTERNAL = 1, 2, 4
EP_DTYPE_BF16, EP_DTYPE_FP8_E4M3 = 0, 1
EP_MAX_RANKS, EP_MAX_TOPK, EP_MAX_EXPERTS, EP_MAX_HIDDEN, EP_MAX_GROUPS = 64, 32, 2048, 65536, 64
EP_GATE_SOFTMAX, EP_GATE_SIGMOID = 0, 1

# Every symbol include/ep.h declares.
EXPORTS = ("ep_abi_version", "ep_status_string", "ep_recv_capacity_rows",
           "ep_layout_workspace_bytes", "ep_layout", "ep_layout_noalloc", "ep_dispatch",
           "ep_layout_dispatch",
           "ep_combine", "ep_combine_shared", "ep_combine_backward", "ep_silu_mul_quant",
           "ep_unpermute", "ep_route", "ep_route_layout")


class EpError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, ep_status_string(status), status))
        self.status = status


class ep_config(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32), ("dispatch_dtype", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int32)]


class ep_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("expert_counts", "expert_offsets", "rank_counts",
                                               "rank_offsets", "slot_of", "src_of", "error_flag")]


class ep_router_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_logical", "gate", "num_groups", "topk_groups",
                                              "group_topn", "renormalize")]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libep.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libep.so is not built (%s); run __graft_entry__.build() or "
                           "python combine_ep_layout_03_amd/build.py" % path)
    _lib = configure(ctypes.CDLL(path))
    return _lib


def configure(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures of include/ep.h on a loaded library."""
    vp, i64, cfgp, hp = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ep_config), ctypes.POINTER(ep_layout_t)
    L.ep_abi_version.restype = ctypes.c_uint32
    L.ep_abi_version.argtypes = []
    L.ep_status_string.restype = ctypes.c_char_p
    L.ep_status_string.argtypes = [ctypes.c_int32]
    L.ep_recv_capacity_rows.restype = i64
    L.ep_recv_capacity_rows.argtypes = [cfgp]
    L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_layout_workspace_bytes.argtypes = [cfgp]
    L.ep_layout.restype = ctypes.c_int32
    L.ep_layout.argtypes = [cfgp, vp, hp, vp, vp]
    L.ep_layout_noalloc.restype = ctypes.c_int32
    L.ep_layout_noalloc.argtypes = [cfgp, vp, hp, vp]
    L.ep_dispatch.restype = ctypes.c_int32
    L.ep_dispatch.argtypes = [cfgp, hp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, vp]
    L.ep_layout_dispatch.restype = ctypes.c_int32
    L.ep_layout_dispatch.argtypes = [cfgp, vp, hp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                     i64, vp]
    L.ep_combine.restype = ctypes.c_int32
    L.ep_combine.argtypes = [cfgp, hp, vp, ctypes.POINTER(vp), vp, vp, i64, vp]
    L.ep_combine_shared.restype = ctypes.c_int32
    L.ep_combine_shared.argtypes = [cfgp, hp, vp, ctypes.POINTER(vp), vp, vp, vp, i64, vp]
    L.ep_combine_backward.restype = ctypes.c_int32
    L.ep_combine_backward.argtypes = [cfgp, hp, vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      vp, i64, vp]
    L.ep_silu_mul_quant.restype = ctypes.c_int32
    L.ep_silu_mul_quant.argtypes = [cfgp, hp, ctypes.c_int32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(vp), i64, vp]
    rtp = ctypes.POINTER(ep_router_t)
    L.ep_route.restype = ctypes.c_int32
    L.ep_route.argtypes = [cfgp, rtp, vp, vp, vp, vp, vp, vp, vp]
    L.ep_route_layout.restype = ctypes.c_int32
    L.ep_route_layout.argtypes = [cfgp, rtp, vp, vp, vp, vp, vp, vp, hp, vp, vp]
    L.ep_unpermute.restype = ctypes.c_int32
    L.ep_unpermute.argtypes = [cfgp, hp, vp, ctypes.POINTER(vp), vp, i64, vp]
    return L


@dataclass
class Config:
    num_tokens: int
    hidden: int
    num_topk: int
    num_experts: int
    num_ranks: int
    fp8: bool = False
    num_workgroups: int = 0

    def c(self) -> ep_config:
        return ep_config(self.num_tokens, self.hidden, self.num_topk, self.num_experts,
                         self.num_ranks, EP_DTYPE_FP8_E4M3 if self.fp8 else EP_DTYPE_BF16,
                         self.num_workgroups)


@dataclass
class Router:
    num_logical: int
    gate: str = "sigmoid"          # "softmax" | "sigmoid"
    n_groups: int = 1
    topk_groups: int = 1
    group_topn: int = 2
    renorm: bool = True

    def c(self) -> ep_router_t:
        g = {"softmax": EP_GATE_SOFTMAX, "sigmoid": EP_GATE_SIGMOID}[self.gate]
        return ep_router_t(self.num_logical, g, self.n_groups, self.topk_groups, self.group_topn,
                           int(self.renorm))


def _router(rt) -> ep_router_t:
    return rt.c() if isinstance(rt, Router) else rt


def _cfg(cfg) -> ep_config:
    return cfg.c() if isinstance(cfg, Config) else cfg


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptrs(ts) -> ctypes.Array:
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def _need(t, nbytes: int, what: str) -> None:
    """A tensor argument must hold at least `nbytes` bytes (raw integer
    pointers are passed through unchecked).  The library checks NULL pointers,
    alignment and sizes it can see; it cannot see a buffer's length."""
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (what, have, nbytes))


def _need_rows(ts, rows: int, row_bytes: int, what: str) -> None:
    if ts is None:
        return
    for r, t in enumerate(ts):
        _need(t, rows * row_bytes, "%s[%d]" % (what, r))


def _row_bytes(c: "ep_config") -> int:
    """Bytes of one received row: H E4M3 codes under FP8, else H bf16."""
    return c.hidden if c.dispatch_dtype == EP_DTYPE_FP8_E4M3 else 2 * c.hidden


def _check(status: int, what: str) -> None:
    if status != EP_OK:
        raise EpError(status, what)


def ep_abi_version() -> int:
    return int(load().ep_abi_version())


def ep_status_string(status: int) -> str:
    return load().ep_status_string(int(status)).decode()


def ep_recv_capacity_rows(cfg) -> int:
    return int(load().ep_recv_capacity_rows(ctypes.byref(_cfg(cfg))))


def ep_layout_workspace_bytes(cfg) -> int:
    return int(load().ep_layout_workspace_bytes(ctypes.byref(_cfg(cfg))))


def _handle(h) -> ep_layout_t:
    if isinstance(h, ep_layout_t):
        return h
    return ep_layout_t(*[_ptr(getattr(h, n)) for n, _ in ep_layout_t._fields_])


def ep_layout(cfg, topk_idx, handle, workspace, stream=None) -> None:
    _check(load().ep_layout(ctypes.byref(_cfg(cfg)), _ptr(topk_idx), ctypes.byref(_handle(handle)),
                            _ptr(workspace), _stream(stream)), "ep_layout")


def _check_dispatch_buffers(c, x, recv_x, recv_scales, capacity_rows) -> None:
    _need(x, c.num_tokens * c.hidden * 2, "x")
    _need_rows(recv_x, capacity_rows, _row_bytes(c), "recv_x")
    if c.dispatch_dtype == EP_DTYPE_FP8_E4M3:
        _need_rows(recv_scales, capacity_rows, 4 * (c.hidden // 128), "recv_scales")


def _check_combine_buffers(c, recv_y, topk_weights, out, capacity_rows, out_rows=None) -> None:
    _need_rows(recv_y, capacity_rows, 2 * c.hidden, "recv_y")
    _need(topk_weights, c.num_tokens * c.num_topk * 4, "topk_weights")
    rows = c.num_tokens if out_rows is None else out_rows
    _need(out, rows * c.hidden * 2, "out")


def ep_layout_noalloc(cfg, topk_idx, handle, stream=None) -> None:
    _check(load().ep_layout_noalloc(ctypes.byref(_cfg(cfg)), _ptr(topk_idx),
                                    ctypes.byref(_handle(handle)), _stream(stream)),
           "ep_layout_noalloc")


def ep_dispatch(cfg, handle, topk_idx, x, recv_x, recv_scales, capacity_rows, stream=None) -> None:
    _check_dispatch_buffers(_cfg(cfg), x, recv_x, recv_scales, int(capacity_rows))
    rs = None if recv_scales is None else _ptrs(recv_scales)
    _check(load().ep_dispatch(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)), _ptr(topk_idx),
                              _ptr(x), _ptrs(recv_x), rs, int(capacity_rows), _stream(stream)),
           "ep_dispatch")


def ep_layout_dispatch(cfg, topk_idx, handle, workspace, x, recv_x, recv_scales, capacity_rows,
                       stream=None) -> None:
    _check_dispatch_buffers(_cfg(cfg), x, recv_x, recv_scales, int(capacity_rows))
    rs = None if recv_scales is None else _ptrs(recv_scales)
    _check(load().ep_layout_dispatch(ctypes.byref(_cfg(cfg)), _ptr(topk_idx),
                                     ctypes.byref(_handle(handle)), _ptr(workspace), _ptr(x),
                                     _ptrs(recv_x), rs, int(capacity_rows), _stream(stream)),
           "ep_layout_dispatch")


def ep_combine(cfg, handle, topk_idx, recv_y, topk_weights, out, capacity_rows, stream=None) -> None:
    _check_combine_buffers(_cfg(cfg), recv_y, topk_weights, out, int(capacity_rows))
    _check(load().ep_combine(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)), _ptr(topk_idx),
                             _ptrs(recv_y), _ptr(topk_weights), _ptr(out), int(capacity_rows),
                             _stream(stream)), "ep_combine")


def ep_combine_shared(cfg, handle, topk_idx, recv_y, topk_weights, shared, out, capacity_rows,
                      stream=None) -> None:
    c = _cfg(cfg)
    _check_combine_buffers(c, recv_y, topk_weights, out, int(capacity_rows))
    _need(shared, c.num_tokens * c.hidden * 2, "shared")
    _check(load().ep_combine_shared(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)),
                                    _ptr(topk_idx), _ptrs(recv_y), _ptr(topk_weights), _ptr(shared),
                                    _ptr(out), int(capacity_rows), _stream(stream)),
           "ep_combine_shared")


def ep_combine_backward(cfg, handle, topk_idx, grad_out, topk_weights, recv_y, grad_recv,
                        grad_weights, capacity_rows, stream=None) -> None:
    c = _cfg(cfg)
    cap = int(capacity_rows)
    _need(grad_out, c.num_tokens * c.hidden * 2, "grad_out")
    _need(topk_weights, c.num_tokens * c.num_topk * 4, "topk_weights")
    _need_rows(recv_y, cap, 2 * c.hidden, "recv_y")
    _need_rows(grad_recv, cap, 2 * c.hidden, "grad_recv")
    _need(grad_weights, c.num_tokens * c.num_topk * 4, "grad_weights")
    ry = None if recv_y is None else _ptrs(recv_y)
    _check(load().ep_combine_backward(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)),
                                      _ptr(topk_idx), _ptr(grad_out), _ptr(topk_weights), ry,
                                      _ptrs(grad_recv), _ptr(grad_weights), int(capacity_rows),
                                      _stream(stream)),
           "ep_combine_backward")


def ep_silu_mul_quant(cfg, handle, intermediate, act_in, q_out, scales_out, capacity_rows,
                      stream=None) -> None:
    cap, I = int(capacity_rows), int(intermediate)
    _need_rows(act_in, cap, 4 * I, "act_in")
    _need_rows(q_out, cap, I, "q_out")
    _need_rows(scales_out, cap, 4 * (I // 128), "scales_out")
    _check(load().ep_silu_mul_quant(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)),
                                    int(intermediate), _ptrs(act_in), _ptrs(q_out),
                                    _ptrs(scales_out), int(capacity_rows), _stream(stream)),
           "ep_silu_mul_quant")


def ep_unpermute(cfg, handle, topk_idx, recv_y, out, capacity_rows, stream=None) -> None:
    c = _cfg(cfg)
    _check_combine_buffers(c, recv_y, None, out, int(capacity_rows), out_rows=c.num_tokens * c.num_topk)
    _check(load().ep_unpermute(ctypes.byref(_cfg(cfg)), ctypes.byref(_handle(handle)), _ptr(topk_idx),
                               _ptrs(recv_y), _ptr(out), int(capacity_rows), _stream(stream)),
           "ep_unpermute")


def ep_route(cfg, router, logits, bias, replica_offsets, replica_slots, topk_idx, topk_weights,
             stream=None) -> None:
    _check(load().ep_route(ctypes.byref(_cfg(cfg)), ctypes.byref(_router(router)), _ptr(logits),
                           _ptr(bias), _ptr(replica_offsets), _ptr(replica_slots), _ptr(topk_idx),
                           _ptr(topk_weights), _stream(stream)), "ep_route")


def ep_route_layout(cfg, router, logits, bias, replica_offsets, replica_slots, topk_idx,
                    topk_weights, handle, workspace, stream=None) -> None:
    _check(load().ep_route_layout(ctypes.byref(_cfg(cfg)), ctypes.byref(_router(router)),
                                  _ptr(logits), _ptr(bias), _ptr(replica_offsets),
                                  _ptr(replica_slots), _ptr(topk_idx), _ptr(topk_weights),
                                  ctypes.byref(_handle(handle)), _ptr(workspace), _stream(stream)),
           "ep_route_layout")
