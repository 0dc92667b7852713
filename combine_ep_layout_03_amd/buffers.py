"""Device buffers for the C ABI, allocated with torch (device memory and
streams are torch's job; the library itself allocates nothing).

`Handle` holds the routing handle's arrays, `RecvBuffers` the R per-rank
receive buffers (capacity rows each) and `alloc_workspace` the layout
workspace, all sized from the config with the library's own size calls.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class Handle:
    expert_counts: torch.Tensor   # [E]
    expert_offsets: torch.Tensor  # [E+1]
    rank_counts: torch.Tensor     # [R]
    rank_offsets: torch.Tensor    # [R+1]
    slot_of: torch.Tensor         # [T*k]
    src_of: torch.Tensor          # [T*k]
    error_flag: torch.Tensor      # [1]

    @staticmethod
    def alloc(cfg: _lib.Config, device="cuda") -> "Handle":
        E, R, P = cfg.num_experts, cfg.num_ranks, cfg.num_tokens * cfg.num_topk
        z = lambda n: torch.zeros(n, dtype=torch.int32, device=device)
        return Handle(z(E), z(E + 1), z(R), z(R + 1), z(P), z(P), z(1))


def alloc_workspace(cfg: _lib.Config, device="cuda") -> torch.Tensor:
    n = _lib.ep_layout_workspace_bytes(cfg)
    if n <= 0:
        raise ValueError("invalid config for ep_layout")
    return torch.empty(n, dtype=torch.uint8, device=device)


@dataclass
class RecvBuffers:
    """R receive buffers of `capacity` rows: `x` holds bf16 rows (int16 view)
    or E4M3 bytes (uint8); `scales` holds [capacity, H/128] fp32 for FP8."""
    x: list
    scales: list | None
    capacity: int

    @staticmethod
    def alloc(cfg: _lib.Config, capacity: int | None = None, fp8: bool | None = None,
              device="cuda", fill: int | None = None) -> "RecvBuffers":
        cap = _lib.ep_recv_capacity_rows(cfg) if capacity is None else capacity
        fp8 = cfg.fp8 if fp8 is None else fp8
        H, R = cfg.hidden, cfg.num_ranks
        if fp8:
            xs = [torch.empty((cap, H), dtype=torch.uint8, device=device) for _ in range(R)]
            ss = [torch.empty((cap, H // 128), dtype=torch.float32, device=device) for _ in range(R)]
        else:
            xs = [torch.empty((cap, H), dtype=torch.int16, device=device) for _ in range(R)]
            ss = None
        if fill is not None:
            for t in xs:
                t.view(torch.uint8).fill_(fill)
            for t in ss or []:
                t.view(torch.uint8).fill_(fill)
        return RecvBuffers(xs, ss, cap)
