"""Seeded synthetic inputs for the MoE dispatch / combine path.

This package holds input generation only (tokens, gates, routing, expert
outputs); it contains none of the layout, dispatch, quantization or combine
arithmetic, and both the HIP path's tests and the CPU oracle read the arrays it
produces.
"""
from .gen import CONFIGS, Workload, make_workload, make_expert_rows, edge_case_x, bf16_from_f32

__all__ = ["CONFIGS", "Workload", "make_workload", "make_expert_rows", "edge_case_x", "bf16_from_f32"]
