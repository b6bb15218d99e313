"""Seeded synthetic inputs for the MoE layer forward.

This package holds workload shapes and random-number generation only. It
contains none of the layer's arithmetic (routing, dispatch, experts, combine):
both the CPU oracle's tests and the GPU path draw their inputs from here, and
neither side imports the other.
"""
from .workloads import WORKLOADS, workload, local_experts
from .inputs import make_inputs, zipf_router_bias

__all__ = ["WORKLOADS", "workload", "local_experts", "make_inputs", "zipf_router_bias"]
