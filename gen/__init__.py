"""Seeded synthetic inputs for the routed FP8 MoE expert step.

This package is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no arithmetic of the method itself (no routing, no
quantisation, no matmul): only a counter-based random generator and the table of
workload shapes.  See ``gen.rng`` and ``gen.workloads``.
"""
from .workloads import CONFIGS, Workload, make_small_inputs, expert_weight_f32  # noqa: F401
