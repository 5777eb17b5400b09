"""Seeded synthetic inputs for the W4A16 MoE layer.

This package is shared by the CPU oracle, the tests and the benchmark. It draws
random numbers and arranges them into the layouts the layer consumes; it holds
none of the layer's arithmetic (no dequantisation, no GEMM, no activation, no
combine).  Float-to-bf16 conversion of the drawn values uses torch's own
conversion, a library routine.
"""

from .gen import (  # noqa: F401
    MoEWorkload,
    bf16_bits_from_f32,
    draw_activations,
    draw_weights,
    draw_routing,
    build_contiguous,
    draw_masked,
    make_workload,
)
from .configs import WORKLOADS, workload_by_name  # noqa: F401
