"""Seeded synthetic inputs for the routed MoE expert-FFN layer.

This package produces the host arrays that both the CPU oracle and the HIP
path consume: packed int4 expert weights with their scales and zero points,
bf16 activations, and top-k routing (expert IDs and combine weights). It
holds none of the layer's own arithmetic (no alignment, dequantisation,
SwiGLU or combine); the router that draws the routing is data generation.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    make_routing,
    make_weights,
    make_workload,
)
