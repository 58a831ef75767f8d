"""Seeded synthetic inputs for the MoE layer (shared by the oracle tests and the HIP path).

This module only draws random numbers and stores them in the layer's storage formats.
It holds none of the layer's arithmetic: no unpacking, no dequantisation, no routing.
"""
from .moe_inputs import (  # noqa: F401
    LayerShape, SHAPES, make_layer, make_tokens, f32_to_bf16_bits, skew_router_bias,
)
