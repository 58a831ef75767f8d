"""Seeded synthetic inputs (shared by the oracle tests and the HIP path): the MoE layer, GQA
decode attention over a block-paged KV cache, the gated delta-rule recurrence, and the greedy
decode step's LM head and token embedding.

These modules only draw random numbers and store them in the storage formats of the
operations. They hold none of the operations' arithmetic.
"""
from .moe_inputs import (  # noqa: F401
    LayerShape, SHAPES, make_layer, make_tokens, f32_to_bf16_bits, skew_router_bias,
)
from .attn_inputs import AttnShape, ATTN_SHAPES, make_attn_inputs  # noqa: F401
from .delta_inputs import DeltaShape, DELTA_SHAPES, make_delta_inputs  # noqa: F401
from .head_inputs import VOCAB, make_head  # noqa: F401
