"""Seeded synthetic inputs for the gated delta-rule recurrence.

Recipe (one independent stream per tensor):
    rng = default_rng(SeedSequence([seed, 200 + kind]))
  * q, k ~ N(0, 1) rounded to bf16, [B, T, Hk, Dk]; v ~ N(0, 1) rounded to bf16, [B, T, Hv, Dv]
  * g = log(alpha) with alpha ~ U(0.90, 0.999), fp32 [B, T, Hv]: a per-token decay close to 1
  * beta = 1 / (1 + exp(-z)) with z ~ N(0, 1), fp32 [B, T, Hv]: the write strength in (0, 1)
  * the initial state ~ N(0, 0.1^2) fp32 [B, Hv, Dv, Dk] (or zeros)
No arithmetic of the recurrence itself lives here (the sigmoid and the log only shape the
random draws into the ranges the inputs take).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe_inputs import f32_to_bf16_bits

_K_Q, _K_K, _K_V, _K_G, _K_B, _K_S = range(6)


@dataclass(frozen=True)
class DeltaShape:
    num_k_heads: int   # query/key heads
    num_v_heads: int   # value heads (a multiple of the key heads; groups share q and k)
    dk: int
    dv: int


# the model's linear-attention layers: hidden 2048 as 16 heads of 128 (the plainest reading of
# the pages, which give the layer type and its fixed-size state but no head geometry)
DELTA_SHAPES = {
    "tiny": DeltaShape(2, 4, 64, 16),
    "mid": DeltaShape(4, 4, 64, 64),
    "full": DeltaShape(16, 16, 128, 128),
    "gva": DeltaShape(8, 16, 128, 128),
    "wide": DeltaShape(2, 4, 256, 48),   # the widest supported key dimension, dv not a multiple of 32
}


def _rng(seed, kind):
    return np.random.default_rng(np.random.SeedSequence([seed, 200 + kind]))


def make_delta_inputs(shape: DeltaShape, B: int, T: int, seed: int = 0, zero_state=False):
    """q, k [B,T,Hk,Dk] and v [B,T,Hv,Dv] as bf16 bits; g, beta [B,T,Hv] fp32; state
    [B,Hv,Dv,Dk] fp32."""
    Hk, Hv, Dk, Dv = shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv
    q = f32_to_bf16_bits(_rng(seed, _K_Q).standard_normal((B, T, Hk, Dk)).astype(np.float32))
    k = f32_to_bf16_bits(_rng(seed, _K_K).standard_normal((B, T, Hk, Dk)).astype(np.float32))
    v = f32_to_bf16_bits(_rng(seed, _K_V).standard_normal((B, T, Hv, Dv)).astype(np.float32))
    g = np.log(_rng(seed, _K_G).uniform(0.90, 0.999, (B, T, Hv))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-_rng(seed, _K_B).standard_normal((B, T, Hv))))).astype(np.float32)
    if zero_state:
        s0 = np.zeros((B, Hv, Dv, Dk), np.float32)
    else:
        s0 = (0.1 * _rng(seed, _K_S).standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    return q, k, v, g, beta, s0
