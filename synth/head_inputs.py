"""Seeded synthetic weights of the greedy decode step: an LM head and a token embedding, both in
the layer's 4-bit group-64 affine format (q [1, V, H/8] uint32, scale / bias [1, V, H/64] bf16
bits), drawn with the same recipe as the expert weights (uniform words, scale ~ U(0.005, 0.02)
rounded to bf16, bias = -8 * scale). Random numbers only: none of the step's arithmetic."""
from __future__ import annotations

import numpy as np

from .moe_inputs import GROUP, f32_to_bf16_bits

# the vocabulary of the default workload: the Qwen3 tokenizer's 151,936 entries (the pages name
# the model but not its vocabulary; any V works)
VOCAB = 151936

_K_HEAD, _K_EMBED = 10, 11


def _w4(seed, kind, V, H):
    rq = np.random.default_rng(np.random.SeedSequence([seed, 300 + kind, 0]))
    rs = np.random.default_rng(np.random.SeedSequence([seed, 300 + kind, 1]))
    q = rq.integers(0, 2 ** 32, size=(1, V, H // 8), dtype=np.uint32)
    s = rs.uniform(0.005, 0.02, size=(1, V, H // GROUP))
    s_bits = f32_to_bf16_bits(s.astype(np.float32))
    s_f32 = (s_bits.astype(np.uint32) << 16).view(np.float32)
    b_bits = f32_to_bf16_bits(-8.0 * s_f32)                  # exact: a power-of-two multiple
    return q, s_bits, b_bits


def make_head(V: int, H: int, seed: int = 0) -> dict:
    """{"head": (q, scale, bias), "embed": (q, scale, bias)} for a vocabulary of V tokens."""
    assert H % GROUP == 0 and V > 0
    return {"head": _w4(seed, _K_HEAD, V, H), "embed": _w4(seed, _K_EMBED, V, H)}
