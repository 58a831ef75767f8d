"""fp64 oracle of the greedy decode step (test infrastructure: only tests/, the smoke check and
the bench's CPU baseline use it; it shares no code with the HIP library).

"Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
Silicon", section "How It Works: Prefill and Decode Strategies": the selected token is written
straight into the next step's GPU-resident input slot; section "Frequently Asked Questions" and
"Perplexity Open Sources Apple Chip Inference Engine Lily": decoding is greedy only. The LM head
and the token embedding are taken in the model's 4-bit group-64 affine format, like every other
weight of the 4-bit model.

  logits[t, v] = x[t] . W_head[v]      (x bf16; W_head dequantised, rounded to bf16 in the "bf16"
                                        profile, as the expert weights are)
  token[t]     = argmax_v logits[t, v] (the lowest v among equal maxima)
  x_next[t]    = RNE_bf16(E[token[t]])  (the embedding row, dequantised)
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_to_f64, dequant, round_to_bf16

ROWS = 8192   # rows of the head dequantised at a time (memory only; no effect on values)


def lm_logits(x_bits, head, profile: str = "bf16") -> np.ndarray:
    """[T, V] fp64 logits of the tokens x [T, H] (bf16 bits) against the head (q, s, b)."""
    q, s, b = head
    x = bf16_to_f64(x_bits)
    V = q.shape[1]
    out = np.empty((x.shape[0], V))
    for r0 in range(0, V, ROWS):
        w = dequant(q[0, r0:r0 + ROWS], s[0, r0:r0 + ROWS], b[0, r0:r0 + ROWS], profile)
        out[:, r0:r0 + ROWS] = x @ w.T
    return out


def greedy(logits) -> np.ndarray:
    """argmax per row, the lowest index among equal maxima (int32 [T])."""
    return np.argmax(np.asarray(logits), axis=1).astype(np.int32)


def near_tie(logits, gap: float = 1e-4) -> np.ndarray:
    """Rows whose two largest logits are closer than `gap` (the argmax may then differ between
    two correct evaluations in different summation orders)."""
    lg = np.asarray(logits)
    if lg.shape[1] < 2:      # a single entry has no rival
        return np.zeros(0, dtype=np.int64)
    top2 = -np.sort(-lg, axis=1)[:, :2]
    return np.nonzero(top2[:, 0] - top2[:, 1] < gap)[0]


def embed(tokens, emb) -> np.ndarray:
    """Embedding rows of the tokens as bf16 bit patterns [T, H] (dequantised, rounded to nearest
    even: s*q + b is exact in fp64, so this is the nearest bf16 of the exact value)."""
    q, s, b = emb
    t = np.asarray(tokens, dtype=np.int64)
    rows = round_to_bf16(dequant(q[0, t], s[0, t], b[0, t], "exact"))
    u = rows.astype(np.float32).view(np.uint32)   # bf16 values: exact in fp32
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def greedy_step(x_bits, head, emb, profile: str = "bf16"):
    """(token [T] int32, x_next [T, H] bf16 bits, logits [T, V] fp64)."""
    lg = lm_logits(x_bits, head, profile)
    tok = greedy(lg)
    return tok, embed(tok, emb), lg
