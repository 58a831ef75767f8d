"""Plain fp64 CPU oracle for grouped-query decode attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. It shares no code with the HIP library; it only consumes the same
seeded inputs.

Source (cited by page title and section): "Perplexity's Lily: A Breakthrough Local Inference
Engine Tailored Exclusively for Apple Silicon", section "The Model: Qwen3.6-35B-A3B in Focus"
(ten full-attention layers use grouped-query attention with 16 query heads and two KV heads;
attention runs over a growing key-value cache) and section "How It Works: Prefill and Decode
Strategies" (coalesced key and value cache reads, GQA packing, a fixed-block cache layout for
long contexts).

What one decode step computes, written out plainly. For a sequence with keys K_g and values
V_g (rows 0..S-1) of KV head g and the new token's query q_h of query head h:
  g(h)   = h // (Hq / Hkv)                      (query heads share KV heads in equal groups)
  s_j    = scale * (q_h . K_g(h)[j])            for j < S
  p_j    = exp(s_j) / sum_i exp(s_i)
  out_h  = sum_j p_j V_g(h)[j]
The cache is stored in fixed blocks of BS tokens: token j of sequence b sits in row j % BS of
physical block block_table[b, j // BS].

Readings where the pages are silent (also listed in the design notes): the head size is not
given (the model's hidden size divided by the 16 query heads, 128, is the default workload);
the softmax scale is a parameter (1/sqrt(D) by default); the output is fp32; q, K and V are
bf16 values taken exactly; a sequence with no tokens has an empty sum and a zero output.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_to_f64


def gather_kv(cache, block_table_row, seq_len: int, block_size: int) -> np.ndarray:
    """Keys (or values) of one sequence as [Hkv, S, D] fp64, token by token from its blocks."""
    cache = np.asarray(cache)
    Hkv, D = cache.shape[1], cache.shape[3]
    out = np.empty((Hkv, seq_len, D))
    for j in range(seq_len):
        blk = int(block_table_row[j // block_size])
        out[:, j, :] = bf16_to_f64(cache[blk, :, j % block_size, :])
    return out


def attention(q, k, v, scale: float) -> np.ndarray:
    """Grouped-query attention of one token: q [Hq, D], k / v [Hkv, S, D] (fp64) -> [Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    Hq, Hkv = q.shape[0], k.shape[0]
    G = Hq // Hkv
    out = np.empty_like(q)
    if k.shape[1] == 0:          # no keys: the weighted sum is empty
        return np.zeros_like(q)
    for h in range(Hq):
        g = h // G
        s = scale * (k[g] @ q[h])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ v[g]
    return out


def decode_attention(q_bits, k_cache, v_cache, block_table, seq_lens, block_size: int,
                     scale: float) -> np.ndarray:
    """A decode step for B sequences: q [B, Hq, D] bf16 bits -> out [B, Hq, D] fp64."""
    q = bf16_to_f64(q_bits)
    out = np.empty_like(q)
    for b in range(q.shape[0]):
        S = int(seq_lens[b])
        k = gather_kv(k_cache, block_table[b], S, block_size)
        v = gather_kv(v_cache, block_table[b], S, block_size)
        out[b] = attention(q[b], k, v, scale)
    return out
