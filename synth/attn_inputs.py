"""Seeded synthetic inputs for GQA decode attention over a block-paged KV cache.

Recipe (one independent stream per tensor):
    rng = default_rng(SeedSequence([seed, 100 + kind]))
  * q      ~ N(0, 1) rounded to bf16, [B, Hq, D]
  * keys   ~ N(0, 1) rounded to bf16, values ~ N(0, 1) rounded to bf16
  * the cache holds n_phys blocks of block_size tokens: k_cache / v_cache [n_phys, Hkv, BS, D]
    bf16; sequence b owns ceil(seq_len[b] / BS) blocks, placed at physical blocks drawn by a
    random permutation (so a sequence's blocks are scattered), listed in block_table [B, MB]
    (entries past a sequence's blocks are -1); cache slots past a sequence's length hold
    finite values that a correct kernel never reads into its result
No arithmetic of the attention itself lives here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe_inputs import f32_to_bf16_bits

_K_Q, _K_K, _K_V, _K_PERM = 0, 1, 2, 3


@dataclass(frozen=True)
class AttnShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int


# the model's full-attention layers: 16 query heads, 2 KV heads; head size hidden / 16
ATTN_SHAPES = {
    "tiny": AttnShape(4, 2, 64, 16),
    "mid": AttnShape(8, 1, 128, 32),
    "wide": AttnShape(16, 2, 256, 64),
    "full": AttnShape(16, 2, 128, 64),
}


def _rng(seed, kind):
    return np.random.default_rng(np.random.SeedSequence([seed, 100 + kind]))


def make_attn_inputs(shape: AttnShape, seq_lens, seed: int = 0, spare_blocks: int = 3):
    """q [B,Hq,D], k_cache / v_cache [n_phys,Hkv,BS,D] (bf16 bits), block_table [B,MB] int32,
    seq_lens [B] int32."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.size
    BS, Hq, Hkv, D = shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    nblk = (seq_lens + BS - 1) // BS
    MB = max(1, int(nblk.max()) if B else 1)
    n_phys = int(nblk.sum()) + spare_blocks
    q = f32_to_bf16_bits(_rng(seed, _K_Q).standard_normal((B, Hq, D)).astype(np.float32))
    kc = f32_to_bf16_bits(_rng(seed, _K_K).standard_normal((n_phys, Hkv, BS, D)).astype(np.float32))
    vc = f32_to_bf16_bits(_rng(seed, _K_V).standard_normal((n_phys, Hkv, BS, D)).astype(np.float32))
    perm = _rng(seed, _K_PERM).permutation(n_phys).astype(np.int32)
    table = np.full((B, MB), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    return q, kc, vc, table, seq_lens
