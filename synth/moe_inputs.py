"""Seeded synthetic MoE-layer inputs.

Recipe (one independent stream per tensor, so any expert can be regenerated alone):
    rng = default_rng(SeedSequence([seed, layer, kind, expert, proj]))
  * x        ~ N(0, 1), rounded to bf16 (round-to-nearest-even)
  * router_w ~ N(0, 0.02^2) fp32, shape [E, H]
  * shared_gate_w ~ N(0, 0.02^2) fp32, shape [H]
  * packed weights: every uint32 word uniform on [0, 2^32); a uniform word is exactly
    eight independent nibbles q ~ U{0..15}, so no packing arithmetic is needed here
  * scale ~ U(0.005, 0.02) rounded to bf16, bias = -8 * scale (exact in bf16)
  * the skewed workload adds router_bias[e] = -1.2 * ln(e + 1) (a Zipf(1.2)-like load)

Storage formats (these are the layer's interface, not its arithmetic):
  * bf16 tensors are uint16 bit patterns
  * a projection with N output rows and Kin inputs is q [n_mat, N, Kin/8] uint32,
    scale / bias [n_mat, N, Kin/64] uint16 (one pair per group of 64 inputs)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64

# stream "kind" ids
_K_X, _K_ROUTER, _K_SGATE, _K_Q, _K_SCALE = 0, 1, 2, 3, 4
# projection ids
_P_GATE, _P_UP, _P_DOWN = 0, 1, 2
_SHARED = -1  # expert id used for the shared expert's streams


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    num_experts: int
    top_k: int
    ffn: int
    shared_ffn: int
    skewed: bool = False

    @property
    def H(self):
        return self.hidden

    @property
    def E(self):
        return self.num_experts

    @property
    def K(self):
        return self.top_k

    @property
    def F(self):
        return self.ffn

    @property
    def Fs(self):
        return self.shared_ffn


# Named workloads: the tiny CPU-checkable layer, a mid-size multi-tile layer, an odd-sized
# layer (input dimensions that end in half a K-chunk, a non-power-of-two expert count), a
# layer wider than 2048 (its decode calls take the general GEMV kernels), and the full-size
# Qwen3.6-35B-A3B MoE layer (uniform and skewed routing). "solo" has one expert per token and
# no shared expert (the smallest entry list of the decode kernels); "many" sits at the largest
# expert count and top-k the library accepts (1024 experts, top-32) with one-group down rows.
SHAPES = {
    "tiny": LayerShape(256, 16, 2, 128, 128),
    "mid": LayerShape(512, 32, 4, 256, 192),
    "odd": LayerShape(320, 7, 3, 192, 64),
    "wide": LayerShape(2560, 16, 2, 128, 128),
    "solo": LayerShape(256, 8, 1, 128, 0),
    "many": LayerShape(256, 1024, 32, 64, 64),
    "full": LayerShape(2048, 256, 8, 512, 512),
    "full_skew": LayerShape(2048, 256, 8, 512, 512, skewed=True),
}


def _rng(seed, layer, kind, expert=0, proj=0):
    # SeedSequence entropy must be non-negative
    return np.random.default_rng(np.random.SeedSequence([seed, layer, kind, expert + 1, proj]))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def skew_router_bias(E: int) -> np.ndarray:
    """Per-expert router bias -1.2*ln(rank), rank = e + 1: Zipf(1.2)-like expert loads."""
    return (-1.2 * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def _proj(seed, layer, expert, proj, n_out, k_in):
    q = _rng(seed, layer, _K_Q, expert, proj).integers(
        0, 2 ** 32, size=(n_out, k_in // 8), dtype=np.uint32)
    s = _rng(seed, layer, _K_SCALE, expert, proj).uniform(0.005, 0.02, size=(n_out, k_in // GROUP))
    s_bits = f32_to_bf16_bits(s.astype(np.float32))
    s_f32 = (s_bits.astype(np.uint32) << 16).view(np.float32)
    b_bits = f32_to_bf16_bits(-8.0 * s_f32)                  # exact: a power-of-two multiple
    return q, s_bits, b_bits


def make_layer(shape: LayerShape, seed: int = 0, layer: int = 0, reuse: dict | None = None) -> dict:
    """Host arrays for one layer. Keys: router_w, router_bias (or None), shared_gate_w,
    gate/up/down and sh_gate/sh_up/sh_down as (q, scale, bias) tuples.

    `reuse`, a dict an earlier call returned for the same shape, has its routed-expert arrays
    overwritten in place (the values are those of a fresh call); it spares the first-touch cost
    of a new 450 MB allocation when many layers pass through host memory one at a time."""
    H, E, F, Fs = shape.H, shape.E, shape.F, shape.Fs
    assert H % GROUP == 0 and F % GROUP == 0 and Fs % GROUP == 0
    out = {}
    out["router_w"] = _rng(seed, layer, _K_ROUTER).normal(0.0, 0.02, size=(E, H)).astype(np.float32)
    out["router_bias"] = skew_router_bias(E) if shape.skewed else None
    out["shared_gate_w"] = _rng(seed, layer, _K_SGATE).normal(0.0, 0.02, size=(H,)).astype(np.float32)

    for name, pid, n_out, k_in in (("gate", _P_GATE, F, H), ("up", _P_UP, F, H), ("down", _P_DOWN, H, F)):
        if reuse is not None:
            q, s, b = reuse[name]
            assert q.shape == (E, n_out, k_in // 8) and s.shape == (E, n_out, k_in // GROUP)
        else:
            q = np.empty((E, n_out, k_in // 8), np.uint32)
            s = np.empty((E, n_out, k_in // GROUP), np.uint16)
            b = np.empty_like(s)
        for e in range(E):
            q[e], s[e], b[e] = _proj(seed, layer, e, pid, n_out, k_in)
        out[name] = (q, s, b)
    if Fs > 0:
        for name, pid, n_out, k_in in (("sh_gate", _P_GATE, Fs, H), ("sh_up", _P_UP, Fs, H),
                                       ("sh_down", _P_DOWN, H, Fs)):
            q, s, b = _proj(seed, layer, _SHARED, pid, n_out, k_in)
            out[name] = (q[None], s[None], b[None])
    else:
        for name in ("sh_gate", "sh_up", "sh_down"):
            out[name] = None
    return out


def make_tokens(shape: LayerShape, T: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    """x [T, H] as bf16 bit patterns; `stream` selects an independent token pool."""
    x = _rng(seed, stream, _K_X, 0, 0).normal(0.0, 1.0, size=(T, shape.H)).astype(np.float32)
    return f32_to_bf16_bits(x)
