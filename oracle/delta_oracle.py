"""Plain fp64 CPU oracle for the gated delta-rule recurrence (the model's linear-attention
layers).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. It shares no code with the HIP library; it only consumes the same
seeded inputs.

Sources: "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for
Apple Silicon", section "The Model: Qwen3.6-35B-A3B in Focus" (thirty Gated DeltaNet layers
run a recurrence whose state has a fixed size, one of the model's three workload patterns).
The pages do not print the recurrence; it is the gated delta rule as published by Yang, Kautz
and Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule" (ICLR 2025), with
L2-normalised queries and keys. For each value head j (query/key head i = j // (Hv/Hk)) and
token t, with the state S a [Dv, Dk] matrix:
  kh_t = k_t / sqrt(|k_t|^2 + eps),  qh_t = scale * q_t / sqrt(|q_t|^2 + eps)
  alpha_t = exp(g_t)
  S_t  = alpha_t * S_{t-1} (I - beta_t kh_t kh_t^T) + beta_t v_t kh_t^T
  o_t  = S_t qh_t
Readings where the pages are silent (also listed in the design notes): the head geometry
(16 heads of 128 by default), eps = 1e-6, scale = 1/sqrt(Dk), q, k and v taken exactly from
their bf16 values, g and beta given per token and value head in fp32, the state and the output
in fp32 on the GPU (fp64 here).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_to_f64

EPS = 1e-6


def l2_normalise(x, eps: float = EPS) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def recurrence(q_bits, k_bits, v_bits, g, beta, state, scale=None, eps: float = EPS):
    """The recurrence for B sequences of T tokens: q, k [B,T,Hk,Dk] and v [B,T,Hv,Dv] (bf16
    bits), g, beta [B,T,Hv], state [B,Hv,Dv,Dk]. Returns (o [B,T,Hv,Dv], final state), fp64.
    The update is applied as written, with the [Dk, Dk] matrix (I - beta kh kh^T)."""
    q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    grp = Hv // Hk
    S = np.array(state, dtype=np.float64, copy=True)
    o = np.zeros((B, T, Hv, Dv))
    eye = np.eye(Dk)
    for b in range(B):
        for t in range(T):
            for j in range(Hv):
                i = j // grp
                kh = l2_normalise(k[b, t, i], eps)
                qh = scale * l2_normalise(q[b, t, i], eps)
                a = np.exp(np.float64(g[b, t, j]))
                bt = np.float64(beta[b, t, j])
                S[b, j] = a * S[b, j] @ (eye - bt * np.outer(kh, kh)) + bt * np.outer(v[b, t, j], kh)
                o[b, t, j] = S[b, j] @ qh
    return o, S
