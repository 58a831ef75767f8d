"""Plain fp64 CPU oracle for the MoE layer's hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. It shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing); it only consumes the same seeded inputs.

Sources (cited by page title and section):
  [P1] "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for
       Apple Silicon": sections "The Model: Qwen3.6-35B-A3B in Focus" and
       "How It Works: Prefill and Decode Strategies".
  [P3] "Perplexity Open Sources Apple Chip Inference Engine Lily": the paragraph on the
       target weights (MLX affine 4-bit, group size 64) and the one on the model structure.

What the layer computes, written out plainly (every weight matrix W = dequant(q, s, b)):
  1. router logits  l[t, e] = x[t] . Wr[e] + b_r[e]
  2. S_t            = the top_k experts with the largest l[t, e]; ties go to the lower index
  3. p[t, e]        = exp(l[t, e]) / sum_{j in S_t} exp(l[t, j])      for e in S_t
  4. FFN(x; Wg, Wu, Wd) = Wd . ( silu(Wg . x) * (Wu . x) ),  silu(z) = z / (1 + exp(-z))
  5. y[t]           = sum_{e in S_t} p[t, e] FFN_e(x[t]) + sigmoid(x[t] . wg) FFN_shared(x[t])

Readings where the pages are silent (each also listed with its reason in the design notes):
  * softmax over all experts then renormalising over the selected ones equals the softmax
    over the selected logits (step 3); the router bias, when present, is added before
    selection; the shared expert's gate is sigmoid(x . wg) with no bias; SwiGLU is
    silu(gate) * up; the output is fp32.
  * nibble order: element 8i+j of a row sits at bits [4j, 4j+4) of little-endian word i.

Rounding profiles:
  * "exact": no intermediate rounding at all (the mathematical definition).
  * "bf16": rounds (nearest, ties to even) at exactly two places, the inputs of the two
    tensor operations of an expert: the reconstructed weights ([P1 "The Model ..."]: the
    4-bit weights are rebuilt into bf16 for the tensor operations, with fp32 accumulation)
    and the SwiGLU output A that the down projection multiplies. The section says nothing of
    the expert outputs, and the weighted combine is a scalar-weighted sum, not a tensor
    operation, so the expert outputs, the combine and everything else stay fp64.

Every function here is pinned by tests/test_oracle*.py against closed forms, brute force
or invariants; no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

GROUP = 64
PROFILES = ("exact", "bf16")


# ----------------------------------------------------------------------------- numbers
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact values in fp64 (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    bf16 carries 8 significant bits. With v = m * 2**e and 0.5 <= |m| < 1 (frexp), the
    nearest bf16 is rint(m * 2**8) * 2**(e - 8); numpy's rint rounds halves to even. The
    product m * 2**8 and the rescaling are exact in fp64. Values below the smallest normal
    bf16 (2**-126) use the fixed subnormal spacing 2**-133. Overflow is not modelled
    (layer values stay far below 2**127).
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e, -125)           # e - 8 >= -133: subnormal bf16 spacing
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


# ----------------------------------------------------------------------- weight format
def unpack_nibbles(words) -> np.ndarray:
    """[..., n/8] uint32 words -> [..., n] uint8 nibbles.

    Element 8i+j of a row is bits [4j, 4j+4) of word i ([P3], target weights paragraph:
    MLX affine 4-bit; the in-word order is the little-endian reading)."""
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty(w.shape[:-1] + (w.shape[-1] * 8,), dtype=np.uint8)
    for j in range(8):
        out[..., j::8] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out


def dequant(q, scale, bias, profile: str = "exact") -> np.ndarray:
    """One projection matrix [N, Kin] in fp64: w = s_g * q + b_g for the group g = i // 64.

    [P1 "The Model ..."]: each group of 64 weights has its own scale and bias.
    In the "bf16" profile the reconstructed weight is rounded to bf16 ([P1 "The Model ..."]:
    tensor operations take bf16 inputs)."""
    qv = unpack_nibbles(q).astype(np.float64)
    s = np.repeat(bf16_to_f64(scale), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(bias), GROUP, axis=-1)
    w = s * qv + b
    return round_to_bf16(w) if profile == "bf16" else w


# ----------------------------------------------------------------------------- routing
def router_logits(x_bits, router_w, router_bias=None) -> np.ndarray:
    """l[t, e] = x[t] . Wr[e] + b[e] in fp64 ([P1 "The Model ..."]: a router scores the experts)."""
    x = bf16_to_f64(x_bits)
    l = x @ np.asarray(router_w, dtype=np.float64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, dtype=np.float64)[None, :]
    return l


def select_topk(logits, k: int):
    """Top-k experts per token, in rank order (largest logit first, ties to the lower index),
    and their renormalised weights softmax(l[S_t]) ([P1 "The Model ..."]: 256 scored, 8 chosen).

    A stable argsort of -l keeps equal logits in ascending expert order."""
    l = np.asarray(logits, dtype=np.float64)
    idx = np.argsort(-l, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(l, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), p


def shared_gate(x_bits, wg) -> np.ndarray:
    """sigmoid(x[t] . wg): the scalar that scales the shared expert's output per token."""
    g = bf16_to_f64(x_bits) @ np.asarray(wg, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-g))


def near_ties(logits, k: int, gap: float = 1e-4) -> np.ndarray:
    """Tokens whose ranked logits 1..k+1 contain an adjacent gap below `gap` (these may be
    ordered differently by a correct fp32 implementation; they are reported, not failed)."""
    l = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)[:, : k + 1]
    return np.nonzero((np.diff(-l, axis=1) < gap).any(axis=1))[0]


# ----------------------------------------------------------------------- permutation
def permute(topk_idx, num_experts: int):
    """Group the T*K (token, rank) slots by expert, stable in slot order s = t*K + k
    ([P1 "How It Works ..."]: histogram, prefix scan, scatter on the GPU).

    Returns counts [E], offsets [E+1] (exclusive scan), sorted_slots [T*K] (slots in
    expert-major, slot-ascending order) and slot_pos [T*K] (its inverse)."""
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_slots = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slots)
    slot_pos[sorted_slots] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_slots, slot_pos


# ------------------------------------------------------------------------------- FFN
def silu(z) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x, wg, wu, wd, profile: str = "exact") -> np.ndarray:
    """FFN(x) = Wd . (silu(Wg . x) * (Wu . x)) for rows x [n, H] (fp64 values).

    In the "bf16" profile the SwiGLU output, the input of the down projection's tensor
    operation, is rounded to bf16; the expert's output is not rounded."""
    a = silu(x @ wg.T) * (x @ wu.T)
    if profile == "bf16":
        a = round_to_bf16(a)
    return a @ wd.T


def _mat(proj, e, profile):
    q, s, b = proj
    return dequant(q[e], s[e], b[e], profile)


def layer_forward(layer: dict, x_bits, top_k: int, profile: str = "exact",
                  topk_idx=None, tokens=None) -> np.ndarray:
    """The whole layer for the selected `tokens` (default: all), as fp64 [n, H].

    `topk_idx` may force the routing (used when a token has a near-tie, to check the rest of
    the layer against the routing a correct fp32 implementation chose). Experts are
    dequantised one at a time, only when some selected token routes to them."""
    assert profile in PROFILES
    x_all = np.asarray(x_bits)
    rows = np.arange(x_all.shape[0]) if tokens is None else np.asarray(tokens)
    xb = x_all[rows]
    x = bf16_to_f64(xb)
    logits = router_logits(xb, layer["router_w"], layer["router_bias"])
    idx, p = select_topk(logits, top_k)
    if topk_idx is not None:
        idx = np.asarray(topk_idx)[rows].astype(np.int32)
        sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
    out = np.zeros((rows.size, x.shape[1]), dtype=np.float64)
    for e in np.unique(idx):
        t_sel, k_sel = np.nonzero(idx == e)
        y = expert_ffn(x[t_sel], _mat(layer["gate"], e, profile), _mat(layer["up"], e, profile),
                       _mat(layer["down"], e, profile), profile)
        np.add.at(out, t_sel, p[t_sel, k_sel][:, None] * y)
    if layer.get("sh_gate") is not None:
        sg = shared_gate(xb, layer["shared_gate_w"])
        y = expert_ffn(x, _mat(layer["sh_gate"], 0, profile), _mat(layer["sh_up"], 0, profile),
                       _mat(layer["sh_down"], 0, profile), profile)
        out += sg[:, None] * y
    return out


def layer_forward_per_token(layer: dict, x_bits, top_k: int, profile: str = "exact") -> np.ndarray:
    """Step 5 token by token with an explicit loop over the token's chosen experts; used on
    small layers to check the grouped evaluation in layer_forward."""
    x_all = bf16_to_f64(x_bits)
    out = np.zeros_like(x_all)
    for t in range(x_all.shape[0]):
        l = router_logits(np.asarray(x_bits)[t:t + 1], layer["router_w"], layer["router_bias"])[0]
        order = sorted(range(l.size), key=lambda e: (-l[e], e))[:top_k]
        den = sum(np.exp(l[j] - l[order[0]]) for j in order)
        for e in order:
            pe = np.exp(l[e] - l[order[0]]) / den
            out[t] += pe * expert_ffn(x_all[t:t + 1], _mat(layer["gate"], e, profile),
                                      _mat(layer["up"], e, profile),
                                      _mat(layer["down"], e, profile), profile)[0]
        if layer.get("sh_gate") is not None:
            g = float(x_all[t] @ np.asarray(layer["shared_gate_w"], dtype=np.float64))
            out[t] += (1.0 / (1.0 + np.exp(-g))) * expert_ffn(
                x_all[t:t + 1], _mat(layer["sh_gate"], 0, profile), _mat(layer["sh_up"], 0, profile),
                _mat(layer["sh_down"], 0, profile), profile)[0]
    return out


# ------------------------------------------------------------------- stack of layers
# The pages give the model's depth ([P1 "The Model ..."]: 10 full-attention and 30 Gated
# DeltaNet layers, each with this MoE block) and keep the next step's input on the GPU
# ([P1 "How It Works ..."]). The stacked workload is read as a pre-norm residual stream:
#   r_0 = x,  x_l = bf16(RMSNorm(r_l)),  r_{l+1} = r_l + MoE_l(x_l)
# with RMSNorm(r) = r / sqrt(mean(r^2) + eps), unit weight, eps = 1e-6.
RMS_EPS = 1e-6


def rms_norm(r, eps: float = RMS_EPS) -> np.ndarray:
    """r / sqrt(mean(r^2) + eps) with unit weight, per row."""
    r = np.asarray(r, dtype=np.float64)
    return r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)


def bf16_bits(values) -> np.ndarray:
    """uint16 patterns of values that are exactly representable in bf16 (e.g. round_to_bf16
    output); bf16 is the upper half of the fp32 pattern."""
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    u = v.view(np.uint32)
    assert np.array_equal(v.astype(np.float64), np.asarray(values, dtype=np.float64)), "not bf16"
    assert not np.any(u & np.uint32(0xFFFF)), "not bf16"
    return (u >> np.uint32(16)).astype(np.uint16)


def residual_rmsnorm(resid, y, eps: float = RMS_EPS):
    """One step of the residual stream: r' = r + y (y may be None: r' = r), and the next
    layer's input x' = bf16(RMSNorm(r')) as bf16 bit patterns. Returns (r', x' bits)."""
    r = np.asarray(resid, dtype=np.float64)
    if y is not None:
        r = r + np.asarray(y, dtype=np.float64)
    return r, bf16_bits(round_to_bf16(rms_norm(r, eps)))


def stack_forward(layers, x_bits, top_k: int, profile: str = "bf16", eps: float = RMS_EPS):
    """The whole stack for tokens x (bf16 bits): returns the final residual stream r_L and
    x_L = bf16(RMSNorm(r_L)) (bits), following the recurrence above layer by layer."""
    r, x = residual_rmsnorm(bf16_to_f64(x_bits), None, eps)
    for layer in layers:
        y = layer_forward(layer, x, top_k, profile)
        r, x = residual_rmsnorm(r, y, eps)
    return r, x


# ---------------------------------------------------------------------- tolerances
def error_stats(y, ref) -> dict:
    """Row-normalised max relative error max_t max_h |y-r| / max_h |r_t| and mean abs error."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(y - ref)
    row_scale = np.maximum(np.abs(ref).max(axis=1), np.finfo(np.float64).tiny)
    return {"max_rel": float((d.max(axis=1) / row_scale).max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0}
