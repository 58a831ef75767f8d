"""Shared helpers for the GPU parity tests (device layers, tokens, oracle comparisons)."""
import functools
import sys

import numpy as np

import synth
from oracle import moe_oracle as O

DEV = "cuda"
TOL_MAX_REL = 2e-2   # row-normalised max relative error against the oracle
TOL_MEAN_ABS = 2e-3  # mean absolute error against the oracle (bf16 rounding profile)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def host_layer(name: str, seed: int = 0, layer: int = 0):
    shape = synth.SHAPES[name]
    if name == "full_skew":  # same experts as "full" (same streams); only the router bias differs
        base = dict(host_layer("full", seed, layer))
        base["router_bias"] = synth.skew_router_bias(shape.E)
        return base
    return synth.make_layer(shape, seed, layer)


@functools.lru_cache(maxsize=None)
def device_layer(name: str, seed: int = 0, layer: int = 0):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    shape = synth.SHAPES[name]
    if name == "full_skew":
        base = device_layer("full", seed, layer)
        t = dict(base.tensors)
        t["router_bias"] = torch.from_numpy(synth.skew_router_bias(shape.E)).to(DEV)
        return M.make_layer(t, shape.H, shape.E, shape.K, shape.F, shape.Fs)
    return M.upload_layer(host_layer(name, seed, layer), shape.H, shape.E, shape.K, shape.F,
                          shape.Fs, device=DEV)


def tokens(name: str, T: int, seed: int = 0, stream: int = 0):
    import torch
    xh = synth.make_tokens(synth.SHAPES[name], T, seed, stream)
    return xh, torch.from_numpy(xh.view(np.int16)).to(DEV)


def u16(t) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def gpu_routing(layer, x, T):
    """top-k ids chosen by the library's router for these tokens (same kernels as the layer)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    K = layer.K
    idx = torch.empty(T * K, dtype=torch.int32, device=DEV)
    w = torch.empty(T * K, dtype=torch.float32, device=DEV)
    sg = torch.empty(max(T, 1), dtype=torch.float32, device=DEV)
    cnt = torch.empty(layer.E, dtype=torch.int32, device=DEV)
    ws = M.alloc_workspace(layer, T)
    M.moe_route(layer, x, idx, w, sg if layer.Fs > 0 else None, cnt, ws)
    return idx.cpu().numpy().reshape(T, K)


def oracle_reference(name, host, xh, K, tokens_sel=None, gpu_idx=None):
    """Oracle output (bf16 profile) for the selected tokens. Tokens whose top-k has a near-tie
    (gap < 1e-4) and where the library picked a different but tie-equivalent set are evaluated
    with the library's routing; the list of such tokens is returned for the report."""
    rows = np.arange(xh.shape[0]) if tokens_sel is None else np.asarray(tokens_sel)
    logits = O.router_logits(xh[rows], host["router_w"], host["router_bias"])
    ridx, _ = O.select_topk(logits, K)
    ties = set(O.near_ties(logits, K).tolist())
    forced = None
    swapped = []
    if gpu_idx is not None:
        g = np.asarray(gpu_idx)[rows]
        for i in range(rows.size):
            if not np.array_equal(g[i], ridx[i]):
                assert i in ties, f"token {rows[i]}: routing differs without a near-tie"
                swapped.append(int(rows[i]))
        if swapped:
            forced = np.zeros((xh.shape[0], K), np.int32)
            forced[rows] = np.where(np.isin(rows, swapped)[:, None], g, ridx)
    ref = O.layer_forward(host, xh, K, "bf16", topk_idx=forced, tokens=rows)
    ref_exact = O.layer_forward(host, xh, K, "exact", topk_idx=forced, tokens=rows)
    return ref, ref_exact, sorted(ties), swapped
