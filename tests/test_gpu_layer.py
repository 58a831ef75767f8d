"""Whole-layer parity: moe_layer_forward (through the C ABI) against the fp64 oracle.

Gate: row-normalised max relative error <= 2e-2 and mean absolute error <= 2e-3 against the
oracle's bf16 profile (the weights and the SwiGLU output rounded to bf16, the inputs of the
method's tensor operations; expert outputs and the combine unrounded); the exact profile's
error is printed beside it. Routing near-ties (gap < 1e-4)
are reported, and such tokens are checked against the oracle run with the library's routing.
"""
import numpy as np
import pytest

from gpu_common import (DEV, TOL_MAX_REL, TOL_MEAN_ABS, device_layer, gpu_routing, host_layer,
                        log, oracle_reference, tokens)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

FORCE = 2
ATOMIC = 1

CASES = [
    # (shape, T, flags): decode path for T <= 16 unless FORCE; prefill otherwise
    ("tiny", 4, 0), ("tiny", 4, FORCE), ("tiny", 1, 0), ("tiny", 37, 0), ("tiny", 37, ATOMIC),
    ("tiny", 4, FORCE | ATOMIC),
    ("odd", 1, 0), ("odd", 16, 0), ("odd", 16, FORCE), ("odd", 130, 0),
    ("mid", 1, 0), ("mid", 13, 0), ("mid", 13, FORCE), ("mid", 17, 0), ("mid", 300, 0),
    ("mid", 300, ATOMIC), ("odd", 130, ATOMIC),
    ("full", 1, 0), ("full", 8, 0), ("full", 16, 0), ("full", 8, FORCE),
    ("wide", 1, 0), ("wide", 4, 0), ("wide", 40, 0),
    ("solo", 1, 0), ("solo", 5, 0), ("solo", 40, 0),
    ("many", 1, 0), ("many", 16, 0), ("many", 16, FORCE), ("many", 40, 0), ("many", 40, ATOMIC),
]


def run_layer(name, T, flags, seed=0, stream=0):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer(name, seed)
    xh, x = tokens(name, T, seed, stream)
    ws = M.alloc_workspace(layer, T, flags)
    out = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_layer_forward(layer, x, out, ws, flags)
    torch.cuda.synchronize()
    return layer, xh, x, out.cpu().numpy()


def check(name, T, flags, y, ref, ref_exact, ties, swapped, what=""):
    st = O.error_stats(y, ref)
    se = O.error_stats(y, ref_exact)
    log(f"[layer] {name} T={T} flags={flags}{what}: vs bf16 profile max_rel={st['max_rel']:.3e} "
        f"mean_abs={st['mean_abs']:.3e} | vs exact max_rel={se['max_rel']:.3e} "
        f"mean_abs={se['mean_abs']:.3e} | near-ties={len(ties)} rerouted={swapped}")
    assert np.all(np.isfinite(y))
    assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS, st


@pytest.mark.parametrize("name,T,flags", CASES)
def test_layer_matches_oracle(name, T, flags):
    log(f"[layer] start {name} T={T} flags={flags}")
    layer, xh, x, y = run_layer(name, T, flags)
    host = host_layer(name)
    gidx = gpu_routing(layer, x, T) if not (flags & FORCE) else None
    ref, ref_exact, ties, swapped = oracle_reference(name, host, xh, layer.K, gpu_idx=gidx)
    check(name, T, flags, y, ref, ref_exact, ties, swapped)


@pytest.mark.parametrize("name,flags,T", [("full", 0, 4096), ("full_skew", 0, 4096),
                                          ("full", ATOMIC, 4096), ("full", 0, 512),
                                          ("full_skew", 0, 512), ("full_skew", ATOMIC, 512)])
def test_prefill_full_size_sampled(name, flags, T):
    """T = 4096 at the full layer size (the timed prefill workload) and T = 512 (a prefill
    chunk: the small-batch GEMM kernels, with blocks of hundreds of rows under skewed routing);
    the oracle checks 40 sampled tokens one by one, including the first and the last."""
    log(f"[layer] start {name} T={T} flags={flags} (sampled)")
    layer, xh, x, y = run_layer(name, T, flags)
    host = host_layer(name)
    rng = np.random.default_rng(123)
    sel = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 38, replace=False)]))
    gidx = gpu_routing(layer, x, T)
    ref, ref_exact, ties, swapped = oracle_reference(name, host, xh, layer.K, tokens_sel=sel,
                                                     gpu_idx=gidx)
    check(name, T, flags, y[sel], ref, ref_exact, ties, swapped, " sampled")
    assert np.all(np.isfinite(y))


def test_decode_and_prefill_paths_agree():
    """Token independence: the same tokens through the decode kernels (T = 8) and the MFMA
    prefill kernels agree to within the accumulation-order noise."""
    _, _, _, y_dec = run_layer("full", 8, 0, stream=5)
    _, _, _, y_pre = run_layer("full", 8, FORCE, stream=5)
    st = O.error_stats(y_dec, y_pre)
    log(f"[layer] decode vs prefill: {st}")
    assert st["max_rel"] <= 2e-3 and st["mean_abs"] <= 1e-4


def test_deterministic_paths_repeat_bit_identically():
    for name, T, flags in (("mid", 300, 0), ("full", 1, 0), ("full", 8, 0), ("full", 512, 0)):
        _, _, _, a = run_layer(name, T, flags, stream=7)
        _, _, _, b = run_layer(name, T, flags, stream=7)
        assert np.array_equal(a, b), (name, T, flags)


def test_zero_tokens_is_a_noop():
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer("tiny")
    x = torch.zeros((0, layer.H), dtype=torch.int16, device=DEV)
    out = torch.full((1, layer.H), 3.0, device=DEV)
    ws = M.alloc_workspace(layer, 4)
    M.moe_layer_forward(layer, x, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_decode_workspace_reuse_across_shapes():
    """One workspace serves decode calls of different T back to back."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer("full")
    ws = M.alloc_workspace(layer, 16)
    host = host_layer("full")
    for T in (16, 1, 3, 8, 1):
        xh, x = tokens("full", T, stream=20 + T)
        out = torch.empty((T, layer.H), dtype=torch.float32, device=DEV)
        M.moe_layer_forward(layer, x, out, ws)
        torch.cuda.synchronize()
        gidx = gpu_routing(layer, x, T)
        ref, ref_exact, ties, swapped = oracle_reference("full", host, xh, layer.K, gpu_idx=gidx)
        check("full", T, 0, out.cpu().numpy(), ref, ref_exact, ties, swapped, " reused ws")


@pytest.mark.parametrize("name,T,flags", [("full", 1, 0), ("full", 8, 0), ("mid", 300, 0),
                                          ("mid", 300, ATOMIC)])
def test_graph_replays_match_eager(name, T, flags):
    """The layer captured into a HIP graph (as the benchmark runs it) replays correctly,
    several times, with eager work and synchronisations between the replays."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer(name)
    xh, x = tokens(name, T, stream=11)
    ws = M.alloc_workspace(layer, T, flags)
    out = torch.empty((T, layer.H), dtype=torch.float32, device=DEV)
    M.moe_layer_forward(layer, x, out, ws, flags)
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_layer_forward(layer, x, out, ws, flags)
    scratch = torch.empty((T, layer.H), dtype=torch.float32, device=DEV)
    for rep in range(3):
        out.fill_(float("nan"))
        M.moe_layer_forward(layer, x, scratch, ws, flags)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y = out.cpu().numpy()
        if flags & ATOMIC:   # the atomic combine: summation order not fixed
            assert O.error_stats(y, eager)["max_rel"] < 1e-5, rep
        else:
            assert np.array_equal(y, eager), rep
