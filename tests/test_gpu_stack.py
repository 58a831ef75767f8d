"""The layer's launch sequence one phase at a time, the residual/RMSNorm step between layers,
and stacks of layers (moe_stack_forward) against the fp64 oracle.

Stacks are checked layer by layer with teacher forcing: the oracle evaluates each layer on the
input the GPU actually produced, so that a routing near-tie in one layer cannot make the
comparison of later layers meaningless; the stack call itself must reproduce the layer-by-layer
composition bit for bit."""
import numpy as np
import pytest

import synth
from gpu_common import (DEV, TOL_MAX_REL, TOL_MEAN_ABS, device_layer, gpu_routing, host_layer,
                        log, oracle_reference, tokens, u16)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

FORCE = 2
ATOMIC = 1


@pytest.mark.parametrize("name,T,flags", [("full", 1, 0), ("full", 8, 0), ("mid", 13, 0),
                                          ("mid", 300, 0), ("odd", 130, 0),
                                          ("odd", 16, FORCE), ("full", 16, 0), ("wide", 4, 0),
                                          ("many", 1, 0), ("many", 40, 0), ("mid", 300, ATOMIC)])
def test_phases_reproduce_forward(name, T, flags):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer(name)
    _, x = tokens(name, T, stream=31)
    n = M.moe_layer_num_phases(layer, T, flags)
    log(f"[phases] {name} T={T} flags={flags}: {n} launches")
    assert n in (3, 4, 6)
    ws = M.alloc_workspace(layer, T, flags)
    ref = torch.empty((T, layer.H), dtype=torch.float32, device=DEV)
    M.moe_layer_forward(layer, x, ref, ws, flags)
    out = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=DEV)
    ws2 = M.alloc_workspace(layer, T, flags)
    for ph in range(n):
        M.moe_layer_forward_phase(layer, x, out, ws2, ph, flags)
    torch.cuda.synchronize()
    if flags & ATOMIC:   # summation order not fixed
        assert O.error_stats(out.cpu().numpy(), ref.cpu().numpy())["max_rel"] < 1e-5
    else:
        assert torch.equal(out, ref)
    with pytest.raises(M.MoEError):
        M.moe_layer_forward_phase(layer, x, out, ws2, n, flags)


@pytest.mark.parametrize("T,H,init", [(37, 320, False), (3, 2048, False), (5, 2048, True),
                                      (64, 64, False)])
def test_residual_rmsnorm_kernel(T, H, init):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    rng = np.random.default_rng(T * 7 + H)
    r0 = (rng.standard_normal((T, H)) * 3.0).astype(np.float32)
    y = rng.standard_normal((T, H)).astype(np.float32)
    xh = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    r = torch.from_numpy(r0).to(DEV)
    yd = torch.from_numpy(y).to(DEV)
    xd = torch.from_numpy(xh.view(np.int16)).to(DEV)
    M.moe_residual_rmsnorm(None if init else yd, r, xd, init=init)
    torch.cuda.synchronize()
    if init:
        want_r, want_x = O.residual_rmsnorm(O.bf16_to_f64(xh), None)
        assert np.array_equal(r.cpu().numpy().astype(np.float64), want_r)   # exact widening
    else:
        want_r, want_x = O.residual_rmsnorm(r0, y)
        got_r = r.cpu().numpy().astype(np.float64)
        assert np.abs(got_r - want_r).max() <= 2 ** -23 * np.abs(want_r).max()  # one fp32 add
    got_x = u16(xd)
    # fp32 statistics against fp64: a bf16 rounding may flip where the value sits within
    # about 1e-6 of a rounding boundary; at most a handful, each by one unit in the last place
    diff = got_x.astype(np.int32) - want_x.astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert (diff != 0).mean() <= 2e-3, (diff != 0).mean()


def _layerwise(layers_dev, layers_host, name, T, flags, stream):
    """The stack evaluated one C-ABI call at a time on the GPU, each layer checked against the
    oracle on the GPU's own input; returns the GPU's final (resid, x)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = synth.SHAPES[name]
    xh, x = tokens(name, T, stream=stream)
    resid = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
    M.moe_residual_rmsnorm(None, resid, x, init=True)
    y = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
    sel = np.arange(T) if T <= 64 else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(T).choice(T, 30, replace=False)]))
    for l, (ld, lh) in enumerate(zip(layers_dev, layers_host)):
        ws = M.alloc_workspace(ld, T, flags)
        M.moe_layer_forward(ld, x, y, ws, flags)
        torch.cuda.synchronize()
        x_in = u16(x)
        gidx = gpu_routing(ld, x, T)
        ref, ref_exact, ties, swapped = oracle_reference(name, lh, x_in, s.K, tokens_sel=sel,
                                                         gpu_idx=gidx)
        st = O.error_stats(y.cpu().numpy()[sel], ref)
        log(f"[stack] {name} T={T} layer {l}: max_rel={st['max_rel']:.3e} "
            f"mean_abs={st['mean_abs']:.3e} near-ties={len(ties)} rerouted={swapped}")
        assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS, (l, st)
        M.moe_residual_rmsnorm(y, resid, x)
    torch.cuda.synchronize()
    return xh, resid, x


@pytest.mark.parametrize("name,T,nl", [("mid", 13, 3), ("mid", 300, 3), ("full", 1, 2),
                                       ("full", 512, 2), ("odd", 16, 2), ("solo", 1, 3),
                                       ("many", 1, 2), ("many", 16, 2)])
def test_stack_matches_layerwise_and_oracle(name, T, nl):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    log(f"[stack] start {name} T={T} layers={nl}")
    layers_dev = [device_layer(name, 0, l) for l in range(nl)]
    layers_host = [host_layer(name, 0, l) for l in range(nl)]
    xh, r_lw, x_lw = _layerwise(layers_dev, layers_host, name, T, 0, stream=50)
    stack = M.Stack(layers_dev)
    ws = stack.alloc_workspace(T)
    x = torch.from_numpy(xh.view(np.int16)).to(DEV)
    resid = torch.empty((T, layers_dev[0].H), dtype=torch.float32, device=DEV)
    stack.forward(resid, x, ws)
    torch.cuda.synchronize()
    assert torch.equal(resid, r_lw) and torch.equal(x, x_lw)
    if T > 16:
        # the atomic combine: its summation order is not fixed, and each layer's
        # input is re-rounded to bf16, so a last-bit difference can move an input by one bf16
        # step and grow over the layers; each layer is therefore checked against the oracle on
        # its own input, and the stack call against the layer-wise run within the parity bar
        _, r_at, _ = _layerwise(layers_dev, layers_host, name, T, ATOMIC, stream=50)
        ws0 = stack.alloc_workspace(T, ATOMIC)
        x0 = torch.from_numpy(xh.view(np.int16)).to(DEV)
        r0 = torch.empty_like(resid)
        stack.forward(r0, x0, ws0, ATOMIC)
        torch.cuda.synchronize()
        st = O.error_stats(r0.cpu().numpy(), r_at.cpu().numpy())
        log(f"[stack] atomic-combine stack vs its layer-wise run: {st}")
        assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS


def test_stack_of_small_layers_end_to_end():
    """Two small layers with no routing near-ties: the whole stack against the oracle's
    stack_forward (no teacher forcing)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    name, T = "tiny", 8
    layers_dev = [device_layer(name, 0, l) for l in range(2)]
    layers_host = [host_layer(name, 0, l) for l in range(2)]
    xh, x = tokens(name, T, stream=60)
    resid = torch.empty((T, layers_dev[0].H), dtype=torch.float32, device=DEV)
    stack = M.Stack(layers_dev)
    ws = stack.alloc_workspace(T)
    stack.forward(resid, x, ws)
    torch.cuda.synchronize()
    # the seed is chosen with no routing near-tie in either layer of the oracle's stack
    r1, x1 = O.residual_rmsnorm(O.bf16_to_f64(xh), None)
    for lh in layers_host:
        logits = O.router_logits(x1, lh["router_w"], lh["router_bias"])
        assert len(O.near_ties(logits, layers_dev[0].K)) == 0
        r1, x1 = O.residual_rmsnorm(r1, O.layer_forward(lh, x1, layers_dev[0].K))
    want_r, want_x = O.stack_forward(layers_host, xh, layers_dev[0].K)
    st = O.error_stats(resid.cpu().numpy(), want_r)
    sx = O.error_stats(O.bf16_to_f64(u16(x)), O.bf16_to_f64(want_x))
    log(f"[stack] tiny end-to-end: resid {st} | next input {sx}")
    assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS
    assert sx["max_rel"] <= TOL_MAX_REL and sx["mean_abs"] <= TOL_MEAN_ABS


def test_stack_prefill_then_fed_back_decode_steps():
    """A 64-token prefill chunk through two full-size layers (every token checked, layer by
    layer), then 8 decode steps whose input is the previous step's normalised output left on
    the device ([P1 "How It Works ..."]: the next step's input stays GPU-resident). Each step is
    checked layer by layer against the oracle on the GPU's own input, and the stack call must
    give the layer-by-layer composition bit for bit, step after step."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    name, nl = "full", 2
    layers_dev = [device_layer(name, 0, l) for l in range(nl)]
    layers_host = [host_layer(name, 0, l) for l in range(nl)]
    log("[stack] prefill chunk T=64, 2 layers, every token")
    xh, r_lw, x_lw = _layerwise(layers_dev, layers_host, name, 64, 0, stream=70)
    stack = M.Stack(layers_dev)
    ws = stack.alloc_workspace(64)
    x = torch.from_numpy(xh.view(np.int16)).to(DEV)
    resid = torch.empty((64, layers_dev[0].H), dtype=torch.float32, device=DEV)
    stack.forward(resid, x, ws)
    torch.cuda.synchronize()
    assert torch.equal(resid, r_lw) and torch.equal(x, x_lw)
    # decode: the first step takes the prefill's last normalised row, then each step its own
    x_step = x[63:64].clone()
    ws1 = stack.alloc_workspace(1)
    r1 = torch.empty((1, layers_dev[0].H), dtype=torch.float32, device=DEV)
    for step in range(8):
        log(f"[stack] decode step {step}")
        _, r_ref, x_ref = _layerwise_from(layers_dev, layers_host, name, x_step.clone(), step)
        xs = x_step.clone()
        stack.forward(r1, xs, ws1)
        torch.cuda.synchronize()
        assert torch.equal(r1, r_ref) and torch.equal(xs, x_ref), step
        x_step = xs


def _layerwise_from(layers_dev, layers_host, name, x, tag):
    """_layerwise for a device input x [T, H] bf16 (updated in place to the next input)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = synth.SHAPES[name]
    T = x.shape[0]
    resid = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
    M.moe_residual_rmsnorm(None, resid, x, init=True)
    y = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
    for l, (ld, lh) in enumerate(zip(layers_dev, layers_host)):
        ws = M.alloc_workspace(ld, T)
        M.moe_layer_forward(ld, x, y, ws)
        torch.cuda.synchronize()
        x_in = u16(x)
        gidx = gpu_routing(ld, x, T)
        ref, _, ties, swapped = oracle_reference(name, lh, x_in, s.K, gpu_idx=gidx)
        st = O.error_stats(y.cpu().numpy(), ref)
        log(f"[stack]   step {tag} layer {l}: max_rel={st['max_rel']:.3e} "
            f"mean_abs={st['mean_abs']:.3e} near-ties={len(ties)} rerouted={swapped}")
        assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS, (l, st)
        M.moe_residual_rmsnorm(y, resid, x)
    torch.cuda.synchronize()
    return None, resid, x
