"""The gated delta-rule recurrence (delta_rule_forward and delta_rule_forward_chunked, through the
C ABI) against the fp64 oracle, element by element: outputs of every token and the final state.

Tolerance (derived from the arithmetic; the layer's 2e-2 / 2e-3 bounds are for the MoE layer):
the state and every product are fp32 and each step contracts the state (alpha <= 1 and
I - beta kh kh^T has norm at most 1), so rounding errors stay at a few fp32 ulps of the
state's scale over any number of tokens; the gate is a row-normalised max relative error of
1e-4 on o and on the state. The chunked form computes the same quantities in another order
(within a chunk through (I + M)^-1 and decays exp(G_s - G_r)), under the same gate.
"""
import numpy as np
import pytest

import synth
from gpu_common import DEV, log
from oracle import delta_oracle as Dn
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-4


def run(shape, B, T, seed=0, zero_state=False, inplace=False, with_state=True, chunked=False):
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, B, T, seed, zero_state)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    qd, kd, vd = dev(q, np.int16), dev(k, np.int16), dev(v, np.int16)
    gd, bd = dev(g, np.float32), dev(beta, np.float32)
    sin = dev(s0, np.float32) if with_state else None
    sout = sin if inplace else torch.full(s0.shape, float("nan"), dtype=torch.float32, device=DEV)
    o = torch.full((B, T, shape.num_v_heads, shape.dv), float("nan"), dtype=torch.float32, device=DEV)
    if chunked:
        ws = DR.alloc_chunked_workspace(d, B, T, device=DEV)
        ws.fill_(0xFF)  # whatever the workspace holds on entry is overwritten
        DR.forward_chunked(d, qd, kd, vd, gd, bd, sin, sout, o, ws)
    else:
        DR.forward(d, qd, kd, vd, gd, bd, sin, sout, o)
    torch.cuda.synchronize()
    ref_o, ref_s = Dn.recurrence(q, k, v, g, beta, s0 if with_state else np.zeros_like(s0),
                                 scale=d.scale, eps=d.eps)
    return o.cpu().numpy().astype(np.float64), sout.cpu().numpy().astype(np.float64), ref_o, ref_s


def check(tag, o, s, ref_o, ref_s):
    so = O.error_stats(o.reshape(-1, o.shape[-1]), ref_o.reshape(-1, ref_o.shape[-1]))
    ss = O.error_stats(s.reshape(-1, s.shape[-1]), ref_s.reshape(-1, ref_s.shape[-1]))
    log(f"[delta] {tag}: o max_rel={so['max_rel']:.2e} mean_abs={so['mean_abs']:.2e} | "
        f"state max_rel={ss['max_rel']:.2e} mean_abs={ss['mean_abs']:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert so["max_rel"] <= TOL and ss["max_rel"] <= TOL


@pytest.mark.parametrize("name,B,T", [("tiny", 3, 7), ("mid", 2, 33), ("full", 1, 1),
                                      ("full", 8, 1), ("full", 2, 64), ("gva", 1, 40),
                                      ("full", 1, 256), ("full", 1, 512), ("wide", 3, 5),
                                      ("wide", 2, 40)])
def test_recurrence_matches_oracle(name, B, T):
    shape = synth.DELTA_SHAPES[name]
    log(f"[delta] start {name} B={B} T={T}")
    check(f"{name} B={B} T={T}", *run(shape, B, T, seed=B * 100 + T))


@pytest.mark.parametrize("name,B,T", [("tiny", 3, 7), ("tiny", 2, 65), ("mid", 2, 33), ("mid", 1, 96),
                                      ("full", 1, 1), ("full", 8, 1), ("full", 2, 31),
                                      ("full", 2, 32), ("full", 1, 64), ("gva", 1, 40),
                                      ("gva", 2, 100), ("full", 1, 256), ("full", 1, 512),
                                      ("wide", 3, 5), ("wide", 2, 70)])
def test_chunked_recurrence_matches_oracle(name, B, T):
    shape = synth.DELTA_SHAPES[name]
    log(f"[delta] chunked start {name} B={B} T={T}")
    check(f"chunked {name} B={B} T={T}", *run(shape, B, T, seed=B * 100 + T + 7, chunked=True))


def test_chunked_zero_state_in_place_and_no_token():
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    shape = synth.DELTA_SHAPES["full"]
    check("chunked no state", *run(shape, 2, 40, seed=13, with_state=False, chunked=True))
    check("chunked in place", *run(shape, 2, 70, seed=14, inplace=True, chunked=True))
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, 1, 0, 5)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    sout = torch.full(s0.shape, float("nan"), dtype=torch.float32, device=DEV)
    o = torch.empty((1, 0, shape.num_v_heads, shape.dv), dtype=torch.float32, device=DEV)
    DR.forward_chunked(d, dev(q, np.int16), dev(k, np.int16), dev(v, np.int16),
                       dev(g, np.float32), dev(beta, np.float32), dev(s0, np.float32), sout, o,
                       torch.empty(16, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(sout.cpu().numpy(), s0)


def test_chunked_graph_replays_match_eager():
    """A captured chunked call replayed three times, with eager calls on other buffers in
    between, gives the eager result bit for bit each time."""
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    shape = synth.DELTA_SHAPES["full"]
    B, T = 1, 100
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, B, T, 15)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    args = (dev(q, np.int16), dev(k, np.int16), dev(v, np.int16), dev(g, np.float32),
            dev(beta, np.float32), dev(s0, np.float32))
    ws = DR.alloc_chunked_workspace(d, B, T, device=DEV)
    s_e = torch.empty(s0.shape, device=DEV)
    o_e = torch.empty((B, T, shape.num_v_heads, shape.dv), device=DEV)
    DR.forward_chunked(d, *args, s_e, o_e, ws)
    torch.cuda.synchronize()
    s_g, o_g = torch.empty_like(s_e), torch.empty_like(o_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        DR.forward_chunked(d, *args, s_g, o_g, ws)
    ws2 = DR.alloc_chunked_workspace(d, B, T, device=DEV)
    for rep in range(3):
        s_g.fill_(float("nan"))
        o_g.fill_(float("nan"))
        DR.forward_chunked(d, *args, torch.empty_like(s_e), torch.empty_like(o_e), ws2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(s_g, s_e) and torch.equal(o_g, o_e), rep


def test_zero_initial_state_and_in_place_update():
    shape = synth.DELTA_SHAPES["full"]
    check("full no state", *run(shape, 2, 5, seed=3, with_state=False))
    check("full in place", *run(shape, 2, 5, seed=4, inplace=True))


def test_decode_steps_chain_like_one_run():
    """Four single-token calls, each starting from the previous call's state, give the outputs
    and the state of one four-token call bit for bit (the same arithmetic per token)."""
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    shape = synth.DELTA_SHAPES["full"]
    B, T = 2, 4
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, B, T, 9)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    o_all = torch.empty((B, T, shape.num_v_heads, shape.dv), device=DEV)
    s_all = torch.empty(s0.shape, device=DEV)
    DR.forward(d, dev(q, np.int16), dev(k, np.int16), dev(v, np.int16), dev(g, np.float32),
               dev(beta, np.float32), dev(s0, np.float32), s_all, o_all)
    s = dev(s0, np.float32)
    outs = []
    for t in range(T):
        o1 = torch.empty((B, 1, shape.num_v_heads, shape.dv), device=DEV)
        sl = slice(t, t + 1)
        DR.forward(d, dev(q[:, sl], np.int16), dev(k[:, sl], np.int16), dev(v[:, sl], np.int16),
                   dev(g[:, sl], np.float32), dev(beta[:, sl], np.float32), s, s, o1)
        outs.append(o1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_all) and torch.equal(s, s_all)


@pytest.mark.parametrize("with_state", [True, False])
def test_no_token_passes_the_state_through(with_state):
    """T = 0: the state comes out unchanged (zero when none is given); no output rows."""
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    shape = synth.DELTA_SHAPES["full"]
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, 2, 0, 5)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    sin = dev(s0, np.float32) if with_state else None
    sout = torch.full(s0.shape, float("nan"), dtype=torch.float32, device=DEV)
    o = torch.empty((2, 0, shape.num_v_heads, shape.dv), dtype=torch.float32, device=DEV)
    DR.forward(d, dev(q, np.int16), dev(k, np.int16), dev(v, np.int16), dev(g, np.float32),
               dev(beta, np.float32), sin, sout, o)
    torch.cuda.synchronize()
    want = s0 if with_state else np.zeros_like(s0)
    assert np.array_equal(sout.cpu().numpy(), want)


def test_graph_replays_match_eager():
    """A captured call replayed three times, with eager calls on other buffers in between, gives
    the eager result bit for bit each time."""
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    shape = synth.DELTA_SHAPES["full"]
    B, T = 2, 3
    q, k, v, g, beta, s0 = synth.make_delta_inputs(shape, B, T, 12)
    d = DR.desc(shape.num_k_heads, shape.num_v_heads, shape.dk, shape.dv)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    args = (dev(q, np.int16), dev(k, np.int16), dev(v, np.int16), dev(g, np.float32),
            dev(beta, np.float32), dev(s0, np.float32))
    s_e = torch.empty(s0.shape, device=DEV)
    o_e = torch.empty((B, T, shape.num_v_heads, shape.dv), device=DEV)
    DR.forward(d, *args, s_e, o_e)
    torch.cuda.synchronize()
    s_g, o_g = torch.empty_like(s_e), torch.empty_like(o_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        DR.forward(d, *args, s_g, o_g)
    for rep in range(3):
        s_g.fill_(float("nan"))
        o_g.fill_(float("nan"))
        DR.forward(d, *args, torch.empty_like(s_e), torch.empty_like(o_e))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(s_g, s_e) and torch.equal(o_g, o_e), rep
