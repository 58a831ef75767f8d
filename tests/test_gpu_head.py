"""The greedy decode step (moe_greedy_next_input, through the C ABI) against the fp64 oracle:
logits, the chosen token, and the next input (the token's embedding row, bit for bit).

Tolerances (derived from the arithmetic): the logits are fp32 sums of exact bf16 products over H
inputs, so they agree with the fp64 sums of the same bf16-rounded weights to about 1e-6 of the
row's scale (gate: row-normalised max relative error 1e-5). The token must be the oracle's,
except for a row whose two largest fp64 logits are closer than 1e-4, where it must be one of the
tied entries. The next input is an exact function of the token: bit-exact."""
import functools

import numpy as np
import pytest

import synth
from gpu_common import DEV, device_layer, log
from oracle import head_oracle as Hd
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL_LOGITS = 1e-5


@functools.lru_cache(maxsize=None)
def host_head(V, H, seed=0):
    return synth.make_head(V, H, seed)


@functools.lru_cache(maxsize=None)
def dev_head(V, H, seed=0):
    from bit_grouped_gemm_amd import greedy_head as Gh
    return Gh.upload_head(host_head(V, H, seed), device=DEV)


def run(V, H, T, seed=0, stream=0, x_host=None, inplace=False):
    import torch
    from bit_grouped_gemm_amd import greedy_head as Gh
    hd = dev_head(V, H, seed)
    if x_host is None:
        x_host = synth.make_tokens(synth.LayerShape(H, 8, 2, 64, 64), T, seed=seed, stream=stream)
    x = torch.from_numpy(x_host.view(np.int16)).to(DEV)
    tok = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    xn = x if inplace else torch.full_like(x, -1)
    ws = Gh.alloc_workspace(V, T)
    Gh.next_input(hd, x, tok, xn, ws)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), xn.cpu().numpy().view(np.uint16),
            Gh.logits_of(ws, V, T).cpu().numpy().astype(np.float64), x_host)


def check(V, H, T, tok, xn, lg, x_host, seed=0):
    w = host_head(V, H, seed)
    ref = Hd.lm_logits(x_host, w["head"])
    st = O.error_stats(lg, ref)
    ties = set(Hd.near_tie(ref).tolist())
    want = Hd.greedy(ref)
    log(f"[head] V={V} H={H} T={T}: logits max_rel={st['max_rel']:.2e}, tokens {tok.tolist()[:4]}..., "
        f"{len(ties)} near-tie rows")
    assert st["max_rel"] <= TOL_LOGITS, st
    for t in range(T):
        if tok[t] != want[t]:
            assert t in ties, (t, tok[t], want[t])
            assert ref[t, want[t]] - ref[t, tok[t]] < 1e-4
    assert np.array_equal(xn, Hd.embed(tok, w["embed"]))


@pytest.mark.parametrize("V,H,T", [(151936, 2048, 3), (1, 512, 1), (7, 512, 2),
                                   (1000, 1024, 16), (40000, 4096, 8), (5000, 2048, 16),
                                   (33, 2048, 5)])
def test_greedy_step_matches_oracle(V, H, T):
    log(f"[head] start V={V} H={H} T={T}")
    tok, xn, lg, xh = run(V, H, T, seed=1, stream=T)
    check(V, H, T, tok, xn, lg, xh, seed=1)


def test_ties_go_to_the_lowest_index_and_x_may_be_updated_in_place():
    """All rows equal (nibbles 9, bias -8*scale, one scale) except rows 3 and 10, which are equal
    to each other and larger (nibbles 15): with a positive input every logit ties but rows 3 and
    10, which tie above the rest, and the token is 3. The next input overwrites x."""
    import torch
    from bit_grouped_gemm_amd import greedy_head as Gh
    V, H = 64, 512
    q, s, b = (a.copy() for a in synth.make_head(V, H, seed=2)["head"])
    q[:] = 0x99999999
    s[:] = s[0, 0, 0]
    b[:] = b[0, 0, 0]
    q[0, 3] = q[0, 10] = 0xFFFFFFFF
    host = {"head": (q, s, b), "embed": synth.make_head(V, H, seed=2)["embed"]}
    hd = Gh.upload_head(host, device=DEV)
    xh = np.full((2, H), 0x3F80, np.uint16)        # 1.0
    x = torch.from_numpy(xh.view(np.int16)).to(DEV)
    tok = torch.empty(2, dtype=torch.int32, device=DEV)
    ws = Gh.alloc_workspace(V, 2)
    Gh.next_input(hd, x, tok, x, ws)
    torch.cuda.synchronize()
    assert tok.cpu().tolist() == [3, 3]
    assert np.array_equal(x.cpu().numpy().view(np.uint16), Hd.embed([3, 3], host["embed"]))


def test_graph_replays_match_eager():
    import torch
    from bit_grouped_gemm_amd import greedy_head as Gh
    V, H, T = 151936, 2048, 1
    tok_e, xn_e, _, xh = run(V, H, T, seed=1, stream=5)
    hd = dev_head(V, H, 1)
    x = torch.from_numpy(xh.view(np.int16)).to(DEV)
    tok = torch.empty(T, dtype=torch.int32, device=DEV)
    xn = torch.empty_like(x)
    ws = Gh.alloc_workspace(V, T)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Gh.next_input(hd, x, tok, xn, ws)
    for rep in range(3):
        tok.fill_(-1)
        xn.fill_(-1)
        Gh.next_input(hd, x, torch.empty_like(tok), torch.empty_like(xn), Gh.alloc_workspace(V, T))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), tok_e), rep
        assert np.array_equal(xn.cpu().numpy().view(np.uint16), xn_e), rep


def test_decode_loop_through_the_stack_and_the_greedy_step():
    """Three decode steps of two full-size layers and a full-size head: each step's final
    normalised state goes through the greedy step, whose embedding is the next step's input, all
    on the device. Each greedy step is checked against the oracle on the GPU's own state."""
    import torch
    from bit_grouped_gemm_amd import greedy_head as Gh
    from bit_grouped_gemm_amd import moe_w4 as M
    V, H = 151936, 2048
    stack = M.Stack([device_layer("full", 0, l) for l in range(2)])
    ws = stack.alloc_workspace(1)
    hd = dev_head(V, H, 0)
    wsg = Gh.alloc_workspace(V, 1)
    first = Hd.embed([17], host_head(V, H, 0)["embed"])
    x = torch.from_numpy(first.view(np.int16)).to(DEV)
    r = torch.empty((1, H), dtype=torch.float32, device=DEV)
    tok = torch.empty(1, dtype=torch.int32, device=DEV)
    for step in range(3):
        stack.forward(r, x, ws)
        torch.cuda.synchronize()
        xf = x.cpu().numpy().view(np.uint16).copy()
        Gh.next_input(hd, x, tok, x, wsg)
        torch.cuda.synchronize()
        t = tok.cpu().numpy()
        log(f"[head] decode step {step}: token {int(t[0])}")
        check(V, H, 1, t, x.cpu().numpy().view(np.uint16), Gh.logits_of(wsg, V, 1).cpu().numpy()
              .astype(np.float64), xf)
