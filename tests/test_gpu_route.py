"""moe_route and moe_permute against the oracle: expert ids, per-expert counts, offsets, the
stable permutation and the block map are compared exactly; routing weights and the shared
gate to fp32 accuracy. Near-ties (gap < 1e-4) may be ordered differently and are reported."""
import numpy as np
import pytest

from gpu_common import DEV, device_layer, host_layer, log, tokens
import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def route(layer, x, T):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    K = layer.K
    idx = torch.full((T * K,), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T * K,), float("nan"), dtype=torch.float32, device=DEV)
    sg = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    cnt = torch.full((layer.E,), -7, dtype=torch.int32, device=DEV)
    ws = M.alloc_workspace(layer, T)
    M.moe_route(layer, x, idx, w, sg, cnt, ws)
    torch.cuda.synchronize()
    return (idx.cpu().numpy().reshape(T, K), w.cpu().numpy().reshape(T, K), sg.cpu().numpy(),
            cnt.cpu().numpy())


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 1), ("odd", 9), ("odd", 1000),
                                    ("mid", 300), ("mid", 16), ("full", 1), ("full", 8),
                                    ("full", 4096), ("full_skew", 4096)])
def test_route_matches_oracle(name, T):
    log(f"[route] {name} T={T}")
    layer, host = device_layer(name), host_layer(name)
    xh, x = tokens(name, T)
    gi, gw, gs, gc = route(layer, x, T)
    logits = O.router_logits(xh, host["router_w"], host["router_bias"])
    ridx, _ = O.select_topk(logits, layer.K)
    ties = set(O.near_ties(logits, layer.K).tolist())
    diff = [t for t in range(T) if not np.array_equal(gi[t], ridx[t])]
    log(f"[route]   near-ties={len(ties)} differing={diff}")
    assert set(diff) <= ties
    for t in diff:  # a tie-equivalent choice: same logits multiset up to the tie gap
        a = np.sort(logits[t, gi[t]])
        b = np.sort(logits[t, ridx[t]])
        assert np.allclose(a, b, atol=1e-4, rtol=0)
    assert np.all((gi >= 0) & (gi < layer.E))
    assert all(len(set(r)) == layer.K for r in gi)
    # weights: softmax of the (fp64) logits of the chosen experts, to fp32 accuracy
    sel = np.take_along_axis(logits, gi.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    assert np.abs(gw - p).max() < 5e-6
    assert np.abs(gw.sum(axis=1) - 1).max() < 2e-6
    assert np.abs(gs - O.shared_gate(xh, host["shared_gate_w"])).max() < 2e-6
    assert np.array_equal(gc, np.bincount(gi.ravel(), minlength=layer.E))
    if not diff:
        assert np.array_equal(gc, O.permute(ridx, layer.E)[0])


def _dummy_desc(E, K, Fs):
    """A descriptor whose weight pointers are valid but never read (permutation only)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    buf = torch.zeros(1024, dtype=torch.int32, device=DEV)
    t = {"router_w": buf.view(torch.float32), "shared_gate_w": buf.view(torch.float32)}
    w = (buf, buf.view(torch.int16), buf.view(torch.int16))
    for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        t[n] = w
    layer = M.make_layer(t, 64, E, K, 64, Fs)
    layer.tensors["_keep"] = buf
    return layer


def _routing(T, E, K, rng, skew=False):
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
        return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


@pytest.mark.parametrize("E,K,T,Fs,skew", [
    (16, 2, 4, 64, False), (7, 3, 1000, 64, False), (32, 4, 300, 0, False), (256, 8, 1, 64, False),
    (256, 8, 8, 64, False), (256, 8, 4096, 64, False), (256, 8, 4096, 64, True),
    (1024, 32, 200, 64, False), (1024, 1, 1, 0, False), (64, 32, 130, 64, False),
    # up to 8192 slots the permutation is one workgroup, above it three passes (histogram
    # rows, scan, scatter): both sides of the limit
    (256, 8, 1024, 64, True), (256, 8, 1025, 64, False), (128, 32, 1100, 0, False),
])
def test_permute_matches_oracle(E, K, T, Fs, skew):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    log(f"[permute] E={E} K={K} T={T} skew={skew}")
    rng = np.random.default_rng(E * 1000 + K * 10 + T)
    idx = _routing(T, E, K, rng, skew)
    layer = _dummy_desc(E, K, Fs)
    plan = M.alloc_plan(layer, T)
    ws = M.alloc_workspace(layer, T, M.MOE_FLAG_ATOMIC_COMBINE)
    M.moe_permute(layer, torch.from_numpy(idx.ravel()).to(DEV), T, plan, ws)
    torch.cuda.synchronize()
    counts, offsets, sorted_slots, slot_pos = O.permute(idx, E)
    TK = T * K
    assert np.array_equal(plan["counts"].cpu().numpy(), counts)
    assert np.array_equal(plan["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(plan["sorted_slots"].cpu().numpy()[:TK], sorted_slots)
    assert np.array_equal(plan["slot_pos"].cpu().numpy()[:TK], slot_pos)
    # block map: tiles of at most MOE_BLOCK_M rows per non-empty expert in expert order, then
    # the shared expert's T rows
    BM = M.MOE_BLOCK_M
    want = [(e, m0, min(BM, int(counts[e]) - m0), int(offsets[e]) + m0)
            for e in range(E) for m0 in range(0, int(counts[e]), BM)]
    if Fs > 0:
        want += [(E, m0, min(BM, T - m0), TK + m0) for m0 in range(0, T, BM)]
    nb = int(plan["num_blocks"].cpu().item())
    got = [tuple(r) for r in plan["blocks"].cpu().numpy().reshape(-1, 4)[:nb].tolist()]
    assert nb == len(want) and got == want
    assert nb <= M.moe_plan_max_blocks(layer, T)


def test_permute_flags_invalid_expert_ids():
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    E, K, T = 16, 2, 50
    idx = _routing(T, E, K, np.random.default_rng(0))
    idx[17, 1] = E          # out of range
    layer = _dummy_desc(E, K, 64)
    plan = M.alloc_plan(layer, T)
    ws = M.alloc_workspace(layer, T, M.MOE_FLAG_ATOMIC_COMBINE)
    M.moe_permute(layer, torch.from_numpy(idx.ravel()).to(DEV), T, plan, ws)
    torch.cuda.synchronize()
    assert int(plan["num_blocks"].cpu().item()) == -1
    assert int(plan["counts"].cpu().numpy().sum()) == T * K - 1


def test_route_negative_logits_and_exact_ties():
    """Every logit far below zero (router bias -60) and exact ties (duplicated router rows):
    the selection must not treat zero as a floor, and equal logits go to the lower expert index.
    Checked through moe_route and through the layer's decode and prefill paths."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    from gpu_common import TOL_MAX_REL, TOL_MEAN_ABS
    base = host_layer("mid")
    host = dict(base)
    rw = base["router_w"].copy()
    for a, b in ((4, 5), (3, 17), (31, 30), (0, 9)):
        rw[b] = rw[a]          # expert b scores exactly like expert a
    host["router_w"] = rw
    host["router_bias"] = np.full(rw.shape[0], -60.0, np.float32)
    s = synth.SHAPES["mid"]
    layer = M.upload_layer(host, s.H, s.E, s.K, s.F, s.Fs, device=DEV)
    for T in (1, 8, 300):
        xh, x = tokens("mid", T, stream=40)
        gi, gw, _, _ = route(layer, x, T)
        logits = O.router_logits(xh, host["router_w"], host["router_bias"])
        assert logits.max() < -50
        ridx, rp = O.select_topk(logits, layer.K)
        assert np.array_equal(gi, ridx), T
        assert np.abs(gw - rp).max() < 5e-6
        for flags in (0, M.MOE_FLAG_FORCE_PREFILL):
            ws = M.alloc_workspace(layer, T, flags)
            out = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
            M.moe_layer_forward(layer, x, out, ws, flags)
            torch.cuda.synchronize()
            st = O.error_stats(out.cpu().numpy(), O.layer_forward(host, xh, layer.K, "bf16"))
            log(f"[route] ties/negative T={T} flags={flags}: {st}")
            assert st["max_rel"] <= TOL_MAX_REL and st["mean_abs"] <= TOL_MEAN_ABS
