"""The decode path's three launches, each checked on its own at the full layer size.

moe_layer_forward_phase runs one launch at a time; the workspace regions it leaves (located
through the test export moe_debug_workspace_layout) are read back after each launch:

  phase 0 (router logits, shared-gate logit, shared expert's gate/up + SwiGLU)
      logits against the oracle's fp64 logits; shared A rows against RNE(oracle SwiGLU)
  phase 1 (top-k in every workgroup, routed gate/up + SwiGLU)
      the route record (entries, rows, token masks: bit-exact; routing weights and shared
      gates against the oracle's softmax and sigmoid); routed A rows against RNE(oracle SwiGLU)
  phase 2 (down projection fused with the weighted combine)
      out against the fp64 down products of the library's own A rows, weighted by the
      library's own routing weights

A token whose fp64 logits have a near-tie (gap < 1e-4) may be routed to a tie-equivalent set;
it is then checked against that set ([P1 "The Model ..."]: 256 experts scored, 8 chosen).
"""
import numpy as np
import pytest

from gpu_common import DEV, device_layer, host_layer, log, tokens
from oracle import moe_oracle as O
from test_gpu_stages import check_a

pytestmark = pytest.mark.gpu


def _layer(name, shared):
    """Device and host layers; shared=False drops the shared expert of the same weights."""
    from bit_grouped_gemm_amd import moe_w4 as M
    dl, hl = device_layer(name), host_layer(name)
    if shared:
        return dl, hl
    hl = dict(hl)
    hl["sh_gate"] = hl["sh_up"] = hl["sh_down"] = None
    return M.make_layer(dict(dl.tensors), dl.H, dl.E, dl.K, dl.F, 0), hl


def _deq(host, name, e):
    q, s, b = host[name]
    return O.dequant(q[e], s[e], b[e], "bf16")


def _read(ws, off, n, dtype):
    """n 4-byte words of the workspace at byte offset off, as a numpy array of dtype."""
    return ws[off:off + n * 4].cpu().numpy().view(dtype)


def _routing(host, xh, K):
    """Oracle selection/weights, near-tie tokens and the fp64 logits."""
    logits = O.router_logits(xh, host["router_w"], host["router_bias"])
    idx, p = O.select_topk(logits, K)
    return logits, idx, p, set(O.near_ties(logits, K).tolist())


@pytest.mark.parametrize("name,T,shared", [("full", 1, True), ("full", 8, True),
                                           ("full", 16, True), ("full", 1, False),
                                           ("full", 8, False), ("full_skew", 8, True)])
def test_decode_launches_one_by_one(name, T, shared):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    log(f"[dec-stages] {name} T={T} shared={shared}")
    layer, host = _layer(name, shared)
    H, E, K, F, Fs = layer.H, layer.E, layer.K, layer.F, layer.Fs
    TK = T * K
    assert M.moe_layer_num_phases(layer, T) == 3
    xh, x = tokens(name, T, stream=90 + T)
    lay = M.moe_debug_workspace_layout(layer, T)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    xf = O.bf16_to_f64(xh)
    logits_ref, idx_ref, p_ref, ties = _routing(host, xh, K)

    # ---- phase 0: router logits, shared-gate logits, shared expert's A rows
    M.moe_layer_forward_phase(layer, x, out, ws, 0)
    torch.cuda.synchronize()
    lg = _read(ws, lay["logits"], T * E + T, np.float32).astype(np.float64)
    err = np.abs(lg[:T * E].reshape(T, E) - logits_ref).max()
    log(f"[dec-stages]   logits max abs error {err:.2e}")
    assert err < 1e-5
    if Fs:
        g_ref = xf @ np.asarray(host["shared_gate_w"], np.float64)
        gerr = np.abs(lg[T * E:] - g_ref).max()
        log(f"[dec-stages]   shared-gate logits max abs error {gerr:.2e}")
        assert gerr < 1e-5
        a_all = ws[lay["a"]:lay["a"] + (TK * F + T * Fs) * 2].view(torch.int16).cpu().numpy()
        a_sh = O.bf16_to_f64(a_all.view(np.uint16)[TK * F:]).reshape(T, Fs)
        wg, wu = _deq(host, "sh_gate", 0), _deq(host, "sh_up", 0)
        check_a(a_sh, O.round_to_bf16(O.silu(xf @ wg.T) * (xf @ wu.T)), "shared A (phase 0)")

    # ---- phase 1: route record and the routed A rows
    M.moe_layer_forward_phase(layer, x, out, ws, 1)
    torch.cuda.synchronize()
    nrw = 1 + 5 * TK + T
    rec = _read(ws, lay["route"], nrw, np.int32)
    recf = rec.view(np.float32)
    D = int(rec[0])
    ent_e, ent_m = rec[1:1 + D], rec[1 + TK:1 + TK + D]
    ent_row0, ent_mask = rec[1 + 2 * TK:1 + 2 * TK + D], rec[1 + 3 * TK:1 + 3 * TK + D].view(np.uint32)
    row_w, sgs = recf[1 + 4 * TK:1 + 5 * TK], recf[1 + 5 * TK:1 + 5 * TK + T]
    # per token: the library's experts with their weights and grouped rows
    lib_sel = [dict() for _ in range(T)]
    if T == 1:
        assert D == K and np.array_equal(ent_m, np.ones(K)) and np.array_equal(ent_row0, np.arange(K))
        assert np.array_equal(ent_mask, np.ones(K, np.uint32))
        for k in range(K):
            lib_sel[0][int(ent_e[k])] = (float(row_w[k]), k)
        # rank order for a single token
        if 0 not in ties:
            assert np.array_equal(ent_e, idx_ref[0]), (ent_e, idx_ref[0])
    else:
        assert np.all(np.diff(ent_e) > 0), "entries in ascending expert order"
        assert np.array_equal(ent_row0, np.concatenate([[0], np.cumsum(ent_m)[:-1]]))
        assert int(ent_m.sum()) == TK
        for d in range(D):
            toks = [t for t in range(T) if (int(ent_mask[d]) >> t) & 1]
            assert len(toks) == ent_m[d]
            for j, t in enumerate(toks):
                lib_sel[t][int(ent_e[d])] = (float(row_w[ent_row0[d] + j]), int(ent_row0[d] + j))
    n_swapped = 0
    for t in range(T):
        want = {int(e): float(p_ref[t, k]) for k, e in enumerate(idx_ref[t])}
        if set(lib_sel[t]) != set(want):
            # only a near-tie token may take another set; it must be tie-equivalent
            assert t in ties, f"token {t}: selection differs without a near-tie"
            srt = np.sort(logits_ref[t])[::-1]
            for e in set(lib_sel[t]) ^ set(want):
                assert abs(logits_ref[t, e] - srt[K - 1]) < 1e-4
            n_swapped += 1
            sel = np.array(sorted(lib_sel[t], key=lambda e: -logits_ref[t, e]))
            z = np.exp(logits_ref[t, sel] - logits_ref[t, sel].max())
            want = dict(zip(sel.tolist(), (z / z.sum()).tolist()))
        werr = max(abs(lib_sel[t][e][0] - want[e]) for e in want)
        assert werr <= 5e-6, (t, werr)
    if Fs:
        sg_ref = O.shared_gate(xh, host["shared_gate_w"])
        assert np.abs(sgs.astype(np.float64) - sg_ref).max() <= 2e-6
    log(f"[dec-stages]   route record: {D} entries, near-ties {len(ties)}, rerouted {n_swapped}")
    a_all = ws[lay["a"]:lay["a"] + (TK * F + T * Fs) * 2].view(torch.int16).cpu().numpy()
    A = O.bf16_to_f64(a_all.view(np.uint16))
    a_rt = A[:TK * F].reshape(TK, F)
    a_ref = np.zeros_like(a_rt)
    used = np.zeros(TK, bool)
    for e in sorted({e for sel in lib_sel for e in sel}):
        toks = [t for t in range(T) if e in lib_sel[t]]
        rows = [lib_sel[t][e][1] for t in toks]
        wg, wu = _deq(host, "gate", e), _deq(host, "up", e)
        a_ref[rows] = O.round_to_bf16(O.silu(xf[toks] @ wg.T) * (xf[toks] @ wu.T))
        used[rows] = True
    assert used.all()
    check_a(a_rt, a_ref, "routed A (phase 1)")

    # ---- phase 2: down projection + weighted combine, from the library's own A and weights
    M.moe_layer_forward_phase(layer, x, out, ws, 2)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    ref = np.zeros((T, H))
    for e in sorted({e for sel in lib_sel for e in sel}):
        wd = _deq(host, "down", e)
        for t in range(T):
            if e in lib_sel[t]:
                w, r = lib_sel[t][e]
                ref[t] += w * (a_rt[r] @ wd.T)
    if Fs:
        wd = _deq(host, "sh_down", 0)
        ref += sgs.astype(np.float64)[:, None] * (A[TK * F:].reshape(T, Fs) @ wd.T)
    st = O.error_stats(y, ref)
    log(f"[dec-stages]   down + combine vs fp64 of the library's A: {st}")
    assert np.all(np.isfinite(y)) and st["max_rel"] < 1e-5
