"""Each C-ABI stage on its own: moe_grouped_gemm_w4 (gate/up + SwiGLU, down, down with the
deterministic or the atomic combine) and moe_combine, against fp64 evaluations of the same
definitions on the stage's own inputs."""
import numpy as np
import pytest

from gpu_common import DEV, device_layer, host_layer, log, tokens, u16
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def pipeline(name, T):
    """Route + permute on the GPU; returns everything the GEMM stages need."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer(name)
    xh, x = tokens(name, T, stream=3)
    K = layer.K
    idx = torch.empty(T * K, dtype=torch.int32, device=DEV)
    w = torch.empty(T * K, dtype=torch.float32, device=DEV)
    sg = torch.empty(T, dtype=torch.float32, device=DEV)
    cnt = torch.empty(layer.E, dtype=torch.int32, device=DEV)
    ws = M.alloc_workspace(layer, T)
    M.moe_route(layer, x, idx, w, sg, cnt, ws)
    plan = M.alloc_plan(layer, T)
    M.moe_permute(layer, idx, T, plan, ws)
    return layer, xh, x, idx, w, sg, plan, ws


def deq(host, name, e):
    q, s, b = host[name]
    return O.dequant(q[e], s[e], b[e], "bf16")


@pytest.mark.parametrize("name,T", [("odd", 130), ("mid", 300), ("tiny", 37), ("mid", 13), ("full", 8)])
def test_grouped_gemm_stages(name, T):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    log(f"[stages] {name} T={T}")
    layer, xh, x, idx, w, sg, plan, ws = pipeline(name, T)
    host = host_layer(name)
    H, E, K, F, Fs = layer.H, layer.E, layer.K, layer.F, layer.Fs
    TK = T * K
    a = torch.empty(TK * F + T * Fs, dtype=torch.int16, device=DEV)
    M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_GATE_UP, x, T, plan, None, None, a, ws)
    y = torch.empty((TK + T) * H, dtype=torch.float32, device=DEV)  # fp32 expert outputs
    M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_DOWN, a, T, plan, None, None, y, ws)
    out_c = torch.empty(T * H, dtype=torch.float32, device=DEV)
    M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_DOWN_COMBINE, a, T, plan, w, sg, out_c, ws)
    out_a = torch.empty(T * H, dtype=torch.float32, device=DEV)
    M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_DOWN_COMBINE_ATOMIC, a, T, plan, w, sg, out_a, ws)
    out_m = torch.empty(T * H, dtype=torch.float32, device=DEV)
    M.moe_combine(layer, y, plan["slot_pos"], w, y[TK * H:] if Fs else None, sg, T, out_m)
    torch.cuda.synchronize()

    xf = O.bf16_to_f64(xh)
    sorted_slots = plan["sorted_slots"].cpu().numpy()[:TK]
    offsets = plan["offsets"].cpu().numpy()
    A = O.bf16_to_f64(u16(a))
    Y = y.cpu().numpy().astype(np.float64).reshape(TK + T, H)
    # gate/up + SwiGLU, per grouped row; then down on the library's own A
    a_ref = np.empty_like(A)
    y_ref = np.empty((TK + T, H))
    for e in range(E + (1 if Fs else 0)):
        if e < E:
            rows = np.arange(offsets[e], offsets[e + 1])
            toks = sorted_slots[rows] // K
            names, n, base = ("gate", "up", "down"), F, 0
        else:
            rows, toks, names, n, base = np.arange(T), np.arange(T), ("sh_gate", "sh_up", "sh_down"), Fs, TK * F
        if rows.size == 0:
            continue
        ee = e if e < E else 0
        wg, wu, wd = (deq(host, nm, ee) for nm in names)
        g, u = xf[toks] @ wg.T, xf[toks] @ wu.T
        ar = O.round_to_bf16(O.silu(g) * u)
        if e < E:
            a_ref[rows[:, None] * F + np.arange(F)] = ar
            a_rows = A[rows[:, None] * F + np.arange(F)]
            y_ref[rows] = a_rows @ wd.T
        else:
            a_ref[base + rows[:, None] * Fs + np.arange(Fs)] = ar
            a_rows = A[base + rows[:, None] * Fs + np.arange(Fs)]
            y_ref[TK + rows] = a_rows @ wd.T
    check_a(A, a_ref, "A")
    # Y is the fp32-accumulated down product of the library's own A: within the fp32
    # accumulation error of the exact product (relative to the row's scale)
    st = O.error_stats(Y, y_ref)
    log(f"[stages]   Y vs exact product of the library's A: {st}")
    assert st["max_rel"] < 1e-5
    # combine from the library's weights and its own fp32 Y; every path sums fp32 terms
    wh = w.cpu().numpy().reshape(T, K)
    sgh = sg.cpu().numpy()
    slot_pos = plan["slot_pos"].cpu().numpy()[:TK].reshape(T, K)
    comb = np.einsum("tk,tkh->th", wh.astype(np.float64), Y[slot_pos])
    if Fs:
        comb += sgh[:, None] * Y[TK:]
    for tag, o in (("deterministic", out_c), ("atomic", out_a), ("moe_combine", out_m)):
        st = O.error_stats(o.cpu().numpy().reshape(T, H), comb)
        log(f"[stages]   combine {tag}: {st}")
        assert st["max_rel"] < 1e-5


def check_a(A, a_ref, what):
    """A is the bf16 rounding of silu(G)*U; G and U carry fp32 accumulation error, so a value
    may round to the neighbouring bf16 (one ulp, 2^-7 relative at most), and values that nearly
    cancel may differ by the accumulation error itself (bounded via the row scale)."""
    mism = np.mean(A != a_ref)
    scale = np.abs(a_ref).max()
    excess = np.abs(A - a_ref) - (2.0 ** -7 * np.abs(a_ref) + 1e-5 * scale)
    log(f"[stages]   {what}: {mism:.2e} of values differ from RNE(exact), worst excess {excess.max():.2e}")
    assert mism < 5e-3 and excess.max() <= 0


def test_combine_entry_point():
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer("mid")
    T, K, H = 77, layer.K, layer.H
    rng = np.random.default_rng(0)
    y_perm = rng.normal(size=(T * K, H)).astype(np.float32)   # fp32 expert outputs
    sh_y = rng.normal(size=(T, H)).astype(np.float32)
    wts = rng.random((T, K)).astype(np.float32)
    sgt = rng.random(T).astype(np.float32)
    slot_pos = rng.permutation(T * K).astype(np.int32)
    d = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    out = torch.empty(T * H, dtype=torch.float32, device=DEV)
    M.moe_combine(layer, d(y_perm), d(slot_pos), d(wts), d(sh_y), d(sgt), T, out)
    torch.cuda.synchronize()
    ref = np.einsum("tk,tkh->th", wts.astype(np.float64),
                    y_perm.astype(np.float64)[slot_pos.reshape(T, K)]) + sgt[:, None] * sh_y
    assert O.error_stats(out.cpu().numpy().reshape(T, H), ref)["max_rel"] < 1e-6
