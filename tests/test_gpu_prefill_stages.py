"""The prefill path's grouped GEMMs checked row by row at the full layer size.

The layer runs through moe_layer_forward (default flags: the deterministic combine), which
leaves in the workspace (located through the test export moe_debug_workspace_layout) the
routing plan, the SwiGLU activations A of every grouped row and the fp32 expert outputs Y.
Every row is checked:

  A (gate/up GEMM + SwiGLU): against RNE(oracle silu(x Wg^T) * (x Wu^T)) of the row's token
      and expert, with the oracle's bf16-rounded weights;
  Y (down GEMM): against the fp64 product of the library's own A row with the oracle's
      bf16-rounded down weights;
  out (combine): against the fp64 weighted sum of the library's own Y rows.

T = 512 runs the small-batch kernels (pieces of at most 64 / 32 rows), T = 4096 the large ones
(256-row blocks); skewed routing gives full 256-row blocks and many empty experts
([P1 "How It Works ..."]: the 4-bit weights are rebuilt inside the grouped GEMM).
"""
import functools

import numpy as np
import pytest

from gpu_common import DEV, device_layer, host_layer, log, tokens
from oracle import moe_oracle as O
from test_gpu_stages import check_a

pytestmark = pytest.mark.gpu

ATOMIC = 1


@functools.lru_cache(maxsize=None)
def _deq32(proj, e):
    """bf16-rounded dequantised weights of the full-size layer, stored as fp32 (exact)."""
    q, s, b = host_layer("full")[proj]
    return O.dequant(q[e], s[e], b[e], "bf16").astype(np.float32)


def _w(proj, e):
    return _deq32(proj, e).astype(np.float64)


FORCE = 2


@pytest.mark.parametrize("name,T", [("full_skew", 512), ("full", 512), ("full", 4096),
                                    ("full_skew", 4096), ("full", 8), ("full", 64)])
def test_prefill_gemms_every_row(name, T):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    flags = FORCE if T <= 16 else 0   # small T: the MFMA path forced
    log(f"[pre-stages] {name} T={T} flags={flags}")
    layer = device_layer(name)
    H, E, K, F, Fs = layer.H, layer.E, layer.K, layer.F, layer.Fs
    TK = T * K
    xh, x = tokens(name, T, stream=40)
    lay = M.moe_debug_workspace_layout(layer, T, flags)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_layer_forward(layer, x, out, ws, flags)
    torch.cuda.synchronize()

    def region(key, n, dtype):
        return ws[lay[key]:lay[key] + n * np.dtype(dtype).itemsize].cpu().numpy().view(dtype)

    offsets = region("offsets", E + 1, np.int32)
    sorted_slots = region("sorted_slots", TK, np.int32)
    slot_pos = region("slot_pos", TK, np.int32)
    topk_w = region("topk_w", TK, np.float32).astype(np.float64).reshape(T, K)
    sgate = region("sgate", T, np.float32).astype(np.float64)
    nblk = int(region("num_blocks", 1, np.int32)[0])
    blocks = region("blocks", 4 * nblk, np.int32).reshape(nblk, 4)
    A = O.bf16_to_f64(region("a", TK * F + T * Fs, np.uint16))
    Y = region("y", (TK + T) * H, np.float32).astype(np.float64).reshape(TK + T, H)
    counts = np.diff(offsets)
    # the prefill router and top-k: indices as the oracle's (near-tie tokens: a tie-equivalent
    # set), weights and shared gates to fp32 accuracy
    host = host_layer(name)
    idx = region("topk_idx", TK, np.int32).reshape(T, K)
    logits = O.router_logits(xh, host["router_w"], host["router_bias"])
    ridx, rp = O.select_topk(logits, K)
    ties = set(O.near_ties(logits, K).tolist())
    same = np.all(idx == ridx, axis=1)
    assert all(t in ties for t in np.nonzero(~same)[0]), "selection differs without a near-tie"
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    werr = np.abs(topk_w - z / z.sum(axis=1, keepdims=True)).max()
    gerr = np.abs(sgate - O.shared_gate(xh, host["shared_gate_w"])).max()
    log(f"[pre-stages]   router: {int((~same).sum())} tokens rerouted ({len(ties)} near-ties), "
        f"weights max abs error {werr:.2e}, shared gate {gerr:.2e}")
    assert werr <= 5e-6 and gerr <= 2e-6
    tall = int((blocks[:, 2] == M.MOE_BLOCK_M).sum())
    log(f"[pre-stages]   {nblk} blocks ({tall} of {M.MOE_BLOCK_M} rows), "
        f"{int((counts == 0).sum())} empty experts, max {counts.max()} rows")
    if name == "full_skew":
        assert tall > 0, "skewed routing gives full 256-row blocks"

    xf = O.bf16_to_f64(xh)
    a_rt = A[:TK * F].reshape(TK, F)
    a_sh = A[TK * F:].reshape(T, Fs)
    a_ref = np.empty_like(a_rt)
    y_ref = np.empty_like(Y)
    for e in np.nonzero(counts)[0]:
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = sorted_slots[rows] // K
        a_ref[rows] = O.round_to_bf16(O.silu(xf[toks] @ _w("gate", e).T) * (xf[toks] @ _w("up", e).T))
        y_ref[rows] = a_rt[rows] @ _w("down", e).T
    wg, wu, wd = (_w(n, 0) for n in ("sh_gate", "sh_up", "sh_down"))
    a_sh_ref = O.round_to_bf16(O.silu(xf @ wg.T) * (xf @ wu.T))
    y_ref[TK:] = a_sh @ wd.T
    check_a(a_rt, a_ref, "routed A, every row")
    check_a(a_sh, a_sh_ref, "shared A, every row")
    st = O.error_stats(Y, y_ref)
    log(f"[pre-stages]   Y (every row) vs fp64 product of the library's A: {st}")
    assert st["max_rel"] < 1e-5
    comb = np.einsum("tk,tkh->th", topk_w, Y[slot_pos.reshape(T, K)]) + sgate[:, None] * Y[TK:]
    st = O.error_stats(out.cpu().numpy(), comb)
    log(f"[pre-stages]   combine vs fp64 sum of the library's Y: {st}")
    assert st["max_rel"] < 1e-5

    # the atomic combine on the same plan: the same output within fp32 summation noise
    ws0 = M.alloc_workspace(layer, T, ATOMIC | flags)
    out0 = torch.empty_like(out)
    M.moe_layer_forward(layer, x, out0, ws0, ATOMIC | flags)
    torch.cuda.synchronize()
    st = O.error_stats(out0.cpu().numpy(), comb)
    log(f"[pre-stages]   atomic combine vs fp64 sum of the library's Y: {st}")
    assert st["max_rel"] < 1e-5
