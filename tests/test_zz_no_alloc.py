"""moe_layer_forward_noalloc (no workspace argument; the library's per-GPU scratch array)
against moe_layer_forward on the same inputs: two calls in a row, the second with a smaller
input, each bit-identical to the workspace entry point (both paths are deterministic), and a
size beyond the array rejected on the host."""
import ctypes

import numpy as np
import pytest

from gpu_common import DEV, device_layer, log, tokens

pytestmark = pytest.mark.gpu


def _ref(layer, x, flags=0):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    ws = M.alloc_workspace(layer, x.shape[0], flags)
    out = torch.full((x.shape[0], layer.H), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_layer_forward(layer, x, out, ws, flags)
    return out


@pytest.mark.parametrize("name,T1,T2", [("full", 300, 5), ("mid", 130, 1)])
def test_noalloc_matches_workspace_entry_point(name, T1, T2):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer(name)
    outs = []
    for i, T in enumerate((T1, T2)):   # two calls in a row, the second smaller
        log(f"[noalloc] {name} call {i} T={T}")
        _, x = tokens(name, T, stream=80 + i)
        need = M.moe_workspace_bytes(layer, T)
        assert need <= M.NOALLOC_SCRATCH_BYTES
        out = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=DEV)
        M.moe_layer_forward_noalloc(layer, x, out)
        outs.append((out, x))
    torch.cuda.synchronize()
    for out, x in outs:
        ref = _ref(layer, x)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all().item()
        assert torch.equal(out, ref), float((out - ref).abs().max())


def test_noalloc_rejects_sizes_beyond_the_array():
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    layer = device_layer("full")
    T = 4096   # needs about 357 MiB with the deterministic combine
    assert M.moe_workspace_bytes(layer, T) > M.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, layer.H), dtype=torch.int16, device=DEV)
    out = torch.zeros((T, layer.H), dtype=torch.float32, device=DEV)
    st = M.lib().moe_layer_forward_noalloc(layer.desc_ptr, ctypes.c_void_p(x.data_ptr()), T,
                                           ctypes.c_void_p(out.data_ptr()), 0, None)
    assert st == M.MOE_WORKSPACE_TOO_SMALL
    assert M.lib().moe_layer_forward_noalloc(layer.desc_ptr, None, 0, None, 0, None) == M.MOE_OK
