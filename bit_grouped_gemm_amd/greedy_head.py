"""ctypes binding of the greedy decode step (include/greedy_head.h) in libmoe_w4.so.

Argument marshalling only: torch tensors supply device memory and the HIP stream; the LM head,
the argmax and the embedding run in the library's HIP kernels. Loading fails loudly if the
library is not built.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from .moe_w4 import W4, _check, _p, _stream, lib

EXPORTS = ("moe_greedy_workspace_bytes", "moe_greedy_next_input")


def _lib():
    L = lib()
    if not getattr(L, "_greedy_types", False):
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pw = ctypes.POINTER(W4)
        L.moe_greedy_workspace_bytes.restype = sz
        L.moe_greedy_workspace_bytes.argtypes = [i32, i32]
        L.moe_greedy_next_input.restype = ctypes.c_int
        L.moe_greedy_next_input.argtypes = [pw, pw, i32, i32, vp, i32, vp, vp, vp, sz, vp]
        L._greedy_types = True
    return L


@dataclass
class DeviceHead:
    """LM head and embedding on the device (tensors kept alive here) with their descriptors."""
    V: int
    H: int
    tensors: dict
    head: W4
    embed: W4


def upload_head(host: dict, device="cuda") -> DeviceHead:
    """host: {"head": (q, scale, bias), "embed": (q, scale, bias)} in the 4-bit storage format
    (q [1, V, H/8] uint32, scale / bias [1, V, H/64] bf16 bits)."""
    import torch

    def dev(a, view):
        return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(device)

    t = {}
    for name in ("head", "embed"):
        q, s, b = host[name]
        t[name] = (dev(q, np.int32), dev(s, np.int16), dev(b, np.int16))
    V, H = host["head"][0].shape[1], host["head"][0].shape[2] * 8
    w = {n: W4(t[n][0].data_ptr(), t[n][1].data_ptr(), t[n][2].data_ptr()) for n in t}
    return DeviceHead(V, H, t, w["head"], w["embed"])


def workspace_bytes(V: int, T: int) -> int:
    return _lib().moe_greedy_workspace_bytes(V, T)


def alloc_workspace(V: int, T: int, device="cuda"):
    import torch
    return torch.empty(max(workspace_bytes(V, T), 256), dtype=torch.uint8, device=device)


def next_input(hd: DeviceHead, x, token, x_next, workspace, stream=None):
    """x [T, H] bf16 (int16 tensor) -> token [T] int32, x_next [T, H] bf16 (may be x)."""
    T = x.shape[0]
    _check(_lib().moe_greedy_next_input(ctypes.byref(hd.head), ctypes.byref(hd.embed), hd.V, hd.H,
                                        _p(x), T, _p(token), _p(x_next), _p(workspace),
                                        workspace.numel(), _stream(stream)), "moe_greedy_next_input")


def logits_of(workspace, V: int, T: int):
    """The fp32 logits [T, V] a call left at the start of its workspace."""
    import torch
    return workspace[:T * V * 4].view(torch.float32).reshape(T, V)
