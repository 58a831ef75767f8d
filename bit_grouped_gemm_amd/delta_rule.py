"""ctypes binding of the gated delta-rule recurrence (include/delta_rule.h) in libmoe_w4.so.

Argument marshalling only: torch tensors supply device memory and the HIP stream; the work
runs in the library's HIP kernel. Loading fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import math

from .moe_w4 import _check, _p, _stream, lib

EXPORTS = ("delta_rule_forward", "delta_rule_chunked_workspace_bytes", "delta_rule_forward_chunked")


class DeltaDesc(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("scale", ctypes.c_float),
                ("eps", ctypes.c_float)]


def desc(num_k_heads, num_v_heads, dk, dv, scale=None, eps=1e-6) -> DeltaDesc:
    return DeltaDesc(num_k_heads, num_v_heads, dk, dv,
                     1.0 / math.sqrt(dk) if scale is None else scale, eps)


def _lib():
    L = lib()
    if not getattr(L, "_delta_types", False):
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.delta_rule_forward.restype = ctypes.c_int
        L.delta_rule_forward.argtypes = [ctypes.POINTER(DeltaDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                         i32, i32, vp]
        L.delta_rule_chunked_workspace_bytes.restype = ctypes.c_size_t
        L.delta_rule_chunked_workspace_bytes.argtypes = [ctypes.POINTER(DeltaDesc), i32, i32]
        L.delta_rule_forward_chunked.restype = ctypes.c_int
        L.delta_rule_forward_chunked.argtypes = [ctypes.POINTER(DeltaDesc), vp, vp, vp, vp, vp, vp,
                                                 vp, vp, i32, i32, vp, ctypes.c_size_t, vp]
        L._delta_types = True
    return L


def forward(d: DeltaDesc, q, k, v, g, beta, state_in, state_out, o, stream=None):
    """q, k [B,T,Hk,dk] and v [B,T,Hv,dv] bf16 (int16 tensors), g, beta [B,T,Hv] fp32,
    state_in (or None) / state_out [B,Hv,dv,dk] fp32, o [B,T,Hv,dv] fp32."""
    B, T = q.shape[0], q.shape[1]
    _check(_lib().delta_rule_forward(ctypes.byref(d), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                     _p(state_in), _p(state_out), _p(o), B, T, _stream(stream)),
           "delta_rule_forward")


def chunked_workspace_bytes(d: DeltaDesc, batch: int, T: int) -> int:
    return int(_lib().delta_rule_chunked_workspace_bytes(ctypes.byref(d), batch, T))


def alloc_chunked_workspace(d: DeltaDesc, batch: int, T: int, device="cuda"):
    import torch
    return torch.empty(max(16, chunked_workspace_bytes(d, batch, T)), dtype=torch.uint8, device=device)


def forward_chunked(d: DeltaDesc, q, k, v, g, beta, state_in, state_out, o, workspace, stream=None):
    """As forward(), over 32-token chunks, with a workspace from alloc_chunked_workspace."""
    B, T = q.shape[0], q.shape[1]
    _check(_lib().delta_rule_forward_chunked(ctypes.byref(d), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                             _p(state_in), _p(state_out), _p(o), B, T,
                                             _p(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)),
           "delta_rule_forward_chunked")
