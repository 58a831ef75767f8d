"""ctypes binding of the decode-attention entry points (include/attn_gqa.h) in libmoe_w4.so.

Argument marshalling only: torch tensors supply device memory and the HIP stream; the work
runs in the library's HIP kernels. Loading fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import math

from .moe_w4 import _check, _p, _stream, lib

ATTN_FLAG_UNPACKED = 1
EXPORTS = ("attn_gqa_decode_workspace_bytes", "attn_gqa_decode")


class AttnDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("scale", ctypes.c_float)]


def desc(num_q_heads, num_kv_heads, head_dim, block_size, scale=None) -> AttnDesc:
    return AttnDesc(num_q_heads, num_kv_heads, head_dim, block_size,
                    1.0 / math.sqrt(head_dim) if scale is None else scale)


def _lib():
    L = lib()
    if not getattr(L, "_attn_types", False):
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pd = ctypes.POINTER(AttnDesc)
        L.attn_gqa_decode_workspace_bytes.restype = sz
        L.attn_gqa_decode_workspace_bytes.argtypes = [pd, i32, i32]
        L.attn_gqa_decode.restype = ctypes.c_int
        L.attn_gqa_decode.argtypes = [pd, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, i32, vp, sz, vp]
        L._attn_types = True
    return L


def workspace_bytes(d: AttnDesc, batch: int, max_seq_len: int) -> int:
    return _lib().attn_gqa_decode_workspace_bytes(ctypes.byref(d), batch, max_seq_len)


def alloc_workspace(d: AttnDesc, batch: int, max_seq_len: int, device="cuda"):
    import torch
    return torch.empty(max(workspace_bytes(d, batch, max_seq_len), 256), dtype=torch.uint8,
                       device=device)


def decode(d: AttnDesc, q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, out,
           workspace, flags: int = 0, stream=None):
    """One decode step: q [B,Hq,D] bf16 (int16 tensor), caches [n_phys,Hkv,BS,D] bf16,
    block_table [B,MB] int32, seq_lens [B] int32 (device), out [B,Hq,D] fp32."""
    B = q.shape[0]
    _check(_lib().attn_gqa_decode(ctypes.byref(d), _p(q), _p(k_cache), _p(v_cache),
                                  k_cache.shape[0], _p(block_table), block_table.shape[1],
                                  _p(seq_lens), B, max_seq_len, _p(out), flags, _p(workspace),
                                  workspace.numel(), _stream(stream)), "attn_gqa_decode")
