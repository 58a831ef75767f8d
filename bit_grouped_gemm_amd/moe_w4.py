"""ctypes binding of libmoe_w4.so (the C ABI in include/moe_w4.h).

Argument marshalling only: torch tensors supply device memory and the HIP stream; every step
of the layer runs in the library's HIP kernels. The library must be built
(bit_grouped_gemm_amd.build); loading fails loudly otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4.so")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_WORKSPACE_TOO_SMALL, MOE_HIP_ERROR = range(5)
MOE_BLOCK_M = 256
MOE_GEMM_GATE_UP, MOE_GEMM_DOWN, MOE_GEMM_DOWN_COMBINE, MOE_GEMM_DOWN_COMBINE_ATOMIC = range(4)
MOE_FLAG_ATOMIC_COMBINE = 1
MOE_FLAG_FORCE_PREFILL = 2
DECODE_MAX_T = 16

EXPORTS = ("moe_status_str", "moe_version", "moe_workspace_bytes", "moe_plan_max_blocks",
           "moe_route", "moe_permute", "moe_grouped_gemm_w4", "moe_combine",
           "moe_layer_forward", "moe_debug_dequant_w4", "moe_layer_num_phases",
           "moe_layer_forward_phase", "moe_residual_rmsnorm", "moe_stack_workspace_bytes",
           "moe_stack_forward", "moe_debug_workspace_layout", "moe_bench_mfma_loop",
           "moe_bench_stream_read", "moe_layer_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20


class W4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ffn", ctypes.c_int32), ("shared_ffn", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("renormalize", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", W4), ("up", W4), ("down", W4),
                ("sh_gate", W4), ("sh_up", W4), ("sh_down", W4),
                ("shared_gate_w", ctypes.c_void_p)]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "offsets", "sorted_slots", "slot_pos", "blocks", "num_blocks")]


_lib = None


def lib():
    """Load libmoe_w4.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_grouped_gemm_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pdesc = ctypes.POINTER(LayerDesc)
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_version.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_workspace_bytes.restype = sz
    L.moe_workspace_bytes.argtypes = [pdesc, i32, i32]
    L.moe_plan_max_blocks.restype = i32
    L.moe_plan_max_blocks.argtypes = [pdesc, i32]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [pdesc, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_permute.restype = ctypes.c_int
    L.moe_permute.argtypes = [pdesc, vp, i32, ctypes.POINTER(Plan), vp, sz, vp]
    L.moe_grouped_gemm_w4.restype = ctypes.c_int
    L.moe_grouped_gemm_w4.argtypes = [pdesc, i32, vp, i32, ctypes.POINTER(Plan), vp, vp, vp, vp,
                                      sz, vp]
    L.moe_combine.restype = ctypes.c_int
    L.moe_combine.argtypes = [pdesc, vp, vp, vp, vp, vp, i32, vp, vp]
    L.moe_layer_forward.restype = ctypes.c_int
    L.moe_layer_forward.argtypes = [pdesc, vp, i32, vp, vp, sz, i32, vp]
    L.moe_layer_forward_noalloc.restype = ctypes.c_int
    L.moe_layer_forward_noalloc.argtypes = [pdesc, vp, i32, vp, i32, vp]
    L.moe_layer_num_phases.restype = i32
    L.moe_layer_num_phases.argtypes = [pdesc, i32, i32]
    L.moe_layer_forward_phase.restype = ctypes.c_int
    L.moe_layer_forward_phase.argtypes = [pdesc, vp, i32, vp, vp, sz, i32, i32, vp]
    L.moe_residual_rmsnorm.restype = ctypes.c_int
    L.moe_residual_rmsnorm.argtypes = [vp, vp, vp, i32, i32, ctypes.c_float, i32, vp]
    ppdesc = ctypes.POINTER(pdesc)
    L.moe_stack_workspace_bytes.restype = sz
    L.moe_stack_workspace_bytes.argtypes = [ppdesc, i32, i32, i32]
    L.moe_stack_forward.restype = ctypes.c_int
    L.moe_stack_forward.argtypes = [ppdesc, i32, vp, vp, i32, ctypes.c_float, vp, sz, i32, vp]
    L.moe_debug_dequant_w4.restype = ctypes.c_int
    L.moe_debug_dequant_w4.argtypes = [ctypes.POINTER(W4), i32, i32, i32, i32, vp, vp, vp]
    L.moe_bench_mfma_loop.restype = ctypes.c_int
    L.moe_bench_mfma_loop.argtypes = [i32, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.moe_bench_stream_read.restype = ctypes.c_int
    L.moe_bench_stream_read.argtypes = [vp, sz, i32, vp, vp]
    L.moe_debug_workspace_layout.restype = ctypes.c_int
    L.moe_debug_workspace_layout.argtypes = [pdesc, i32, i32, ctypes.POINTER(sz), i32]
    _lib = L
    return L


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().moe_status_str(status).decode()} (status {status})")


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoEError(status, what)


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ device-resident layer
@dataclass
class DeviceLayer:
    """A layer's tensors on the device plus its C descriptor (tensors are kept alive here)."""
    H: int
    E: int
    K: int
    F: int
    Fs: int
    tensors: dict
    desc: LayerDesc

    @property
    def desc_ptr(self):
        return ctypes.byref(self.desc)


def _w4(tensors, name):
    if name not in tensors:
        return W4(None, None, None)
    q, s, b = tensors[name]
    return W4(q.data_ptr(), s.data_ptr(), b.data_ptr())


def upload_layer(host: dict, H: int, E: int, K: int, F: int, Fs: int, device="cuda") -> DeviceLayer:
    """Copy a host layer (numpy arrays in the storage formats of include/moe_w4.h) to the device."""
    import torch

    def dev(a, view):
        return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(device)

    t = {"router_w": dev(host["router_w"].astype(np.float32), np.float32),
         "shared_gate_w": dev(host["shared_gate_w"].astype(np.float32), np.float32)}
    if host.get("router_bias") is not None:
        t["router_bias"] = dev(host["router_bias"].astype(np.float32), np.float32)
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        if host.get(name) is not None:
            q, s, b = host[name]
            t[name] = (dev(q, np.int32), dev(s, np.int16), dev(b, np.int16))
    return make_layer(t, H, E, K, F, Fs)


def make_layer(t: dict, H: int, E: int, K: int, F: int, Fs: int) -> DeviceLayer:
    desc = LayerDesc(hidden=H, num_experts=E, top_k=K, ffn=F, shared_ffn=Fs, bits=4, group_size=64,
                     renormalize=1,
                     router_w=t["router_w"].data_ptr(),
                     router_bias=t["router_bias"].data_ptr() if "router_bias" in t else None,
                     gate=_w4(t, "gate"), up=_w4(t, "up"), down=_w4(t, "down"),
                     sh_gate=_w4(t, "sh_gate"), sh_up=_w4(t, "sh_up"), sh_down=_w4(t, "sh_down"),
                     shared_gate_w=t["shared_gate_w"].data_ptr() if Fs > 0 else None)
    return DeviceLayer(H, E, K, F, Fs, t, desc)


# ------------------------------------------------------------------------ entry points
def moe_version() -> str:
    return lib().moe_version().decode()


def moe_workspace_bytes(layer: DeviceLayer, T_max: int, flags: int = 0) -> int:
    n = lib().moe_workspace_bytes(layer.desc_ptr, T_max, flags)
    if n == 0 and T_max >= 0:
        raise MoEError(MOE_UNSUPPORTED, "moe_workspace_bytes")
    return n


def moe_plan_max_blocks(layer: DeviceLayer, T: int) -> int:
    return lib().moe_plan_max_blocks(layer.desc_ptr, T)


def alloc_workspace(layer: DeviceLayer, T_max: int, flags: int = 0, device="cuda"):
    import torch
    return torch.empty(moe_workspace_bytes(layer, T_max, flags), dtype=torch.uint8, device=device)


def alloc_plan(layer: DeviceLayer, T: int, device="cuda") -> dict:
    import torch
    i32 = dict(dtype=torch.int32, device=device)
    TK = T * layer.K
    return {"counts": torch.empty(layer.E, **i32), "offsets": torch.empty(layer.E + 1, **i32),
            "sorted_slots": torch.empty(max(TK, 1), **i32), "slot_pos": torch.empty(max(TK, 1), **i32),
            "blocks": torch.empty(max(moe_plan_max_blocks(layer, T), 1) * 4, **i32),
            "num_blocks": torch.empty(1, **i32)}


def _plan_struct(plan: dict) -> Plan:
    return Plan(*(plan[n].data_ptr() for n in
                  ("counts", "offsets", "sorted_slots", "slot_pos", "blocks", "num_blocks")))


def moe_route(layer, x, topk_idx, topk_w, shared_gate, counts, workspace, stream=None):
    T = x.shape[0]
    _check(lib().moe_route(layer.desc_ptr, _p(x), T, _p(topk_idx), _p(topk_w), _p(shared_gate),
                           _p(counts), _p(workspace), workspace.numel(), _stream(stream)),
           "moe_route")


def moe_permute(layer, topk_idx, T, plan: dict, workspace, stream=None):
    ps = _plan_struct(plan)
    _check(lib().moe_permute(layer.desc_ptr, _p(topk_idx), T, ctypes.byref(ps), _p(workspace),
                             workspace.numel(), _stream(stream)), "moe_permute")


def moe_grouped_gemm_w4(layer, which, inp, T, plan: dict, topk_w, shared_gate, out, workspace,
                        stream=None):
    ps = _plan_struct(plan)
    _check(lib().moe_grouped_gemm_w4(layer.desc_ptr, which, _p(inp), T, ctypes.byref(ps),
                                     _p(topk_w), _p(shared_gate), _p(out), _p(workspace),
                                     0 if workspace is None else workspace.numel(),
                                     _stream(stream)), "moe_grouped_gemm_w4")


def moe_combine(layer, y_perm, slot_pos, topk_w, shared_y, shared_gate, T, out, stream=None):
    _check(lib().moe_combine(layer.desc_ptr, _p(y_perm), _p(slot_pos), _p(topk_w), _p(shared_y),
                             _p(shared_gate), T, _p(out), _stream(stream)), "moe_combine")


def moe_layer_forward(layer, x, out, workspace, flags: int = 0, stream=None):
    _check(lib().moe_layer_forward(layer.desc_ptr, _p(x), x.shape[0], _p(out), _p(workspace),
                                   workspace.numel(), flags, _stream(stream)), "moe_layer_forward")


def moe_layer_forward_noalloc(layer, x, out, flags: int = 0, stream=None):
    """moe_layer_forward with the library's own per-GPU scratch array (no workspace argument)."""
    _check(lib().moe_layer_forward_noalloc(layer.desc_ptr, _p(x), x.shape[0], _p(out), flags,
                                           _stream(stream)), "moe_layer_forward_noalloc")


def moe_debug_dequant_w4(w4: tuple, n_rows: int, kin: int, mat: int, row: int, out_f32=None,
                         out_bf16=None, stream=None):
    q, s, b = w4
    st = W4(q.data_ptr(), s.data_ptr(), b.data_ptr())
    _check(lib().moe_debug_dequant_w4(ctypes.byref(st), n_rows, kin, mat, row, _p(out_f32),
                                      _p(out_bf16), _stream(stream)), "moe_debug_dequant_w4")


WS_REGIONS = ("logits", "topk_idx", "topk_w", "sgate", "route", "counts", "offsets",
              "sorted_slots", "slot_pos", "blocks", "num_blocks", "a", "y", "total")


def moe_debug_workspace_layout(layer, T: int, flags: int = 0) -> dict:
    """Byte offsets of the workspace regions (test export), keyed by WS_REGIONS."""
    arr = (ctypes.c_size_t * len(WS_REGIONS))()
    _check(lib().moe_debug_workspace_layout(layer.desc_ptr, T, flags, arr, len(WS_REGIONS)),
           "moe_debug_workspace_layout")
    return dict(zip(WS_REGIONS, (int(v) for v in arr)))


def moe_bench_mfma_loop(workgroups: int, iters: int, sink, stream=None) -> float:
    """Enqueue the MFMA-loop measurement kernel; returns the flops it performs."""
    fl = ctypes.c_double(0.0)
    _check(lib().moe_bench_mfma_loop(workgroups, iters, _p(sink), ctypes.byref(fl),
                                     _stream(stream)), "moe_bench_mfma_loop")
    return fl.value


def moe_bench_stream_read(buf, workgroups: int, sink, stream=None):
    """Enqueue the streaming-read measurement kernel over the whole of buf."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().moe_bench_stream_read(_p(buf), nbytes, workgroups, _p(sink), _stream(stream)),
           "moe_bench_stream_read")


def moe_layer_num_phases(layer, T: int, flags: int = 0) -> int:
    return lib().moe_layer_num_phases(layer.desc_ptr, T, flags)


def moe_layer_forward_phase(layer, x, out, workspace, phase: int, flags: int = 0, stream=None):
    _check(lib().moe_layer_forward_phase(layer.desc_ptr, _p(x), x.shape[0], _p(out), _p(workspace),
                                         workspace.numel(), flags, phase, _stream(stream)),
           "moe_layer_forward_phase")


RMS_EPS = 1e-6


def moe_residual_rmsnorm(y, resid, x, init: bool = False, eps: float = RMS_EPS, stream=None):
    T, H = resid.shape
    _check(lib().moe_residual_rmsnorm(_p(y), _p(resid), _p(x), T, H, eps, 1 if init else 0,
                                      _stream(stream)), "moe_residual_rmsnorm")


class Stack:
    """A stack of device layers for moe_stack_forward (keeps the descriptor array alive)."""

    def __init__(self, layers):
        self.layers = list(layers)
        arr = (ctypes.POINTER(LayerDesc) * len(self.layers))()
        for i, l in enumerate(self.layers):
            arr[i] = ctypes.pointer(l.desc)
        self._arr = arr

    def workspace_bytes(self, T_max: int, flags: int = 0) -> int:
        n = lib().moe_stack_workspace_bytes(self._arr, len(self.layers), T_max, flags)
        if n == 0:
            raise MoEError(MOE_UNSUPPORTED, "moe_stack_workspace_bytes")
        return n

    def alloc_workspace(self, T_max: int, flags: int = 0, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(T_max, flags), dtype=torch.uint8, device=device)

    def forward(self, resid, x, workspace, flags: int = 0, eps: float = RMS_EPS, stream=None):
        _check(lib().moe_stack_forward(self._arr, len(self.layers), _p(resid), _p(x), x.shape[0],
                                       eps, _p(workspace), workspace.numel(), flags,
                                       _stream(stream)), "moe_stack_forward")
