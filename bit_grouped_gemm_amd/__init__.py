"""MI355X (gfx950) MoE layer with 4-bit group-64 affine experts: HIP kernels behind a C ABI.

The compute lives in libmoe_w4.so (bit_grouped_gemm_amd/csrc, declared in include/moe_w4.h);
moe_w4 is its ctypes binding.
"""
from . import moe_w4  # noqa: F401
from .moe_w4 import (  # noqa: F401
    DeviceLayer, upload_layer, make_layer, alloc_workspace, alloc_plan, moe_version,
    moe_workspace_bytes, moe_plan_max_blocks, moe_route, moe_permute, moe_grouped_gemm_w4,
    moe_combine, moe_layer_forward, moe_debug_dequant_w4,
)
