"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and
rejects bad arguments on the host before any kernel is enqueued."""
import ctypes
import os
import re

import pytest

from bit_grouped_gemm_amd import moe_w4 as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


ATTN_HEADER = os.path.join(ROOT, "include", "attn_gqa.h")
DELTA_HEADER = os.path.join(ROOT, "include", "delta_rule.h")
GREEDY_HEADER = os.path.join(ROOT, "include", "greedy_head.h")


def declared_in(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**((?:moe|attn|delta)_\w+)\s*\(",
                                 text, flags=re.M)))


def test_every_header_is_exported():
    """Each header's declarations are exactly its binding's export list, and the library
    exports every one of them."""
    from bit_grouped_gemm_amd import attn_gqa, delta_rule, greedy_head
    lib = ctypes.CDLL(M.LIB_PATH)
    for path, exports in ((HEADER, M.EXPORTS), (ATTN_HEADER, attn_gqa.EXPORTS),
                          (DELTA_HEADER, delta_rule.EXPORTS), (GREEDY_HEADER, greedy_head.EXPORTS)):
        names = declared_in(path)
        assert set(names) == set(exports), path
        for n in names:
            assert hasattr(lib, n), n


def test_attention_rejections():
    from bit_grouped_gemm_amd import attn_gqa as G
    L = G._lib()
    ok = G.desc(16, 2, 128, 64)
    assert G.workspace_bytes(ok, 1, 32768) >= 16 * 128 * 4
    for bad in (G.desc(16, 2, 96, 64), G.desc(16, 3, 128, 64), G.desc(32, 2, 128, 64),
                G.desc(16, 2, 128, 48)):
        assert G.workspace_bytes(bad, 1, 100) == 0
        assert L.attn_gqa_decode(ctypes.byref(bad), FAKE, FAKE, FAKE, 4, FAKE, 4, FAKE, 1, 100,
                                 FAKE, 0, FAKE, 1 << 30, None) == M.MOE_UNSUPPORTED
    # the block table cannot hold max_seq_len tokens; a bad flag; a workspace too small
    assert L.attn_gqa_decode(ctypes.byref(ok), FAKE, FAKE, FAKE, 4, FAKE, 1, FAKE, 1, 65, FAKE, 0,
                             FAKE, 1 << 30, None) == M.MOE_INVALID_ARG
    assert L.attn_gqa_decode(ctypes.byref(ok), FAKE, FAKE, FAKE, 4, FAKE, 2, FAKE, 1, 65, FAKE, 2,
                             FAKE, 1 << 30, None) == M.MOE_INVALID_ARG
    assert L.attn_gqa_decode(ctypes.byref(ok), FAKE, FAKE, FAKE, 4, FAKE, 2, FAKE, 1, 65, FAKE, 0,
                             FAKE, 16, None) == M.MOE_WORKSPACE_TOO_SMALL
    assert L.attn_gqa_decode(ctypes.byref(ok), None, None, None, 0, None, 0, None, 0, 0, None, 0,
                             None, 0, None) == M.MOE_OK


def test_delta_rule_rejections():
    from bit_grouped_gemm_amd import delta_rule as DR
    L = DR._lib()
    call = lambda d, B=1, T=1, sin=FAKE: L.delta_rule_forward(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, sin, FAKE, FAKE, B, T, None)
    for bad in (DR.desc(16, 16, 96, 128), DR.desc(16, 24, 128, 128), DR.desc(16, 16, 128, 120)):
        assert call(bad) == M.MOE_UNSUPPORTED
    ok = DR.desc(16, 16, 128, 128)
    assert call(ok, T=-1) == M.MOE_INVALID_ARG
    assert call(ok, B=0) == M.MOE_OK
    assert call(DR.desc(16, 16, 128, 128, eps=-1.0)) == M.MOE_INVALID_ARG
    assert L.delta_rule_forward(ctypes.byref(ok), FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 1, 1, None) == M.MOE_INVALID_ARG   # misaligned q


def test_delta_rule_chunked_sizes_and_rejections():
    """Workspace sizes of the chunked entry point and the argument checks that return before
    any launch."""
    from bit_grouped_gemm_amd import delta_rule as DR
    L = DR._lib()
    ok = DR.desc(16, 16, 128, 128)
    # 16 chunks of 32 tokens x 16 heads, each record three 32 x dk matrices, two 32 x dv
    # matrices and 64 scalars, fp32
    rec = 3 * 32 * 128 + 2 * 32 * 128 + 64
    assert DR.chunked_workspace_bytes(ok, 1, 512) == 16 * 16 * rec * 4
    assert DR.chunked_workspace_bytes(ok, 2, 33) == 2 * 16 * 2 * rec * 4
    assert DR.chunked_workspace_bytes(DR.desc(2, 4, 256, 48), 1, 40) == 4 * 2 * (3 * 32 * 256 + 2 * 32 * 48 + 64) * 4
    assert DR.chunked_workspace_bytes(ok, 1, 0) == 0
    assert DR.chunked_workspace_bytes(DR.desc(16, 16, 96, 128), 1, 64) == 0
    call = lambda d, B=1, T=64, ws=FAKE, n=1 << 30: L.delta_rule_forward_chunked(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, T, ws, n, None)
    for bad in (DR.desc(16, 16, 96, 128), DR.desc(16, 24, 128, 128), DR.desc(16, 16, 128, 120)):
        assert call(bad) == M.MOE_UNSUPPORTED
    assert call(ok, T=-1) == M.MOE_INVALID_ARG
    assert call(ok, B=0) == M.MOE_OK
    assert call(ok, ws=None) == M.MOE_INVALID_ARG
    assert call(ok, ws=FAKE + 8) == M.MOE_INVALID_ARG
    assert call(ok, n=DR.chunked_workspace_bytes(ok, 1, 64) - 1) == M.MOE_WORKSPACE_TOO_SMALL


def test_header_declares_the_five_layer_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm_w4", "moe_combine", "moe_layer_forward"):
        assert n in names
    assert set(names) == set(M.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(M.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert "gfx950" in M.moe_version()
    L = M.lib()
    assert L.moe_status_str(M.MOE_OK) == b"ok"
    assert L.moe_status_str(M.MOE_WORKSPACE_TOO_SMALL) == b"workspace too small"
    assert L.moe_status_str(99) == b"unknown status"


FAKE = 0x10000  # an aligned non-null address; never dereferenced by the host checks below


def fake_desc(H=2048, E=256, K=8, F=512, Fs=512, **over):
    w = M.W4(FAKE, FAKE, FAKE)
    d = M.LayerDesc(hidden=H, num_experts=E, top_k=K, ffn=F, shared_ffn=Fs, bits=4, group_size=64,
                    renormalize=1, router_w=FAKE, router_bias=None, gate=w, up=w, down=w,
                    sh_gate=w, sh_up=w, sh_down=w, shared_gate_w=FAKE)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def ws_bytes(d, T, flags=0):
    return M.lib().moe_workspace_bytes(ctypes.byref(d), T, flags)


def forward(d, T, ws, flags=0, x=FAKE, out=FAKE):
    return M.lib().moe_layer_forward(ctypes.byref(d), x, T, out, FAKE, ws, flags, None)


def test_workspace_sizes():
    d = fake_desc()
    base = ws_bytes(d, 4096)
    atomic = ws_bytes(d, 4096, M.MOE_FLAG_ATOMIC_COMBINE)
    # the default (deterministic) combine stages fp32 expert outputs for T*K + T grouped rows;
    # the fused atomic combine needs none
    assert base - atomic >= (4096 * 8 + 4096) * 2048 * 4
    # unknown flag bits are rejected
    assert ws_bytes(d, 4096, 4) == 0 and ws_bytes(d, 4096, 8) == 0
    assert ws_bytes(d, 1) < ws_bytes(d, 8) < base
    assert M.lib().moe_plan_max_blocks(ctypes.byref(d), 4096) == 32768 // M.MOE_BLOCK_M + 256 + 4096 // M.MOE_BLOCK_M
    assert M.lib().moe_plan_max_blocks(ctypes.byref(d), 1) == 1 + 8 + 1


@pytest.mark.parametrize("field,value,status", [
    ("bits", 3, M.MOE_UNSUPPORTED), ("group_size", 32, M.MOE_UNSUPPORTED),
    ("renormalize", 0, M.MOE_UNSUPPORTED), ("hidden", 2000, M.MOE_UNSUPPORTED),
    ("ffn", 500, M.MOE_UNSUPPORTED), ("shared_ffn", 100, M.MOE_UNSUPPORTED),
    ("top_k", 300, M.MOE_UNSUPPORTED), ("num_experts", 2048, M.MOE_UNSUPPORTED),
    ("top_k", 0, M.MOE_INVALID_ARG), ("hidden", -64, M.MOE_INVALID_ARG),
    ("router_w", None, M.MOE_INVALID_ARG), ("router_w", FAKE + 4, M.MOE_INVALID_ARG),
    ("shared_gate_w", None, M.MOE_INVALID_ARG),
])
def test_descriptor_rejections(field, value, status):
    d = fake_desc(**{field: value})
    assert forward(d, 4, 1 << 40) == status
    assert ws_bytes(d, 4) == 0


def test_weight_pointer_rejections():
    d = fake_desc()
    d.down = M.W4(FAKE + 8, FAKE, FAKE)          # q must be 16-byte aligned
    assert forward(d, 4, 1 << 40) == M.MOE_INVALID_ARG
    d = fake_desc()
    d.sh_up = M.W4(None, FAKE, FAKE)
    assert forward(d, 4, 1 << 40) == M.MOE_INVALID_ARG
    d = fake_desc(shared_ffn=0, shared_gate_w=None)   # no shared expert: its pointers unused
    d.sh_up = M.W4(None, None, None)
    assert forward(d, 0, 0) == M.MOE_OK


def test_call_rejections_before_launch():
    d = fake_desc()
    need = ws_bytes(d, 64)
    assert forward(d, 64, need - 1) == M.MOE_WORKSPACE_TOO_SMALL
    assert forward(d, -1, need) == M.MOE_INVALID_ARG
    assert forward(d, 0, 0) == M.MOE_OK                     # T = 0 is a no-op
    assert forward(d, 64, need, flags=8) == M.MOE_INVALID_ARG
    assert forward(d, 64, need, x=FAKE + 2) == M.MOE_INVALID_ARG
    assert forward(d, 64, need, out=None) == M.MOE_INVALID_ARG
    assert M.lib().moe_layer_forward(ctypes.byref(d), FAKE, 64, FAKE, FAKE + 16, need, 0, None) \
        == M.MOE_INVALID_ARG                                   # workspace must be 256-byte aligned
    L = M.lib()
    assert L.moe_route(ctypes.byref(d), FAKE, 4, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) \
        == M.MOE_INVALID_ARG                                   # shared_gate needed when Fs > 0
    assert L.moe_route(ctypes.byref(d), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) \
        == M.MOE_WORKSPACE_TOO_SMALL
    plan = M.Plan(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE)      # blocks must be 16-byte aligned
    assert L.moe_permute(ctypes.byref(d), FAKE, 4, ctypes.byref(plan), FAKE, 1 << 30, None) \
        == M.MOE_INVALID_ARG
    plan = M.Plan(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_grouped_gemm_w4(ctypes.byref(d), 7, FAKE, 4, ctypes.byref(plan), None, None,
                                 FAKE, FAKE, 1 << 30, None) == M.MOE_INVALID_ARG
    assert L.moe_grouped_gemm_w4(ctypes.byref(d), M.MOE_GEMM_DOWN_COMBINE, FAKE, 4,
                                 ctypes.byref(plan), None, FAKE, FAKE, FAKE, 1 << 30, None) \
        == M.MOE_INVALID_ARG                                   # combine needs topk_w
    assert L.moe_combine(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 4, FAKE, None) \
        == M.MOE_INVALID_ARG                                   # shared_y needed when Fs > 0
    w = M.W4(FAKE, FAKE, FAKE)
    assert L.moe_debug_dequant_w4(ctypes.byref(w), 4, 128, 0, 4, FAKE, None, None) \
        == M.MOE_INVALID_ARG                                   # row out of range
    assert L.moe_debug_dequant_w4(ctypes.byref(w), 4, 96, 0, 0, FAKE, None, None) \
        == M.MOE_UNSUPPORTED



def test_workspace_layout_export():
    """The test export reports the regions in order, inside the workspace size."""
    import ctypes as C
    d = fake_desc()
    for T, flags in ((1, 0), (8, 0), (4096, 0), (4096, M.MOE_FLAG_ATOMIC_COMBINE)):
        arr = (C.c_size_t * len(M.WS_REGIONS))()
        assert M.lib().moe_debug_workspace_layout(C.byref(d), T, flags, arr, len(arr)) == M.MOE_OK
        off = list(arr)
        assert off[-1] == ws_bytes(d, T, flags)
        assert off == sorted(off) and all(o % 256 == 0 for o in off)
        # A holds T*K*F + T*Fs bf16 values, Y (deterministic only) (T*K + T)*H fp32
        a, y, total = off[M.WS_REGIONS.index("a")], off[M.WS_REGIONS.index("y")], off[-1]
        assert y - a >= (T * 8 * 512 + T * 512) * 2
        if flags & M.MOE_FLAG_ATOMIC_COMBINE:
            assert total == y
        else:
            assert total - y >= (T * 8 + T) * 2048 * 4
    arr = (C.c_size_t * 14)()
    assert M.lib().moe_debug_workspace_layout(C.byref(d), 4, 4, arr, 14) == M.MOE_INVALID_ARG


def test_greedy_step_rejections():
    """Host-side checks of moe_greedy_next_input (no kernel is enqueued on these paths)."""
    from bit_grouped_gemm_amd import greedy_head as Gh
    L = Gh._lib()
    w = M.W4(FAKE, FAKE, FAKE)
    ws = Gh.workspace_bytes(151936, 1)
    assert ws >= 151936 * 4 and Gh.workspace_bytes(0, 1) == 0 and Gh.workspace_bytes(10, 17) == 0

    def call(V=1000, H=2048, T=1, x=FAKE, tok=FAKE, xn=FAKE, wsp=FAKE, nbytes=1 << 30, head=w):
        return L.moe_greedy_next_input(ctypes.byref(head), ctypes.byref(w), V, H, x, T, tok, xn,
                                       wsp, nbytes, None)
    assert call(H=3072) == M.MOE_UNSUPPORTED
    assert call(H=4096, T=9) == M.MOE_UNSUPPORTED
    assert call(T=0) == M.MOE_INVALID_ARG and call(T=17) == M.MOE_INVALID_ARG
    assert call(V=0) == M.MOE_INVALID_ARG
    assert call(x=None) == M.MOE_INVALID_ARG and call(tok=None) == M.MOE_INVALID_ARG
    assert call(x=FAKE + 2) == M.MOE_INVALID_ARG           # x must be 16-byte aligned
    assert call(wsp=FAKE + 16) == M.MOE_INVALID_ARG        # workspace 256-byte aligned
    assert call(nbytes=16) == M.MOE_WORKSPACE_TOO_SMALL
    assert call(head=M.W4(None, FAKE, FAKE)) == M.MOE_INVALID_ARG
