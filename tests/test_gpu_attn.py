"""GQA decode attention over a block-paged KV cache (attn_gqa_decode, through the C ABI)
against the fp64 oracle, element by element.

Tolerance (derived from the arithmetic; the layer's 2e-2 / 2e-3 bounds are for the MoE
layer): scores, exponentials and sums are fp32, so the output carries relative errors of a
few 1e-6; the gate is a row-normalised max relative error of 1e-4, which a single dropped or
repeated token of a 32K context (a change of about 1/S of the weight) still exceeds. A single
token is exact: its weight is exp(0)/1 = 1.
"""
import numpy as np
import pytest

import synth
from gpu_common import DEV, log
from oracle import attn_oracle as A
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-4


_INPUTS = {}


def inputs(shape, lens, seed, spare):
    """Seeded inputs, kept for the packed and the unpacked run of the same case."""
    key = (shape, tuple(lens), seed, spare)
    if key not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[key] = synth.make_attn_inputs(shape, lens, seed=seed, spare_blocks=spare)
    return _INPUTS[key]


def run(shape, lens, flags=0, seed=0, spare=3):
    import torch
    from bit_grouped_gemm_amd import attn_gqa as G
    q, kc, vc, table, sl = inputs(shape, lens, seed, spare)
    d = G.desc(shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.block_size)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a).view(t)).to(DEV)  # noqa: E731
    qd, kd, vd = dev(q, np.int16), dev(kc, np.int16), dev(vc, np.int16)
    td, ld = dev(table, np.int32), dev(sl, np.int32)
    max_len = int(max(lens)) if len(lens) else 0
    ws = G.alloc_workspace(d, len(lens), max_len)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    G.decode(d, qd, kd, vd, td, ld, max_len, out, ws, flags)
    torch.cuda.synchronize()
    ref = A.decode_attention(q, kc, vc, table, sl, shape.block_size, d.scale)
    return out.cpu().numpy().astype(np.float64), ref, (d, qd, kd, vd, td, ld, max_len, ws, out)


# ("tiny", [20000]): 157 spans of head size 64, merged in 32-dimension slices
CASES = [("tiny", [1, 15, 16, 17, 40]), ("tiny", [0, 3]), ("tiny", [20000]),
         ("mid", [31, 32, 33, 700]),
         ("wide", [63, 64, 65, 1500]), ("full", [1]), ("full", [4096]), ("full", [100, 2500, 64, 4097]),
         ("full", [32768]), ("full", [70001, 5, 131072, 1])]


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("name,lens", CASES)
def test_decode_attention_matches_oracle(name, lens, flags):
    shape = synth.ATTN_SHAPES[name]
    log(f"[attn] {name} lens={lens} flags={flags}")
    y, ref, _ = run(shape, lens, flags)
    assert np.all(np.isfinite(y))
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(y[b] == 0)
            continue
        st = O.error_stats(y[b], ref[b])
        log(f"[attn]   b={b} S={L}: max_rel={st['max_rel']:.2e} mean_abs={st['mean_abs']:.2e}")
        assert st["max_rel"] <= TOL, (b, L, st)
        if L == 1:   # one token: out = its value row exactly
            assert np.array_equal(y[b], ref[b])


def test_packed_and_unpacked_agree_and_repeat_bit_identically():
    import torch
    from bit_grouped_gemm_amd import attn_gqa as G
    shape = synth.ATTN_SHAPES["full"]
    y0, _, args = run(shape, [3000, 17], 0, seed=4)
    y1, _, _ = run(shape, [3000, 17], 1, seed=4)
    assert O.error_stats(y1.reshape(-1, 128), y0.reshape(-1, 128))["max_rel"] < 1e-5
    d, qd, kd, vd, td, ld, max_len, ws, out = args
    G.decode(d, qd, kd, vd, td, ld, max_len, out, ws, 0)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), y0.astype(np.float32))


def test_graph_replays_match_eager():
    import torch
    from bit_grouped_gemm_amd import attn_gqa as G
    shape = synth.ATTN_SHAPES["full"]
    y, _, (d, qd, kd, vd, td, ld, max_len, ws, out) = run(shape, [5000, 900], 0, seed=8)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.decode(d, qd, kd, vd, td, ld, max_len, out, ws, 0)
    for rep in range(3):
        out.fill_(float("nan"))
        G.decode(d, qd, kd, vd, td, ld, max_len, torch.empty_like(out), ws, 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), y.astype(np.float32)), rep
