#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X (tokens/s, and the fraction of the roofline).

    python bench.py [--gpus 1] [--steps 640] [--warmup 80] [--only SECTION]

Workload (seeded synthetic data): the MoE layer of Qwen3.6-35B-A3B -- hidden 2048, 256 experts,
top-8, expert FFN 512, one shared expert with FFN 512, 4-bit group-64 affine weights. A step is
one full layer call (router, top-k, permutation, gate/up + SwiGLU, down + combine). The headline
is batch-1 decode (T = 1); the same JSON line carries batch-8 decode, T = 4096 prefill (uniform
and skewed routing) and the 40-layer stack (4096-token prefill in 512-token chunks, then 256
decode steps).

Inputs are resident in HBM before timing starts. Consecutive calls rotate over a pool of 40
independently seeded layers (18 GB; several times the 256 MiB Infinity Cache between two uses of
one layer) and a pool of tokens, so every call streams its weights from HBM. Timed regions are
HIP-graph replays bracketed by device synchronisation and HIP events on the stream the kernels
are launched on.

The headline times exactly --steps layer calls after --warmup untimed ones; latency
percentiles (p10 / median / p90 per call) come from separate series of graph replays. The
same run measures the ceilings the chip reaches in practice (a 1 GiB copy, a 1 GiB read, the
library's MFMA-loop kernel) and reports every roofline fraction against both the datasheet
peak and that measured ceiling. The CPU baseline is the fp64 oracle on bounded samples.

--only decode_t1 | decode_t8 | prefill_uniform | prefill_skewed | stack | copy | peaks runs one
section (for profiler runs; "copy" is a plain 256 MiB device copy and a 256 MiB read used to
calibrate the memory counters) and prints no JSON.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed FMA), TFLOP/s
N_LAYERS = 40                  # the stack, also the rotation pool of the single-layer sections
T_PREFILL = 4096
CHUNK = 512
DECODE_STEPS_STACK = 256
METRIC = "MoE-layer tokens/s at T=1 and T=4096; % HBM-BW / % bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed decode layer calls (T=1)")
    ap.add_argument("--warmup", type=int, default=80, help="untimed decode layer calls first")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle CPU-baseline budget of the decode leg")
    ap.add_argument("--only", choices=["decode_t1", "decode_t8", "prefill_uniform",
                                       "prefill_skewed", "stack", "copy", "peaks", "attn",
                                       "delta", "greedy"])
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--attn-contexts", default="4096,32768,131072",
                    help="context lengths of the attention section (comma-separated)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(key: str):
    """HBM bytes per launch from the committed counter summary (profiles/traffic.json), or None
    if it is absent or was taken on other sources of that kernel."""
    from bit_grouped_gemm_amd.profiling import traffic_entry
    return traffic_entry(os.path.join(ROOT, "profiles", "traffic.json"), key)


# ----------------------------------------------------------------------------- workload
class Pool:
    """Device-resident layers (uniform and skewed-router views of the same weights) and tokens."""

    def __init__(self, n_layers: int):
        import numpy as np
        import torch
        import synth
        from bit_grouped_gemm_amd import moe_w4 as M
        self.shape = s = synth.SHAPES["full"]
        t0 = time.time()
        self.layers, self.skew_layers = [], []
        bias = torch.from_numpy(synth.skew_router_bias(s.E)).cuda()
        self.host0 = synth.make_layer(s, seed=0, layer=0)     # kept for the CPU baseline
        host = None                                           # one buffer for layers 1..n-1
        for i in range(n_layers):
            if i > 0:
                host = synth.make_layer(s, seed=0, layer=i, reuse=host)
            dl = M.upload_layer(self.host0 if i == 0 else host, s.H, s.E, s.K, s.F, s.Fs)
            self.layers.append(dl)
            t = dict(dl.tensors)
            t["router_bias"] = bias
            self.skew_layers.append(M.make_layer(t, s.H, s.E, s.K, s.F, s.Fs))
        del host
        torch.cuda.synchronize()
        log(f"{n_layers} layers resident ({n_layers * 452984832 / 1e9:.1f} GB of routed weights) "
            f"in {time.time() - t0:.1f}s")
        self.tok_host = synth.make_tokens(s, 1024, seed=0, stream=0)
        self.tok = torch.from_numpy(self.tok_host.view(np.int16)).cuda()
        self.prefill_host = [synth.make_tokens(s, T_PREFILL, seed=0, stream=10 + j) for j in range(2)]
        self.prefill = [torch.from_numpy(x.view(np.int16)).cuda() for x in self.prefill_host]

    def head(self, seed: int):
        """A device LM head and embedding of the default vocabulary (built once per seed)."""
        if not hasattr(self, "_heads"):
            self._heads = {}
        if seed not in self._heads:
            import synth
            from bit_grouped_gemm_amd import greedy_head as Gh
            self._heads[seed] = Gh.upload_head(synth.make_head(synth.VOCAB, self.shape.H, seed))
        return self._heads[seed]

    def token_slice(self, i, T):
        n = self.tok.shape[0]
        o = (i * T) % (n - T + 1)
        return self.tok[o:o + T]


GRAPH_MAX_CALLS = 640


def _capture(calls):
    """Capture zero-argument launchers into HIP graphs of at most GRAPH_MAX_CALLS calls each
    (after one eager pass that loads code objects and checks for errors)."""
    import torch
    for c in calls:
        c()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    for i in range(0, len(calls), GRAPH_MAX_CALLS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in calls[i:i + GRAPH_MAX_CALLS]:
                c()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_exact(timed, warm) -> float:
    """Replay the `warm` calls untimed, then exactly the `timed` calls between two HIP events on
    the stream the replays run on (the current stream); returns ms per timed call."""
    import torch
    gw = _capture(warm) if warm else []
    gt = _capture(timed)
    for g in gw:
        g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for g in gt:
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / len(timed)


def graph_time(calls, reps: int, warm_reps: int) -> float:
    """One graph of `calls`, replayed `warm_reps` times untimed and `reps` times timed (one
    event pair around all of them); returns ms per call."""
    return replay_stats(calls, reps, warm_reps)["mean"]


def replay_stats(calls, reps: int, warm_reps: int = 1) -> dict:
    """One graph of `calls` replayed `reps` times, each replay between its own pair of events on
    the replay stream: ms per call as the mean over all replays and the 10th, 50th and 90th
    percentile over the replays."""
    import numpy as np
    import torch
    (g,) = _capture(calls) if len(calls) <= GRAPH_MAX_CALLS else (None,)
    assert g is not None, "replay_stats takes at most GRAPH_MAX_CALLS calls"
    for _ in range(warm_reps):
        g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(cur)
    for r in range(reps):
        g.replay()
        ev[r + 1].record(cur)
    torch.cuda.synchronize()
    per = np.array([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]) / len(calls)
    return {"mean": float(ev[0].elapsed_time(ev[reps]) / (reps * len(calls))),
            "p10": float(np.percentile(per, 10)), "median": float(np.median(per)),
            "p90": float(np.percentile(per, 90)), "replays": reps, "calls_per_replay": len(calls)}


def pct_us(st: dict) -> dict:
    """Latency percentiles in microseconds per call (over graph replays)."""
    return {"p10": st["p10"] * 1e3, "median": st["median"] * 1e3, "p90": st["p90"] * 1e3,
            "over": f"{st['replays']} graph replays of {st['calls_per_replay']} calls"}


# ------------------------------------------------------------------------------ measured peaks
def measured_peaks() -> dict:
    """The ceilings this chip reaches in practice, beside the datasheet figures: a 1 GiB
    device-to-device copy (bytes read + written per second), a 1 GiB read-only reduction, and
    the MFMA-loop kernel of the library (independent bf16 MFMAs on every SIMD)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    cur = torch.cuda.current_stream()

    def best(fn, reps=5):
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            fn()
            e1.record(cur)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    b.copy_(a)
    copy_ms = best(lambda: b.copy_(a))
    sink = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    reads = {}
    for wg in (1024, 2048):
        M.moe_bench_stream_read(a, wg, sink)
        reads[wg] = best(lambda: M.moe_bench_stream_read(a, wg, sink))
    read_ms = min(reads.values())
    flops = M.moe_bench_mfma_loop(1024, 200, sink)  # warm-up launch
    flops = M.moe_bench_mfma_loop(1024, 20000, sink)
    mfma_ms = best(lambda: M.moe_bench_mfma_loop(1024, 20000, sink), reps=3)
    del a, b, sink
    return {"copy_gbs": 2 * n / (copy_ms * 1e-3) / 1e9, "read_gbs": n / (read_ms * 1e-3) / 1e9,
            "mfma_bf16_tflops": flops / (mfma_ms * 1e-3) / 1e12,
            "how": "1 GiB device copy (read + write bytes); 1 GiB streaming read with 16-byte "
                   "loads (library kernel, 1024 or 2048 workgroups); MFMA-loop kernel: 1024 "
                   "workgroups x 4 waves x 20000 x 8 independent v_mfma_f32_32x32x16_bf16; "
                   "best of 5 / 5 / 3 runs"}


# ------------------------------------------------------------------------ algorithmic work
def expert_bytes(s, ffn):
    """Packed words + bf16 scales + bf16 biases of one expert's three projections."""
    per_mat = ffn * s.H // 2 + 2 * 2 * ffn * (s.H // 64)
    return 3 * per_mat


def gateup_bytes(s, ffn):
    return 2 * (ffn * s.H // 2 + 2 * 2 * ffn * (s.H // 64))


def decode_layer_bytes(s, T, distinct):
    """Algorithmic HBM bytes of one decode call: each selected expert's weights once, the shared
    expert, the router and shared-gate weights, the tokens and the output."""
    return ((distinct + 1) * expert_bytes(s, s.F) + s.E * s.H * 4 + s.H * 4
            + T * s.H * 2 + T * s.H * 4)


def layer_flops(s, T):
    """Algorithmic flops of one layer call: router, gate/up, down (shared expert included)."""
    return (2.0 * T * s.H * s.E + 2.0 * T * s.K * s.H * 2 * s.F + 2.0 * T * s.K * s.F * s.H
            + 2.0 * T * s.H * 2 * s.Fs + 2.0 * T * s.Fs * s.H)


def gateup_flops(s, T):
    return 2.0 * s.H * 2 * s.F * T * s.K + 2.0 * s.H * 2 * s.Fs * T


def down_flops(s, T):
    return 2.0 * s.F * s.H * T * s.K + 2.0 * s.Fs * s.H * T


# ----------------------------------------------------------------------------- sections
def decode_section(pool: Pool, T: int, steps: int, warmup: int):
    """Exactly `steps` layer calls at T tokens (all launches; layers and tokens rotate), after
    `warmup` untimed calls; latency percentiles over replays of 40 calls (each layer once);
    then the dominant launch alone: phase 1 (top-k + gate/up of the selected experts) replayed
    on workspaces prepared by a full call."""
    import numpy as np
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.layers
    out = torch.empty((T, s.H), dtype=torch.float32, device="cuda")
    ws = M.alloc_workspace(L[0], T)

    def call(i):
        x = pool.token_slice(i, T)
        return lambda: M.moe_layer_forward(L[i % len(L)], x, out, ws)

    ms = time_exact([call(i) for i in range(steps)], [call(i) for i in range(warmup)])
    pct = replay_stats([call(i) for i in range(len(L))], 24)

    # the dominant kernel, live: per-call workspaces hold the state phase 1 starts from
    states = []
    for i in range(len(L)):
        layer, x = L[i], pool.token_slice(i, T)
        wsi = M.alloc_workspace(layer, T)
        M.moe_layer_forward(layer, x, out, wsi)
        idx = torch.empty(T * s.K, dtype=torch.int32, device="cuda")
        cnt = torch.empty(s.E, dtype=torch.int32, device="cuda")
        M.moe_route(layer, x, idx, torch.empty(T * s.K, device="cuda"),
                    torch.empty(T, device="cuda"), cnt, M.alloc_workspace(layer, T))
        states.append((layer, x, wsi, cnt))
    torch.cuda.synchronize()
    distinct = [int((st[3] > 0).sum().item()) for st in states]
    kb = float(np.mean([d * gateup_bytes(s, s.F) for d in distinct]))
    kb += T * (s.E + 1) * 4 + T * s.H * 2 + T * s.K * s.F * 2    # logits, x in; A out
    phases = {}
    for ph, name in enumerate(("k_dec_a", "k_dec_b", "k_dec_c")):
        phases[name] = replay_stats([(lambda st=st, ph=ph: M.moe_layer_forward_phase(
            st[0], st[1], out, st[2], ph)) for st in states], 8)["mean"] * 1e3
    d_mean = float(np.mean(distinct))
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "steps": steps,
            "warmup": warmup, "distinct_experts": d_mean, "latency_us": pct_us(pct),
            "layer_bytes": decode_layer_bytes(s, T, d_mean), "phases_us": phases,
            "kernel": {"name": "k_dec_b (top-k + gate/up of the selected experts)",
                       "us": phases["k_dec_b"], "bytes": kb}}


def padding_frac(counts, rows=32):
    """Share of the MFMA rows that are padding: experts' rows rounded up to whole row tiles."""
    import numpy as np
    c = np.asarray(counts, dtype=np.int64)
    padded = ((c + rows - 1) // rows * rows).sum()
    return float(padded - c.sum()) / float(padded) if padded else 0.0


def prefill_section(pool: Pool, steps: int, skewed: bool):
    """Exactly `steps` layer calls at T = 4096 (layers rotate, two token batches alternate);
    latency percentiles over replays of 8 calls; the time of each launch of the layer replayed
    on its own on prepared workspaces."""
    import numpy as np
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.skew_layers if skewed else pool.layers
    T = T_PREFILL
    ws = M.alloc_workspace(L[0], T)
    out = torch.empty((T, s.H), dtype=torch.float32, device="cuda")

    def call(i):
        return lambda: M.moe_layer_forward(L[i % len(L)], pool.prefill[i % 2], out, ws)

    ms = time_exact([call(i) for i in range(steps)], [call(i) for i in range(2)])
    pct = replay_stats([call(i) for i in range(8)], 8)
    # each launch on its own, on workspaces prepared by a full call
    nk = min(8, len(L))
    states = []
    for i in range(nk):
        wsi = M.alloc_workspace(L[i], T)
        M.moe_layer_forward(L[i], pool.prefill[i % 2], out, wsi)
        states.append((L[i], pool.prefill[i % 2], wsi))
    torch.cuda.synchronize()
    names = ("router", "top-k", "permutation", "gate/up GEMM", "down GEMM", "combine")
    assert M.moe_layer_num_phases(L[0], T) == len(names)
    phases = {}
    for ph, name in enumerate(names):
        phases[name] = replay_stats([(lambda st=st, ph=ph: M.moe_layer_forward_phase(
            st[0], st[1], out, st[2], ph)) for st in states], 6)["mean"] * 1e3
    # routing of the timed batches: padding of the 32-row MFMA tiles
    pads = []
    for i in range(2):
        cnt = torch.empty(s.E, dtype=torch.int32, device="cuda")
        M.moe_route(L[i], pool.prefill[i], torch.empty(T * s.K, dtype=torch.int32, device="cuda"),
                    torch.empty(T * s.K, device="cuda"), torch.empty(T, device="cuda"), cnt,
                    M.alloc_workspace(L[i], T))
        c = cnt.cpu().numpy()
        pads.append(padding_frac(np.concatenate([c, [T]])))
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "steps": steps,
            "latency_us": pct_us(pct), "phases_us": phases,
            "mfma_row_padding_frac": float(np.mean(pads)),
            "kernel": {"name": "k_gemm_w4_gate_up (grouped GEMM, SwiGLU epilogue)",
                       "us": phases["gate/up GEMM"], "flops": gateup_flops(s, T)},
            "down_kernel": {"name": "k_gemm_w4_down (grouped GEMM, fp32 expert outputs)",
                            "us": phases["down GEMM"], "flops": down_flops(s, T)}}


def stack_section(pool: Pool):
    """The 40-layer stack: 4096-token prefill in 512-token chunks, then 256 decode steps at T=1
    whose input is the previous step's normalised output, left on the device."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    stack = M.Stack(pool.layers)
    ws = stack.alloc_workspace(CHUNK)
    x_all = pool.prefill[0]
    xs = [x_all[c * CHUNK:(c + 1) * CHUNK].clone() for c in range(T_PREFILL // CHUNK)]
    rs = [torch.empty((CHUNK, s.H), dtype=torch.float32, device="cuda") for _ in xs]
    prefill_calls = [(lambda x=x, r=r: stack.forward(r, x, ws)) for x, r in zip(xs, rs)]
    ms_chunk = graph_time(prefill_calls, 2, 1)
    prefill_ms = ms_chunk * len(xs)
    ws1 = stack.alloc_workspace(1)
    x1 = pool.token_slice(3, 1).clone()
    r1 = torch.empty((1, s.H), dtype=torch.float32, device="cuda")
    st = replay_stats([lambda: stack.forward(r1, x1, ws1)], DECODE_STEPS_STACK, 8)
    ms_step = st["mean"]
    assert torch.isfinite(r1).all().item()
    # the whole greedy decode step: the 40 layers, then the LM head, the argmax and the chosen
    # token's embedding written into the input slot the next step reads
    from bit_grouped_gemm_amd import greedy_head as Gh
    hd = pool.head(0)
    wsg = Gh.alloc_workspace(hd.V, 1)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    xg = pool.token_slice(5, 1).clone()

    def step():
        stack.forward(r1, xg, ws1)
        Gh.next_input(hd, xg, tok, xg, wsg)
    stg = replay_stats([step], DECODE_STEPS_STACK, 8)
    assert 0 <= int(tok.item()) < hd.V
    return {"layers": len(pool.layers), "prefill_tokens": T_PREFILL, "chunk": CHUNK,
            "prefill_ms": prefill_ms, "prefill_tokens_per_s": T_PREFILL / (prefill_ms * 1e-3),
            "decode_steps": DECODE_STEPS_STACK, "decode_ms_per_token": ms_step,
            "decode_tokens_per_s": 1.0 / (ms_step * 1e-3),
            "decode_latency_us": pct_us(st),
            "decode_hbm_frac": len(pool.layers) * decode_layer_bytes(s, 1, s.K) / (ms_step * 1e-3)
            / 1e9 / HBM_PEAK_GBS,
            "greedy_decode": {"what": "40 layers + LM head + argmax + embedding of the token into "
                                      "the input slot, per token (vocabulary %d)" % hd.V,
                              "ms_per_token": stg["mean"], "tokens_per_s": 1.0 / (stg["mean"] * 1e-3),
                              "latency_us": pct_us(stg)}}


def greedy_section(pool: Pool):
    """The greedy step alone at T = 1: the 4-bit LM head over the vocabulary (151,936 x 2048),
    the argmax and the embedding row. Calls alternate between two heads (350 MB together, more
    than the memory-side cache). Algorithmic bytes: the head's packed words, scales and biases
    once, x, the token's embedding row (packed) and the next input."""
    import torch
    from bit_grouped_gemm_amd import greedy_head as Gh
    heads = [pool.head(0), pool.head(1)]
    V, H = heads[0].V, heads[0].H
    ws = Gh.alloc_workspace(V, 1)
    xs = [pool.token_slice(7 + i, 1).clone() for i in range(2)]
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    xn = torch.empty_like(xs[0])
    calls = [(lambda h=h, x=x: Gh.next_input(h, x, tok, xn, ws)) for h, x in zip(heads, xs)]
    st = replay_stats(calls, 64)
    nbytes = V * H // 2 + 2 * 2 * V * (H // 64) + H * 2 + H // 2 + 4 * (H // 64) + H * 2
    gbs = nbytes / (st["mean"] * 1e-3) / 1e9
    return {"workload": f"greedy step, T=1: 4-bit LM head {V} x {H}, argmax, embedding",
            "us_per_call": st["mean"] * 1e3, "latency_us": pct_us(st), "bytes_per_call": nbytes,
            "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "logits_kernel_traffic": measured_traffic(f"greedy@v{V}_t1")}


def attention_section(contexts=(4096, 32768, 131072)):
    """GQA decode attention of the model's full-attention layers (16 query heads, 2 KV heads,
    head size 128, 64-token cache blocks), batch 1, at several context lengths. Calls rotate
    over disjoint sequences of one 512 MiB block pool (blocks scattered by a random
    permutation), so every call reads its keys and values from HBM; the same sequences are
    also timed unpacked (one query head per workgroup) and with their blocks in physical order.
    Algorithmic bytes: the sequence's keys and values once, the block-table entries, q and out."""
    import torch
    from bit_grouped_gemm_amd import attn_gqa as G
    import synth
    shape = synth.ATTN_SHAPES["full"]
    Hq, Hkv, D, BS = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.block_size
    d = G.desc(Hq, Hkv, D, BS)
    blk_bytes = Hkv * BS * D * 2
    n_phys = (512 << 20) // blk_bytes
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    kc = torch.randn((n_phys, Hkv, BS, D), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((n_phys, Hkv, BS, D), generator=gen, device="cuda").to(torch.bfloat16)
    perm = torch.randperm(n_phys, generator=gen, device="cuda").to(torch.int32)
    out = {}
    for S in contexts:
        nb = S // BS
        nseq = min(64, n_phys // nb)
        tables = [perm[i * nb:(i + 1) * nb].reshape(1, nb).contiguous() for i in range(nseq)]
        lens = torch.full((1,), S, dtype=torch.int32, device="cuda")
        qs = [torch.randn((1, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
              for _ in range(nseq)]
        o = torch.empty((1, Hq, D), dtype=torch.float32, device="cuda")
        ws = G.alloc_workspace(d, 1, S)
        # the same sequences with their blocks in physical order (a contiguous cache)
        in_order = [torch.arange(i * nb, (i + 1) * nb, dtype=torch.int32, device="cuda").reshape(1, nb)
                    for i in range(nseq)]
        res = {}
        for flags, tag, tabs in ((0, "packed", tables), (G.ATTN_FLAG_UNPACKED, "unpacked", tables),
                                 (0, "packed_blocks_in_order", in_order)):
            calls = [(lambda i=i, f=flags, t=tabs: G.decode(d, qs[i].view(torch.int16),
                                                            kc.view(torch.int16), vc.view(torch.int16),
                                                            t[i], lens, S, o, ws, f))
                     for i in range(nseq)]
            st = replay_stats(calls, max(4, 256 // nseq))
            nbytes = 2.0 * Hkv * S * D * 2 + nb * 4 + Hq * D * 2 + Hq * D * 4
            gbs = nbytes / (st["mean"] * 1e-3) / 1e9
            res[tag] = {"us_per_call": st["mean"] * 1e3, "latency_us": pct_us(st),
                        "bytes_per_call": nbytes, "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        # HBM bytes of the packed split kernel from the committed counter runs
        res["packed"]["split_kernel_traffic"] = measured_traffic(f"attn_split@ctx{S // 1024}k")
        res["packing_speedup"] = res["unpacked"]["us_per_call"] / res["packed"]["us_per_call"]
        out[f"S={S}"] = res
        del ws
    return {"workload": "GQA decode attention, batch 1: 16 query heads, 2 KV heads, head size 128, "
                        "bf16 KV cache in 64-token blocks scattered over a 512 MiB pool",
            "contexts": out}


def delta_section():
    """The gated delta rule of the model's linear-attention layers (16 heads, 128 x 128 fp32
    state): a decode step at batch 1 and 8 (token-by-token kernel), and a 512-token prefill at
    batch 1 (chunkwise kernels; the token-by-token kernel is timed beside it). Calls rotate over
    states in a pool of at least 320 MiB. Algorithmic bytes: the state read and written once,
    plus the tokens' q, k, v, g, beta and o."""
    import torch
    from bit_grouped_gemm_amd import delta_rule as DR
    import synth
    sh = synth.DELTA_SHAPES["full"]
    Hk, Hv, dk, dv = sh.num_k_heads, sh.num_v_heads, sh.dk, sh.dv
    d = DR.desc(Hk, Hv, dk, dv)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    res = {}
    for B, T in ((1, 1), (8, 1), (1, 512)):
        state_bytes = B * Hv * dv * dk * 4
        npool = max(4, min(320, (320 << 20) // state_bytes))
        pool = [torch.randn((B, Hv, dv, dk), generator=gen, device="cuda") * 0.1 for _ in range(npool)]
        q = torch.randn((B, T, Hk, dk), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        k = torch.randn((B, T, Hk, dk), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        v = torch.randn((B, T, Hv, dv), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        g = torch.log(torch.rand((B, T, Hv), generator=gen, device="cuda") * 0.099 + 0.9)
        beta = torch.sigmoid(torch.randn((B, T, Hv), generator=gen, device="cuda"))
        o = torch.empty((B, T, Hv, dv), device="cuda")
        calls = [(lambda st=st: DR.forward(d, q, k, v, g, beta, st, st, o)) for st in pool]
        n = min(len(calls), 320 if T == 1 else 16)
        token_st = None
        if T > 1:
            token_st = replay_stats(calls[:n], 3)
            ws = DR.alloc_chunked_workspace(d, B, T)
            calls = [(lambda st=st: DR.forward_chunked(d, q, k, v, g, beta, st, st, o, ws))
                     for st in pool]
        st = replay_stats(calls[:n], max(2, 640 // n) if T == 1 else 3)
        nbytes = 2.0 * state_bytes + B * T * (2 * Hk * dk * 2 + Hv * dv * 2 + 2 * Hv * 4 + Hv * dv * 4)
        gbs = nbytes / (st["mean"] * 1e-3) / 1e9
        res[f"B={B},T={T}"] = {"us_per_call": st["mean"] * 1e3, "latency_us": pct_us(st),
                               "tokens_per_s": B * T / (st["mean"] * 1e-3),
                               "bytes_per_call": nbytes, "achieved_gbs": gbs,
                               "hbm_frac": gbs / HBM_PEAK_GBS,
                               "traffic": measured_traffic(f"delta@b{B}_t{T}")}
        if token_st is not None:
            res[f"B={B},T={T}"]["path"] = "chunked (32-token chunks)"
            res[f"B={B},T={T}"]["token_path_us"] = token_st["mean"] * 1e3
            # HBM bytes per launch of the prep kernel ("traffic" is the main kernel's)
            res[f"B={B},T={T}"]["prep_traffic"] = measured_traffic(f"delta_prep@b{B}_t{T}")
            res[f"B={B},T={T}"]["chunked_speedup"] = token_st["mean"] / st["mean"]
            # fp32 multiply-adds of the chunkwise form per (sequence, head, 32-token chunk): the
            # chunk's kh.kh and qh.kh products, then per state row kh.S and qh.S, T R, P delta
            # and the rank-32 state update
            C = 32
            fma = B * Hv * ((T + C - 1) // C) * (dv * (3 * C * dk + C * C) + 2 * C * C * dk)
            tf = 2.0 * fma / (st["mean"] * 1e-3) / 1e12
            res[f"B={B},T={T}"]["alu"] = {"flops_per_call": 2.0 * fma, "achieved_tflops": tf,
                                          "peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                                          "frac": tf / FP32_VECTOR_PEAK_TFLOPS}
        del pool
    return {"workload": "gated delta rule, 16 heads, 128 x 128 fp32 state per head; decode steps "
                        "(T=1) and a 512-token prefill", "cases": res}


def copy_section():
    """Calibration kernels for FETCH_SIZE / WRITE_SIZE: a plain 256 MiB device-to-device copy
    (reads and writes 256 MiB) and a 256 MiB fp32 sum (reads 256 MiB, writes 4 bytes)."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    af = a.view(torch.float32)
    for _ in range(3):
        af.sum()
    torch.cuda.synchronize()
    log(f"copied {n} bytes 3 times, summed {n} bytes 3 times")


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    return threads, blas


def cpu_baseline(pool: Pool, budget_s: float):
    """The fp64 oracle on the host (as it stands) for the same workload, on bounded samples:
      * decode T = 1: whole layer calls of layer 0 on successive tokens until the budget is used;
      * prefill T = 4096: the routing of all 4096 tokens, the shared expert on all of them, and
        16 of the 256 routed experts on their routed rows, the expert time scaled by 256/16;
      * 40-layer stack: 40 x (8 chunks of 512 tokens timed as above, 24 experts sampled) for the
        prefill, 40 x the T = 1 layer time for a decode step.
    Returns tokens/s figures; everything but the decode leg is labelled "extrapolated"."""
    import numpy as np
    from oracle import moe_oracle as O
    threads, blas = _blas_info()
    host, s = pool.host0, pool.shape
    n, t0 = 0, time.time()
    while n < 2 or time.time() - t0 < budget_s:
        O.layer_forward(host, pool.tok_host[n:n + 1], s.K, "bf16")
        n += 1
    dt = time.time() - t0
    decode_s = dt / n

    def layer_time(xh, n_sample):
        """Oracle seconds for one layer on tokens xh: routing + shared expert + all routed
        experts, the latter extrapolated from n_sample experts spread over the expert ids."""
        t = time.time()
        logits = O.router_logits(xh, host["router_w"], host["router_bias"])
        idx, p = O.select_topk(logits, s.K)
        sg = O.shared_gate(xh, host["shared_gate_w"])
        x = O.bf16_to_f64(xh)
        deq = lambda nm, e: O.dequant(host[nm][0][e], host[nm][1][e], host[nm][2][e], "bf16")  # noqa: E731
        ysh = O.expert_ffn(x, deq("sh_gate", 0), deq("sh_up", 0), deq("sh_down", 0), "bf16")
        out = sg[:, None] * ysh
        t_fixed = time.time() - t
        t = time.time()
        for e in np.linspace(0, s.E - 1, n_sample).astype(int):
            tt, kk = np.nonzero(idx == e)
            y = O.expert_ffn(x[tt], deq("gate", e), deq("up", e), deq("down", e), "bf16")
            np.add.at(out, tt, p[tt, kk][:, None] * y)
        return t_fixed + (time.time() - t) * s.E / n_sample

    xp = pool.prefill_host[0]
    prefill_s = layer_time(xp, 16)
    chunk_s = layer_time(xp[:CHUNK], 24)
    stack_prefill_s = N_LAYERS * (T_PREFILL // CHUNK) * chunk_s
    stack_decode_s = N_LAYERS * decode_s
    return {"value": 1.0 / decode_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"decode T=1: {n} tokens through layer 0 of the full-size layer in {dt:.1f}s "
                      f"(fp64 NumPy oracle, bf16 profile); BLAS={blas}, "
                      f"host cpus={len(os.sched_getaffinity(0))}",
            "prefill_t4096": {"value": T_PREFILL / prefill_s, "unit": "tokens/s",
                              "kind": "oracle, extrapolated",
                              "sample": "routing and shared expert of all 4096 tokens, 16 of 256 "
                                        "routed experts on their rows, scaled by 256/16"},
            "stack_40_layers": {"prefill_tokens_per_s": T_PREFILL / stack_prefill_s,
                                "decode_tokens_per_s": 1.0 / stack_decode_s,
                                "kind": "oracle, extrapolated",
                                "sample": "one 512-token chunk of layer 0 (24 of 256 experts, "
                                          "scaled) x 8 chunks x 40 layers; decode: the T=1 layer "
                                          "time x 40 layers"}}


def roofline_hbm(k, peaks=None):
    ach = k["bytes"] / (k["us"] * 1e-6) / 1e9
    r = {"bound": "hbm", "kernel": k["name"], "achieved": ach, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "bytes_per_launch": k["bytes"],
         "avg_launch_us": k["us"]}
    if peaks:
        r["measured_peak"] = max(peaks["copy_gbs"], peaks["read_gbs"])
        r["frac_of_measured_peak"] = ach / r["measured_peak"]
    return r


def roofline_mfma(k, peaks=None):
    ach = k["flops"] / (k["us"] * 1e-6) / 1e12
    r = {"bound": "mfma", "kernel": k["name"], "achieved": ach, "peak": BF16_PEAK_TFLOPS,
         "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "flops_per_launch": k["flops"],
         "avg_launch_us": k["us"]}
    if peaks:
        r["measured_peak"] = peaks["mfma_bf16_tflops"]
        r["frac_of_measured_peak"] = ach / r["measured_peak"]
    return r


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the MoE layer is not sharded "
                                   "across GPUs; run it with --gpus 1"}))
        sys.exit(2)
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    from bit_grouped_gemm_amd.profiling import kernel_source_hash
    M.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    log(f"device {torch.cuda.get_device_name(0)}, {M.moe_version()}")
    if args.only == "copy":
        copy_section()
        return
    if args.only == "peaks":
        log(f"peaks: {measured_peaks()}")
        return
    contexts = tuple(int(c) for c in args.attn_contexts.split(","))
    if args.only == "attn":
        log(f"attention: {json.dumps(attention_section(contexts))}")
        return
    if args.only == "delta":
        log(f"delta rule: {json.dumps(delta_section())}")
        return

    pool = Pool(N_LAYERS)
    s = pool.shape
    t_all = time.time()
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    if args.only == "decode_t1":
        r = decode_section(pool, 1, steps, warmup)
        log(f"decode T=1: {r['ms_per_step'] * 1e3:.2f} us/layer; phases {r['phases_us']}")
        return
    if args.only == "decode_t8":
        r = decode_section(pool, 8, steps, warmup)
        log(f"decode T=8: {r['ms_per_step'] * 1e3:.2f} us/layer; phases {r['phases_us']}")
        return
    if args.only in ("prefill_uniform", "prefill_skewed"):
        r = prefill_section(pool, args.prefill_steps, args.only == "prefill_skewed")
        log(f"{args.only}: {r['ms_per_step'] * 1e3:.1f} us/layer; phases {r['phases_us']}")
        return
    if args.only == "stack":
        r = stack_section(pool)
        log(f"stack: {r}")
        return
    if args.only == "greedy":
        log(f"greedy step: {json.dumps(greedy_section(pool))}")
        return

    peaks = measured_peaks()
    log(f"measured peaks: copy {peaks['copy_gbs']:.0f} GB/s, read {peaks['read_gbs']:.0f} GB/s, "
        f"MFMA loop {peaks['mfma_bf16_tflops']:.0f} TFLOP/s")
    d1 = decode_section(pool, 1, steps, warmup)
    log(f"decode T=1: {d1['ms_per_step'] * 1e3:.2f} us/layer, {d1['tokens_per_s']:.0f} tok/s; "
        f"phases {d1['phases_us']}")
    d8 = decode_section(pool, 8, max(1, steps // 2), warmup)
    log(f"decode T=8: {d8['ms_per_step'] * 1e3:.2f} us/layer, {d8['tokens_per_s']:.0f} tok/s")
    prefill = {}
    for skewed in (False, True):
        tag = "skewed" if skewed else "uniform"
        p = prefill_section(pool, args.prefill_steps, skewed)
        fl = layer_flops(s, T_PREFILL)
        tf = fl / (p["ms_per_step"] * 1e-3) / 1e12
        rk = roofline_mfma(p["kernel"], peaks)
        rk["traffic"] = measured_traffic(f"gate_up@prefill_{tag}")
        prefill[tag] = {"value": p["tokens_per_s"], "unit": "tokens/s",
                        "ms_per_step": p["ms_per_step"], "steps": p["steps"],
                        "latency_us": p["latency_us"],
                        "layer_tflops": tf, "layer_mfma_frac": tf / BF16_PEAK_TFLOPS,
                        "layer_frac_of_measured_mfma_peak": tf / peaks["mfma_bf16_tflops"],
                        "mfma_row_padding_frac": p["mfma_row_padding_frac"],
                        "phases_us": p["phases_us"],
                        "roofline": rk, "down_roofline": roofline_mfma(p["down_kernel"], peaks)}
        prefill[tag]["down_roofline"]["traffic"] = measured_traffic(f"down@prefill_{tag}")
        prefill[tag]["combine_traffic"] = measured_traffic(f"combine@prefill_{tag}")
        log(f"prefill T=4096 {tag}: {p['ms_per_step'] * 1e3:.1f} us/layer "
            f"({p['tokens_per_s'] / 1e6:.2f} M tok/s, {tf:.0f} TFLOP/s); phases {p['phases_us']}")
    st = stack_section(pool)
    log(f"stack ({st['layers']} layers): prefill {st['prefill_tokens_per_s']:.0f} tok/s, "
        f"decode {st['decode_tokens_per_s']:.0f} tok/s ({st['decode_ms_per_token'] * 1e3:.0f} us/token); "
        f"with the greedy step {st['greedy_decode']['tokens_per_s']:.0f} tok/s")
    attn = attention_section(contexts)
    for k_, r_ in attn["contexts"].items():
        log(f"decode attention {k_}: {r_['packed']['us_per_call']:.1f} us "
            f"({r_['packed']['hbm_frac'] * 100:.1f} % of HBM), unpacked "
            f"{r_['unpacked']['us_per_call']:.1f} us")
    greedy = greedy_section(pool)
    log(f"greedy step (LM head {greedy['bytes_per_call'] / 1e6:.0f} MB): {greedy['us_per_call']:.1f} us "
        f"({greedy['hbm_frac'] * 100:.1f} % of HBM)")
    delta = delta_section()
    for k_, r_ in delta["cases"].items():
        if "alu" in r_:
            log(f"delta rule {k_}: {r_['us_per_call']:.2f} us chunkwise ({r_['alu']['frac'] * 100:.1f} % "
                f"of fp32 vector peak; token by token {r_['token_path_us']:.1f} us)")
        else:
            log(f"delta rule {k_}: {r_['us_per_call']:.2f} us ({r_['hbm_frac'] * 100:.1f} % of HBM)")
    log(f"timed sections took {time.time() - t_all:.1f}s")
    cpu = None if args.skip_cpu else cpu_baseline(pool, args.cpu_seconds)

    roof = roofline_hbm(d1["kernel"], peaks)
    roof["traffic"] = measured_traffic("k_dec_b@decode_t1")
    lbytes = d1["layer_bytes"] / (d1["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": d1["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": d1["steps"], "warmup": d1["warmup"], "ms_per_step": d1["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded: 4-bit g64 weights, x ~ N(0,1) bf16; no checkpoint)",
        "config": {"workload": "MoE layer, decode T=1 (batch 1): hidden 2048, 256 experts, top-8, "
                               "expert FFN 512, one shared expert FFN 512, 4-bit group-64 affine",
                   "layer_pool": N_LAYERS, "token_pool": int(pool.tok.shape[0])},
        "timing": f"exactly {d1['steps']} timed layer calls after {d1['warmup']} untimed ones, "
                  f"replayed from HIP graphs of at most {GRAPH_MAX_CALLS} calls between two HIP "
                  "events on the replay stream; layers rotate over the 40-layer pool",
        "roofline": roof,
        "cpu_baseline": cpu,
        "latency_us": d1["latency_us"],
        "phases_us": d1["phases_us"],
        "layer_bytes_per_token": d1["layer_bytes"],
        "layer_hbm_frac": lbytes / HBM_PEAK_GBS,
        "layer_frac_of_measured_hbm_peak": lbytes / max(peaks["copy_gbs"], peaks["read_gbs"]),
        "measured_peaks": peaks,
        "decode_t8": {"value": d8["tokens_per_s"], "unit": "tokens/s",
                      "ms_per_step": d8["ms_per_step"], "steps": d8["steps"],
                      "latency_us": d8["latency_us"], "phases_us": d8["phases_us"],
                      "distinct_experts": d8["distinct_experts"],
                      "layer_hbm_frac": d8["layer_bytes"] / (d8["ms_per_step"] * 1e-3) / 1e9
                      / HBM_PEAK_GBS,
                      "roofline": roofline_hbm(d8["kernel"], peaks)},
        "prefill_t4096": prefill,
        "stack_40_layers": st,
        "gqa_decode_attention": attn,
        "gated_delta_rule": delta,
        "greedy_step": greedy,
        "source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
