#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X (tokens/s, and the fraction of the roofline).

    python bench.py [--gpus 1] [--steps 640] [--warmup 64] [--only SECTION]

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

--only decode_t1 | decode_t8 | prefill_uniform | prefill_skewed | stack | copy runs one section (for profiler runs;
"copy" is a plain 256 MiB device copy used to calibrate the memory counters) and prints no JSON.
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
N_LAYERS = 40                  # the stack, also the rotation pool of the single-layer sections
T_PREFILL = 4096
CHUNK = 512
DECODE_STEPS_STACK = 256
METRIC = "MoE-layer tokens/s at T=1 and T=4096; % HBM-BW / % bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed decode layer calls (T=1)")
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget")
    ap.add_argument("--only", choices=["decode_t1", "decode_t8", "prefill_uniform",
                                       "prefill_skewed", "stack", "copy"])
    ap.add_argument("--skip-cpu", action="store_true")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(key: str):
    """HBM bytes per launch from the committed counter summary (profiles/traffic.json), or None
    if it is absent or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    from bit_grouped_gemm_amd.profiling import kernel_source_hash
    if data.get("source_hash") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(key)
    return None if entry is None else entry.get("bytes_per_launch")


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

    def token_slice(self, i, T):
        n = self.tok.shape[0]
        o = (i * T) % (n - T + 1)
        return self.tok[o:o + T]


def graph_time(calls, reps: int, warm_reps: int) -> float:
    """Capture `calls` (zero-argument launchers) into one HIP graph, replay it `warm_reps` times
    untimed and `reps` times timed; return ms per call."""
    import torch
    for c in calls:             # eager pass: loads code objects, checks for errors
        c()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    for _ in range(warm_reps):
        g.replay()
    torch.cuda.synchronize()
    # replays run on the current stream; the events are recorded on that same stream
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(reps):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls))


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


# ----------------------------------------------------------------------------- sections
def decode_section(pool: Pool, T: int, steps: int, warmup: int):
    """Layer time at T tokens (all launches), then the dominant launch alone: phase 1 (top-k +
    gate/up of the selected experts) replayed on workspaces prepared by a full call."""
    import numpy as np
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.layers
    n = 2 * len(L)                      # calls per graph: each layer twice, new tokens each time
    out = torch.empty((T, s.H), dtype=torch.float32, device="cuda")
    ws = M.alloc_workspace(L[0], T)

    def call(i):
        x = pool.token_slice(i, T)
        return lambda: M.moe_layer_forward(L[i % len(L)], x, out, ws)

    reps, warm = max(1, math.ceil(steps / n)), max(1, math.ceil(warmup / n))
    ms = graph_time([call(i) for i in range(n)], reps, warm)

    # the dominant kernel, live: per-call workspaces hold the state phase 1 starts from
    states = []
    for i in range(n):
        layer, x = L[i % len(L)], pool.token_slice(i, T)
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
    kms = graph_time([(lambda st=st: M.moe_layer_forward_phase(st[0], st[1], out, st[2], 1))
                      for st in states], max(2, reps), 1)
    d_mean = float(np.mean(distinct))
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "steps": reps * n,
            "warmup": warm * n, "distinct_experts": d_mean,
            "layer_bytes": decode_layer_bytes(s, T, d_mean),
            "kernel": {"name": "k_dec_b (top-k + gate/up of the selected experts)",
                       "us": kms * 1e3, "bytes": kb}}


def prefill_section(pool: Pool, steps: int, skewed: bool):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.skew_layers if skewed else pool.layers
    T = T_PREFILL
    n = min(steps, len(L))
    ws = M.alloc_workspace(L[0], T)
    out = torch.empty((T, s.H), dtype=torch.float32, device="cuda")
    calls = [(lambda i=i: M.moe_layer_forward(L[i % len(L)], pool.prefill[i % 2], out, ws))
             for i in range(n)]
    reps = max(1, math.ceil(steps / n))
    ms = graph_time(calls, reps, 1)
    # the dominant kernel (phase 3: gate/up GEMM), on workspaces prepared by a full call
    nk = min(8, len(L))
    states = []
    for i in range(nk):
        wsi = M.alloc_workspace(L[i], T)
        M.moe_layer_forward(L[i], pool.prefill[i % 2], out, wsi)
        states.append((L[i], pool.prefill[i % 2], wsi))
    torch.cuda.synchronize()
    kms = graph_time([(lambda st=st: M.moe_layer_forward_phase(st[0], st[1], out, st[2], 3))
                      for st in states], 3, 1)
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "steps": reps * n,
            "kernel": {"name": "k_gemm_w4<gate_up> (grouped GEMM, SwiGLU epilogue)",
                       "us": kms * 1e3, "flops": gateup_flops(s, T)}}


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
    ms_step = graph_time([lambda: stack.forward(r1, x1, ws1)], DECODE_STEPS_STACK, 8)
    assert torch.isfinite(r1).all().item()
    return {"layers": len(pool.layers), "prefill_tokens": T_PREFILL, "chunk": CHUNK,
            "prefill_ms": prefill_ms, "prefill_tokens_per_s": T_PREFILL / (prefill_ms * 1e-3),
            "decode_steps": DECODE_STEPS_STACK, "decode_ms_per_token": ms_step,
            "decode_tokens_per_s": 1.0 / (ms_step * 1e-3),
            "decode_hbm_frac": len(pool.layers) * decode_layer_bytes(s, 1, s.K) / (ms_step * 1e-3)
            / 1e9 / HBM_PEAK_GBS}


def copy_section():
    """A plain 256 MiB device-to-device copy (calibrates FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {n} bytes 3 times")


def cpu_baseline(pool: Pool, budget_s: float):
    """The fp64 oracle on the host for T = 1 decode tokens of the same workload (layer 0),
    repeated until the time budget is used; tokens/s."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    n, t0 = 0, time.time()
    while n < 2 or time.time() - t0 < budget_s:
        O.layer_forward(pool.host0, pool.tok_host[n:n + 1], pool.shape.K, "bf16")
        n += 1
    dt = time.time() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode tokens (T=1) through layer 0 of the full-size layer, fp64 NumPy "
                      f"oracle, bf16 profile, {dt:.1f}s; BLAS={blas}, "
                      f"host cpus={len(os.sched_getaffinity(0))}"}


def roofline_hbm(k):
    ach = k["bytes"] / (k["us"] * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": k["name"], "achieved": ach, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "bytes_per_launch": k["bytes"],
            "avg_launch_us": k["us"]}


def roofline_mfma(k):
    ach = k["flops"] / (k["us"] * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": k["name"], "achieved": ach, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "flops_per_launch": k["flops"],
            "avg_launch_us": k["us"]}


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

    pool = Pool(N_LAYERS)
    s = pool.shape
    t_all = time.time()
    if args.only == "decode_t1":
        r = decode_section(pool, 1, args.steps, args.warmup)
        log(f"decode T=1: {r['ms_per_step'] * 1e3:.2f} us/layer; k_dec_b {r['kernel']['us']:.2f} us")
        return
    if args.only == "decode_t8":
        r = decode_section(pool, 8, args.steps // 2, args.warmup)
        log(f"decode T=8: {r['ms_per_step'] * 1e3:.2f} us/layer; k_dec_b {r['kernel']['us']:.2f} us")
        return
    if args.only in ("prefill_uniform", "prefill_skewed"):
        r = prefill_section(pool, args.prefill_steps, args.only == "prefill_skewed")
        log(f"{args.only}: {r['ms_per_step'] * 1e3:.1f} us/layer; gate/up {r['kernel']['us']:.1f} us")
        return
    if args.only == "stack":
        r = stack_section(pool)
        log(f"stack: {r}")
        return

    d1 = decode_section(pool, 1, args.steps, args.warmup)
    log(f"decode T=1: {d1['ms_per_step'] * 1e3:.2f} us/layer, {d1['tokens_per_s']:.0f} tok/s; "
        f"k_dec_b {d1['kernel']['us']:.2f} us for {d1['kernel']['bytes'] / 1e6:.2f} MB")
    d8 = decode_section(pool, 8, args.steps // 2, args.warmup)
    log(f"decode T=8: {d8['ms_per_step'] * 1e3:.2f} us/layer, {d8['tokens_per_s']:.0f} tok/s")
    prefill = {}
    for skewed in (False, True):
        tag = "skewed" if skewed else "uniform"
        p = prefill_section(pool, args.prefill_steps, skewed)
        fl = layer_flops(s, T_PREFILL)
        tf = fl / (p["ms_per_step"] * 1e-3) / 1e12
        rk = roofline_mfma(p["kernel"])
        rk["traffic"] = measured_traffic(f"gate_up@prefill_{tag}")
        prefill[tag] = {"value": p["tokens_per_s"], "unit": "tokens/s",
                        "ms_per_step": p["ms_per_step"], "steps": p["steps"],
                        "layer_tflops": tf, "layer_mfma_frac": tf / BF16_PEAK_TFLOPS,
                        "roofline": rk}
        log(f"prefill T=4096 {tag}: {p['ms_per_step'] * 1e3:.1f} us/layer "
            f"({p['tokens_per_s'] / 1e6:.2f} M tok/s, {tf:.0f} TFLOP/s); gate/up GEMM "
            f"{p['kernel']['us']:.1f} us = {rk['achieved']:.0f} TFLOP/s")
    st = stack_section(pool)
    log(f"stack ({st['layers']} layers): prefill {st['prefill_tokens_per_s']:.0f} tok/s, "
        f"decode {st['decode_tokens_per_s']:.0f} tok/s ({st['decode_ms_per_token'] * 1e3:.0f} us/token)")
    cpu = None if args.skip_cpu else cpu_baseline(pool, args.cpu_seconds)

    roof = roofline_hbm(d1["kernel"])
    roof["traffic"] = measured_traffic("k_dec_b@decode_t1")
    line = {
        "metric": METRIC,
        "value": d1["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": d1["steps"], "warmup": d1["warmup"], "ms_per_step": d1["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded: 4-bit g64 weights, x ~ N(0,1) bf16; no checkpoint)",
        "config": {"workload": "MoE layer, decode T=1 (batch 1): hidden 2048, 256 experts, top-8, "
                               "expert FFN 512, one shared expert FFN 512, 4-bit group-64 affine",
                   "layer_pool": N_LAYERS, "token_pool": int(pool.tok.shape[0])},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer_bytes_per_token": d1["layer_bytes"],
        "layer_hbm_frac": d1["layer_bytes"] / (d1["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "decode_t8": {"value": d8["tokens_per_s"], "unit": "tokens/s",
                      "ms_per_step": d8["ms_per_step"], "steps": d8["steps"],
                      "distinct_experts": d8["distinct_experts"],
                      "layer_hbm_frac": d8["layer_bytes"] / (d8["ms_per_step"] * 1e-3) / 1e9
                      / HBM_PEAK_GBS,
                      "roofline": roofline_hbm(d8["kernel"])},
        "prefill_t4096": prefill,
        "stack_40_layers": st,
        "source_hash": kernel_source_hash(),
    }
    log(f"timed sections took {time.time() - t_all:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
