#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X (tokens/s, and the fraction of the roofline).

    python bench.py [--gpus 1] [--steps 640] [--warmup 64]

Workload (seeded synthetic data, see the design doc for the recipe): the MoE layer of
Qwen3.6-35B-A3B -- hidden 2048, 256 experts, top-8, expert FFN 512, one shared expert with
FFN 512, 4-bit group-64 affine weights. A step is one full layer call (route, permute,
gate/up + SwiGLU, down + combine). The headline is batch-1 decode (T = 1); the same JSON line
also carries batch-8 decode and T = 4096 prefill (uniform and skewed routing).

Inputs are resident in HBM before timing starts. Consecutive steps rotate over a pool of
independently seeded layers (more bytes between two uses of one layer than the 256 MiB
Infinity Cache holds) and over a pool of tokens, so every step streams its weights from HBM.
Timed regions are HIP-graph replays bracketed by device synchronisation and HIP events on
the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
SHAPE_NAME = "full"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed decode steps (T=1 layer calls)")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--pool", type=int, default=20, help="distinct layers rotated through")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_grouped_gemm_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if absent or
    if the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(f"{kernel}@{workload}")
    return None if entry is None else entry.get("bytes_per_launch")


class Pool:
    """Device-resident layers and token pools."""

    def __init__(self, n_layers: int):
        import numpy as np
        import torch
        import synth
        from bit_grouped_gemm_amd import moe_w4 as M
        self.shape = synth.SHAPES[SHAPE_NAME]
        s = self.shape
        t0 = time.time()
        self.layers = []
        self.skew_layers = []
        for i in range(n_layers):
            host = synth.make_layer(s, seed=0, layer=i)
            dl = M.upload_layer(host, s.H, s.E, s.K, s.F, s.Fs)
            self.layers.append(dl)
            t = dict(dl.tensors)
            t["router_bias"] = torch.from_numpy(synth.skew_router_bias(s.E)).cuda()
            self.skew_layers.append(M.make_layer(t, s.H, s.E, s.K, s.F, s.Fs))
            if i == 0:
                self.host0 = host
            del host
        torch.cuda.synchronize()
        log(f"{n_layers} layers resident ({n_layers * 452984832 / 2**30:.1f} GiB of routed "
            f"weights) in {time.time() - t0:.1f}s")
        self.tok_host = synth.make_tokens(s, 1024, seed=0, stream=0)
        self.tok = torch.from_numpy(self.tok_host.view(np.int16)).cuda()
        self.prefill_host = [synth.make_tokens(s, 4096, seed=0, stream=10 + j) for j in range(2)]
        self.prefill = [torch.from_numpy(x.view(np.int16)).cuda() for x in self.prefill_host]


def graph_time(calls, reps: int, warm_reps: int) -> float:
    """Capture `calls` (a list of zero-argument launchers) into one HIP graph, replay it
    `warm_reps` times untimed and `reps` times timed; return ms per call."""
    import torch
    for c in calls:             # eager pass: loads code objects, checks for errors
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for _ in range(warm_reps):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls))


def decode_bench(pool: Pool, T: int, steps: int, warmup: int):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    L = pool.layers
    per_graph = 4 * len(L)              # each layer 4 times per replay, a new token each time
    reps = max(1, math.ceil(steps / per_graph))
    warm = max(1, math.ceil(warmup / per_graph))
    ws = M.alloc_workspace(L[0], T)
    out = torch.empty((T, pool.shape.H), dtype=torch.float32, device="cuda")
    ntok = pool.tok.shape[0]

    def call(i):
        x = pool.tok[(i * T) % ntok:(i * T) % ntok + T]
        return lambda: M.moe_layer_forward(L[i % len(L)], x, out, ws)

    ms = graph_time([call(i) for i in range(per_graph)], reps, warm)
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "steps": reps * per_graph, "warmup": warm * per_graph}


def decode_kernel_bench(pool: Pool, T: int, reps: int = 20):
    """Live timing of the dominant decode kernel (gate/up + SwiGLU GEMV, one launch per call)
    on prepared plans, and its algorithmic bytes per launch."""
    import numpy as np
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.layers
    n = 4 * len(L)
    states = []
    ntok = pool.tok.shape[0]
    for i in range(n):
        layer = L[i % len(L)]
        x = pool.tok[(i * T) % ntok:(i * T) % ntok + T]
        idx = torch.empty(T * s.K, dtype=torch.int32, device="cuda")
        w = torch.empty(T * s.K, dtype=torch.float32, device="cuda")
        sg = torch.empty(T, dtype=torch.float32, device="cuda")
        cnt = torch.empty(s.E, dtype=torch.int32, device="cuda")
        ws = M.alloc_workspace(layer, T)
        M.moe_route(layer, x, idx, w, sg, cnt, ws)
        plan = M.alloc_plan(layer, T)
        M.moe_permute(layer, idx, T, plan, ws)
        a = torch.empty(T * s.K * s.F + T * s.Fs, dtype=torch.int16, device="cuda")
        states.append((layer, x, plan, a, ws, cnt))
    torch.cuda.synchronize()
    distinct = [int((st[5] > 0).sum().item()) + 1 for st in states]       # + shared expert
    per_matrix = s.F * s.H // 2 + 2 * 2 * s.F * (s.H // 64)                # q + scale + bias
    bytes_per = float(np.mean([d * 2 * per_matrix for d in distinct]))
    bytes_per += T * s.H * 2 + (T * s.K + T) * s.F * 2                     # x in, A out

    def call(st):
        layer, x, plan, a, ws, _ = st
        return lambda: M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_GATE_UP, x, T, plan, None, None,
                                             a, ws)

    ms = graph_time([call(st) for st in states], reps, 2)
    return {"kernel": "k_dec_gateup", "ms": ms, "bytes": bytes_per,
            "distinct_experts": float(np.mean(distinct))}


def prefill_bench(pool: Pool, steps: int, skewed: bool):
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    L = pool.skew_layers if skewed else pool.layers
    T = 4096
    ws = M.alloc_workspace(L[0], T)
    out = torch.empty((T, pool.shape.H), dtype=torch.float32, device="cuda")
    n = min(steps, len(L))

    def call(i):
        return lambda: M.moe_layer_forward(L[i % len(L)], pool.prefill[i % 2], out, ws)

    reps = max(1, math.ceil(steps / n))
    ms = graph_time([call(i) for i in range(n)], reps, 1)
    return {"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "steps": reps * n}


def prefill_kernel_bench(pool: Pool, skewed: bool, reps: int = 5):
    """Live timing of the dominant prefill kernel (MFMA gate/up + SwiGLU grouped GEMM)."""
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    s = pool.shape
    L = pool.skew_layers if skewed else pool.layers
    T = 4096
    n = min(8, len(L))
    states = []
    for i in range(n):
        layer = L[i]
        x = pool.prefill[i % 2]
        idx = torch.empty(T * s.K, dtype=torch.int32, device="cuda")
        w = torch.empty(T * s.K, dtype=torch.float32, device="cuda")
        sg = torch.empty(T, dtype=torch.float32, device="cuda")
        cnt = torch.empty(s.E, dtype=torch.int32, device="cuda")
        ws = M.alloc_workspace(layer, T, M.MOE_FLAG_ATOMIC_COMBINE)
        M.moe_route(layer, x, idx, w, sg, cnt, ws)
        plan = M.alloc_plan(layer, T)
        M.moe_permute(layer, idx, T, plan, ws)
        a = torch.empty(T * s.K * s.F + T * s.Fs, dtype=torch.int16, device="cuda")
        states.append((layer, x, plan, a, ws))
    torch.cuda.synchronize()
    flops = 2.0 * s.H * 2 * s.F * T * s.K + 2.0 * s.H * 2 * s.Fs * T

    def call(st):
        layer, x, plan, a, ws = st
        return lambda: M.moe_grouped_gemm_w4(layer, M.MOE_GEMM_GATE_UP, x, T, plan, None, None,
                                             a, ws)

    ms = graph_time([call(st) for st in states], reps, 1)
    return {"kernel": "k_gemm_w4<gate_up>", "ms": ms, "flops": flops}


def layer_flops(s, T):
    """Algorithmic flops of one layer call: router, gate/up, down (shared expert included)."""
    return (2.0 * T * s.H * s.E + 2.0 * T * s.K * s.H * 2 * s.F + 2.0 * T * s.K * s.F * s.H
            + 2.0 * T * s.H * 2 * s.Fs + 2.0 * T * s.Fs * s.H)


def decode_layer_bytes(s, T, distinct):
    """Algorithmic HBM bytes of one decode call: each selected expert's weights once, the
    shared expert, router and gate weights, the tokens and the output."""
    per_expert = 3 * (s.F * s.H // 2 + 4 * s.F * (s.H // 64))
    return (distinct + 1) * per_expert + s.E * s.H * 4 + s.H * 4 + T * s.H * 2 + T * s.H * 4


def cpu_baseline(pool: Pool, budget_s: float):
    """The fp64 oracle on the host for T = 1 decode tokens of the same workload (layer 0),
    repeated until the time budget is used; tokens/s."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    n, t0 = 0, time.time()
    while n < 2 or time.time() - t0 < budget_s:
        O.layer_forward(pool.host0, pool.tok_host[n:n + 1], pool.shape.K, "bf16")
        n += 1
    dt = time.time() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode tokens (T=1) through layer 0, fp64 NumPy oracle, bf16 profile, "
                      f"{dt:.1f}s; BLAS={blas}, host cpus={len(os.sched_getaffinity(0))}"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the MoE layer is not "
                                   "sharded (see DESIGN.md for how it would shard); use --gpus 1"}))
        sys.exit(2)
    import torch
    from bit_grouped_gemm_amd import moe_w4 as M
    M.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    log(f"device {torch.cuda.get_device_name(0)}, {M.moe_version()}")

    pool = Pool(args.pool)
    s = pool.shape
    torch.cuda.synchronize()
    t_all = time.time()

    d1 = decode_bench(pool, 1, args.steps, args.warmup)
    log(f"decode T=1: {d1['ms_per_step'] * 1e3:.2f} us/layer, {d1['tokens_per_s']:.0f} tok/s")
    k1 = decode_kernel_bench(pool, 1)
    log(f"  dominant kernel {k1['kernel']}: {k1['ms'] * 1e3:.2f} us, {k1['bytes'] / 1e6:.2f} MB")
    d8 = decode_bench(pool, 8, args.steps // 2, args.warmup)
    k8 = decode_kernel_bench(pool, 8)
    log(f"decode T=8: {d8['ms_per_step'] * 1e3:.2f} us/layer, {d8['tokens_per_s']:.0f} tok/s")

    prefill = {}
    if not args.skip_prefill:
        for skewed in (False, True):
            tag = "skewed" if skewed else "uniform"
            p = prefill_bench(pool, args.prefill_steps, skewed)
            k = prefill_kernel_bench(pool, skewed)
            fl = layer_flops(s, 4096)
            tf = fl / (p["ms_per_step"] * 1e-3) / 1e12
            ktf = k["flops"] / (k["ms"] * 1e-3) / 1e12
            prefill[tag] = {
                "value": p["tokens_per_s"], "unit": "tokens/s", "ms_per_step": p["ms_per_step"],
                "steps": p["steps"], "layer_tflops": tf, "layer_mfma_frac": tf / BF16_PEAK_TFLOPS,
                "roofline": {"bound": "mfma", "kernel": k["kernel"], "achieved": ktf,
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": ktf / BF16_PEAK_TFLOPS,
                             "traffic": measured_traffic(k["kernel"], f"prefill_{tag}"),
                             "flops_per_launch": k["flops"], "avg_launch_us": k["ms"] * 1e3}}
            log(f"prefill T=4096 {tag}: {p['ms_per_step'] * 1e3:.1f} us/layer "
                f"({p['tokens_per_s'] / 1e6:.2f} M tok/s, {tf:.0f} TFLOP/s); gate/up kernel "
                f"{k['ms'] * 1e3:.1f} us = {ktf:.0f} TFLOP/s")

    cpu = None if args.skip_cpu else cpu_baseline(pool, args.cpu_seconds)

    ach = k1["bytes"] / (k1["ms"] * 1e-3) / 1e9
    lb1 = decode_layer_bytes(s, 1, s.K)
    lb8 = decode_layer_bytes(s, 8, k8["distinct_experts"] - 1)
    line = {
        "metric": "MoE-layer tokens/s at T=1 and T=4096; % HBM-BW / % bf16 MFMA peak",
        "value": d1["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": d1["steps"], "warmup": d1["warmup"], "ms_per_step": d1["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; 4-bit g64 weights, x ~ N(0,1) bf16)",
        "config": {"workload": "MoE layer decode T=1 (batch 1): hidden 2048, 256 experts, top-8, "
                               "expert FFN 512, shared expert FFN 512, 4-bit group-64 affine",
                   "layer_pool": args.pool, "token_pool": int(pool.tok.shape[0])},
        "roofline": {"bound": "hbm", "kernel": k1["kernel"], "achieved": ach,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": measured_traffic(k1["kernel"], "decode_t1"),
                     "bytes_per_launch": k1["bytes"], "avg_launch_us": k1["ms"] * 1e3},
        "cpu_baseline": cpu,
        "layer_bytes_per_token": lb1,
        "layer_hbm_frac": lb1 / (d1["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "decode_t8": {"value": d8["tokens_per_s"], "unit": "tokens/s",
                      "ms_per_step": d8["ms_per_step"], "steps": d8["steps"],
                      "distinct_experts": k8["distinct_experts"] - 1,
                      "layer_hbm_frac": lb8 / (d8["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "gateup_kernel_us": k8["ms"] * 1e3,
                      "gateup_kernel_gbs": k8["bytes"] / (k8["ms"] * 1e-3) / 1e9},
        "prefill_t4096": prefill,
        "source_hash": kernel_source_hash(),
    }
    log(f"timed sections took {time.time() - t_all:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
