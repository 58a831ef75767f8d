"""Summaries of rocprofv3 CSV output (``--output-format csv``): per-kernel launch statistics and
HBM traffic per launch from the FETCH_SIZE / WRITE_SIZE counters.

    python -m bit_grouped_gemm_amd.profiling stats TRACE_DIR --cmd "COMMAND" --out FILE.md
    python -m bit_grouped_gemm_amd.profiling traffic --fetch DIR --write DIR \
        --copy-fetch DIR --copy-write DIR --copy-bytes N --kernel REGEX [--grid N] --key NAME \
        --out profiles/traffic.json
    python -m bit_grouped_gemm_amd.profiling counters PMC_DIR --cmd "COMMAND" --out FILE.md

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch. They count what the L2 requests
from the memory fabric, so each is divided by the ratio it shows on a plain device copy of a
known size (the copy-calibration runs) before it is taken as HBM bytes. The same calibration
run also holds a read-only reduction over the same bytes; its FETCH_SIZE ratio is stored beside
the copy's as a cross-check of the factor.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
from collections import OrderedDict

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash(files=None) -> str:
    """Hash of HIP sources (all of csrc by default, else the named files of csrc); a traffic
    figure is valid only for the sources it was taken on."""
    h = hashlib.sha256()
    d = os.path.join(PKG, "csrc")
    for f in sorted(files if files is not None else os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def kernel_sources(kernel_regex: str):
    """The csrc files a kernel's code can come from: the sources that name its identifier (the
    leading name of the regex) plus every header of csrc."""
    m = re.match(r"[A-Za-z_]\w*", kernel_regex)
    if not m:
        raise ValueError(f"no kernel name at the start of /{kernel_regex}/")
    d = os.path.join(PKG, "csrc")
    out = []
    for f in sorted(os.listdir(d)):
        text = open(os.path.join(d, f), encoding="utf-8", errors="replace").read()
        if f.endswith(".h") or re.search(r"\b" + m.group(0) + r"\b", text):
            out.append(f)
    return out


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def short_name(name: str) -> str:
    """Kernel name without its argument list."""
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("void ", "").strip()


def kernel_stats(trace_dir: str):
    """Per kernel (by short name and grid): launches, mean/min/max duration in microseconds."""
    rows = list(csv.DictReader(open(_find(trace_dir, "_kernel_trace.csv"))))
    agg: "OrderedDict[str, list]" = OrderedDict()
    for r in rows:
        key = short_name(r["Kernel_Name"])
        grid = tuple(int(r.get(f"Grid_Size_{a}", 1) or 1) // max(1, int(r.get(f"Workgroup_Size_{a}", 1) or 1))
                     for a in "XYZ")
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault((key, grid), []).append(d)
    total = sum(sum(v) for v in agg.values())
    out = []
    for (k, g), v in agg.items():
        out.append({"kernel": k, "grid": g, "calls": len(v), "avg_us": statistics.fmean(v),
                    "min_us": min(v), "max_us": max(v), "total_pct": 100.0 * sum(v) / total})
    out.sort(key=lambda r: -r["avg_us"] * r["calls"])
    return out


def write_stats_md(trace_dir: str, cmd: str, out: str, title: str, top: int = 25):
    st = kernel_stats(trace_dir)
    lines = [f"# {title}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
             "| kernel | workgroups | launches | avg us | min us | max us | % of kernel time |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for r in st[:top]:
        g = "x".join(str(x) for x in r["grid"] if x > 1) or "1"
        lines.append(f"| `{r['kernel']}` | {g} | {r['calls']} | {r['avg_us']:.2f} | "
                     f"{r['min_us']:.2f} | {r['max_us']:.2f} | {r['total_pct']:.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return st


def counter_per_dispatch(pmc_dir: str, counter: str, kernel_regex: str, grid=None):
    """Values of one counter for every dispatch whose kernel name matches (and whose grid, in
    work-items, equals `grid` when given)."""
    rx = re.compile(kernel_regex)
    vals = []
    for r in csv.DictReader(open(_find(pmc_dir, "_counter_collection.csv"))):
        if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"]):
            if grid is None or int(r["Grid_Size"]) == int(grid):
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} rows for /{kernel_regex}/ (grid {grid}) in {pmc_dir}")
    return vals


def copy_factor(pmc_dir: str, counter: str, nbytes: int, kernel_regex: str = "copyBuffer"):
    """Counter KiB per byte actually moved, from the largest dispatches of a plain copy."""
    vals = sorted(counter_per_dispatch(pmc_dir, counter, kernel_regex))
    big = [v for v in vals if v >= 0.5 * vals[-1]]
    return statistics.fmean(big) * 1024.0 / nbytes, len(big)


def update_traffic(args):
    ff, nf = copy_factor(args.copy_fetch, "FETCH_SIZE", args.copy_bytes)
    fw, nw = copy_factor(args.copy_write, "WRITE_SIZE", args.copy_bytes)
    try:   # the read-only reduction of the calibration run (absent in older runs)
        fr, _ = copy_factor(args.copy_fetch, "FETCH_SIZE", args.copy_bytes, "reduce")
    except ValueError:
        fr = None
    grid = getattr(args, "grid", None)
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel, grid)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel, grid)
    data = {"kernels": {}}
    if os.path.exists(args.out):
        data = json.load(open(args.out))
    data.pop("source_hash", None)   # figures carry the hash of their own sources
    data["copy_calibration"] = {"bytes": args.copy_bytes, "fetch_factor": ff, "write_factor": fw,
                                "dispatches": [nf, nw], "read_only_fetch_factor": fr}
    fk, wk = statistics.fmean(fetch), statistics.fmean(write)
    srcs = kernel_sources(args.kernel)
    data.setdefault("kernels", {})[args.key] = {
        "kernel_regex": args.kernel, "grid": grid, "dispatches": [len(fetch), len(write)],
        "fetch_kib": fk, "write_kib": wk,
        "bytes_per_launch": (fk / ff + wk / fw) * 1024.0,
        "sources": srcs, "source_hash": kernel_source_hash(srcs),
        "fetch_dirs": [args.fetch, args.write]}
    with open(args.out, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(data["kernels"][args.key]))


def traffic_entry(path: str, key: str):
    """HBM bytes per launch stored under `key`, or None if absent or taken on other sources."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entry = json.load(f).get("kernels", {}).get(key)
    if entry is None or "sources" not in entry:
        return None
    try:
        if kernel_source_hash(entry["sources"]) != entry["source_hash"]:
            return None
    except FileNotFoundError:
        return None
    return entry["bytes_per_launch"]


def counter_table(pmc_dir: str):
    """Mean value per dispatch of every counter, per kernel (short name): {kernel: {counter: (n, mean)}}."""
    agg: "OrderedDict[str, dict]" = OrderedDict()
    for r in csv.DictReader(open(_find(pmc_dir, "_counter_collection.csv"))):
        k = short_name(r["Kernel_Name"])
        agg.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return OrderedDict((k, {c: (len(v), statistics.fmean(v)) for c, v in cs.items()})
                       for k, cs in agg.items())


def write_counters_md(pmc_dir: str, cmd: str, out: str, title: str, top: int = 20):
    tab = counter_table(pmc_dir)
    names = sorted({c for cs in tab.values() for c in cs})
    lines = [f"# {title}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
             "Mean per dispatch (counters summed over the chip).", "",
             "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---:|" + "---:|" * len(names)]
    rows = sorted(tab.items(), key=lambda kv: -max(v[1] for v in kv[1].values()))[:top]
    for k, cs in rows:
        n = max(v[0] for v in cs.values())
        vals = " | ".join(f"{cs[c][1]:.3g}" if c in cs else "" for c in names)
        lines.append(f"| `{k}` | {n} | {vals} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return tab


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="rocprofv3 kernel trace")
    s.add_argument("--top", type=int, default=25, help="kernels listed, by total time")
    t = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "key", "out"):
        t.add_argument("--" + a.replace("_", "-"), dest=a, required=True)
    t.add_argument("--copy-bytes", dest="copy_bytes", type=int, default=256 << 20)
    t.add_argument("--grid", type=int, default=None, help="only dispatches of this many work-items")
    c = sub.add_parser("counters")
    c.add_argument("pmc_dir")
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    args = ap.parse_args()
    if args.action == "counters":
        for k, cs in list(write_counters_md(args.pmc_dir, args.cmd, args.out, args.title).items())[:12]:
            print(k[:60], {c: round(v[1], 1) for c, v in cs.items()})
        return
    if args.action == "stats":
        for r in write_stats_md(args.trace_dir, args.cmd, args.out, args.title, args.top)[:12]:
            print(f"{r['kernel'][:60]:60s} {r['calls']:6d} {r['avg_us']:9.2f}")
    else:
        update_traffic(args)


if __name__ == "__main__":
    main()
