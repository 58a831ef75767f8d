"""Host-side tools on the CPU: the rocprofv3 CSV summaries behind the bench line's roofline and
traffic figures, and bench.py's single-GPU rule."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp",
                                          "Grid_Size_X", "Workgroup_Size_X"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow({"Grid_Size": 256, **r})


def test_short_name_drops_arguments_not_template_parameters():
    from bit_grouped_gemm_amd.profiling import short_name
    assert short_name("void moe::k_dec_b<1, 4>(moe::DecodeArgs)") == "moe::k_dec_b<1, 4>"
    assert short_name("moe::k_scan(int*, int)") == "moe::k_scan"


def test_kernel_stats_groups_by_name_and_grid(tmp_path):
    from bit_grouped_gemm_amd.profiling import kernel_stats
    d = str(tmp_path / "trace")
    _write_trace(d, [
        # two launches of one kernel on 4 workgroups: 2 us and 4 us
        {"Kernel_Name": "k_a(int)", "Start_Timestamp": 0, "End_Timestamp": 2000,
         "Grid_Size_X": 1024, "Workgroup_Size_X": 256},
        {"Kernel_Name": "k_a(int)", "Start_Timestamp": 5000, "End_Timestamp": 9000,
         "Grid_Size_X": 1024, "Workgroup_Size_X": 256},
        # the same kernel on another grid is a separate line
        {"Kernel_Name": "k_a(int)", "Start_Timestamp": 0, "End_Timestamp": 10000,
         "Grid_Size_X": 256, "Workgroup_Size_X": 256},
    ])
    st = kernel_stats(d)
    by = {(r["kernel"], r["grid"][0]): r for r in st}
    a4 = by[("k_a", 4)]
    assert a4["calls"] == 2 and a4["avg_us"] == pytest.approx(3.0)
    assert a4["min_us"] == pytest.approx(2.0) and a4["max_us"] == pytest.approx(4.0)
    a1 = by[("k_a", 1)]
    assert a1["calls"] == 1 and a1["avg_us"] == pytest.approx(10.0)
    assert sum(r["total_pct"] for r in st) == pytest.approx(100.0)
    assert st[0]["kernel"] == "k_a" and st[0]["grid"][0] == 1  # sorted by total time


def test_traffic_scales_counters_by_the_copy_calibration(tmp_path):
    """HBM bytes per launch = FETCH/fetch_factor + WRITE/write_factor, the factors taken from a
    plain copy of a known size."""
    from bit_grouped_gemm_amd import profiling as P
    n = 1 << 20  # copy size in bytes
    _write_counters(str(tmp_path / "cf"), [{"Kernel_Name": "copyBuffer", "Counter_Name": "FETCH_SIZE",
                                            "Counter_Value": n / 1024 * 0.5}])
    _write_counters(str(tmp_path / "cw"), [{"Kernel_Name": "copyBuffer", "Counter_Name": "WRITE_SIZE",
                                            "Counter_Value": n / 1024}])
    _write_counters(str(tmp_path / "f"), [
        {"Kernel_Name": "void moe::k_x<1>(A)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": "void moe::k_x<1>(A)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
        {"Kernel_Name": "void moe::k_x<1>(A)", "Grid_Size": 512, "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 900.0},
        {"Kernel_Name": "void moe::k_y(A)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 7.0}])
    _write_counters(str(tmp_path / "w"), [
        {"Kernel_Name": "void moe::k_x<1>(A)", "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
        {"Kernel_Name": "void moe::k_x<1>(A)", "Grid_Size": 512, "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 30.0}])
    out = str(tmp_path / "traffic.json")

    class Args:
        pass
    a = Args()
    a.copy_fetch, a.copy_write = str(tmp_path / "cf"), str(tmp_path / "cw")
    a.fetch, a.write = str(tmp_path / "f"), str(tmp_path / "w")
    a.copy_bytes, a.kernel, a.key, a.out, a.grid = n, r"k_x<1>", "x", out, 256
    P.update_traffic(a)
    a.grid, a.key = 512, "x512"
    P.update_traffic(a)
    data = json.load(open(out))
    assert data["copy_calibration"]["fetch_factor"] == pytest.approx(0.5)
    assert data["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    e = data["kernels"]["x"]
    assert e["dispatches"] == [2, 1]
    # mean FETCH 200 KiB / 0.5 + WRITE 10 KiB / 1.0
    assert e["bytes_per_launch"] == pytest.approx((200.0 / 0.5 + 10.0) * 1024)
    assert data["kernels"]["x512"]["bytes_per_launch"] == pytest.approx((900.0 / 0.5 + 30.0) * 1024)
    # the figure is tied to the hash of the sources it was taken on
    assert e["source_hash"] == P.kernel_source_hash(e["sources"])
    assert P.traffic_entry(out, "x") == pytest.approx(e["bytes_per_launch"])
    e["source_hash"] = "0" * 16
    json.dump(data, open(out, "w"))
    assert P.traffic_entry(out, "x") is None and P.traffic_entry(out, "absent") is None


def test_kernel_sources_name_the_defining_file_and_the_headers():
    from bit_grouped_gemm_amd.profiling import kernel_sources
    src = kernel_sources("k_dec_b<1, 4>")
    assert "decode.hip" in src and "moe_internal.h" in src and "attn.hip" not in src
    assert "attn.hip" in kernel_sources("k_attn_split<128, 8>")


def test_kernel_source_hash_is_stable():
    from bit_grouped_gemm_amd.profiling import kernel_source_hash
    h = kernel_source_hash()
    assert h == kernel_source_hash() and len(h) == 16


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
