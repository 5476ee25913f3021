"""bench.py's contract: one GPU only, the JSON line's fields, the traffic
lookup that ties a counter summary to the kernel source it was taken on, and
the CPU-oracle baseline."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_is_read_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    src_rel = bench.KERNEL_SOURCES["share"]
    src = tmp_path / src_rel
    src.parent.mkdir(parents=True)
    src.write_bytes(b"kernel source v1")
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "traffic_reduce_w8_bs16384_h8192_mx_e4m3_bf16.txt"
    digest = hashlib.sha256(b"kernel source v1").hexdigest()
    summary.write_text(f"# header\nkernel_source_sha256: {digest}\nhbm_bytes_per_launch: 177272000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("w8_bs16384_h8192_mx_e4m3_bf16", "share") == 177272000
    assert bench.read_traffic("w8_bs65536_h5120_mx_e5m2_f32", "share") is None  # no summary
    src.write_bytes(b"kernel source v2")  # the kernel changed since the counters were taken
    assert bench.read_traffic("w8_bs16384_h8192_mx_e4m3_bf16", "share") is None


def test_cpu_baseline_fields():
    wl = workloads.WORKLOADS["w2_bs32_h1024_int8_f32"]
    xs, ss = workloads.generate(wl)
    cb = bench.cpu_baseline(wl, xs, ss, min_seconds=0.0, min_reps=3)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["value"] > 0 and cb["unit"] == "GB/s" and cb["cores"] == 1 and cb["kind"] == "oracle"


def test_cpu_baseline_all_cores_fields():
    wl = workloads.WORKLOADS["w2_bs32_h1024_int8_f32"]
    xs, ss = workloads.generate(wl)
    cb = bench.cpu_baseline_all_cores(wl, xs, ss, min_seconds=0.0, min_reps=3, block_rows=4)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["value"] > 0 and cb["unit"] == "GB/s" and 1 <= cb["cores"] <= 16 and cb["kind"] == "oracle"


@pytest.mark.parametrize("name", ["w2_bs32_h1024_int8_f32", "w8_bs16384_h8192_mx_e4m3_bf16"])
def test_oracle_row_blocks_concatenate_to_the_whole_share(name):
    """The all-cores baseline runs the oracle on row blocks: that is the same
    work only if the blocks' results, stacked, are the whole share's."""
    import numpy as np

    import oracle

    wl = workloads.WORKLOADS[name]
    wl = wl.with_(bs=wl.world_size * min(wl.rows, 12))
    xs, ss = workloads.generate(wl)
    whole = oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
    parts = [oracle.reduce_scatter_share([x[s:s + 5] for x in xs], [c[s:s + 5] for c in ss], wl.x_format,
                                         wl.scale_layout, wl.out_dtype) for s in range(0, wl.rows, 5)]
    assert np.array_equal(np.concatenate(parts).view(np.uint8), whole.view(np.uint8))


@pytest.mark.gpu
@pytest.mark.parametrize("op", ["share", "strided", "all_shares", "quantize"])
def test_json_line(gpu, op):
    wl = "w4_bs4096_h4096_e4m3_bf16"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--op", op, "--workload", wl, "--steps",
                          "20", "--warmup", "10", "--no-cpu-baseline", "--no-largest"], capture_output=True, text=True,
                         timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, "exactly one line on stdout"
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 10
    assert d["value"] > 0 and d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["cpu_baseline"] is None
    assert d["cpu_baseline_all_cores"] is None and d["hot"] is None and d["overlap_2streams"] is None
    m = d["device_memory"]
    assert m is not None and m["memory_bus_width_bits"] > 0 and m["memory_clock_khz"] > 0
    c = d["copy_calibration"]
    assert c["GBps"] > 0 and abs(c["GBps"] - c["bytes_moved"] / c["us"] / 1e3) < 0.01 * c["GBps"]
    assert d["config"]["workload"].startswith(wl) and d["config"]["op"] == op
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert "traffic" in r and 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert d["largest_workload"] is None
    assert d["dtype"] == "f32" and set(d["config"]["element_types"]) >= {"scales"}


@pytest.mark.gpu
def test_largest_workload_is_timed_beside_the_headline(gpu):
    """The default share run also times the largest workload (W=8,
    BS=65536, H=5120) and reports it under its own key."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "w4_bs4096_h4096_e4m3_bf16",
                          "--steps", "20", "--warmup", "5", "--no-cpu-baseline"], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    d = json.loads([ln for ln in res.stdout.splitlines() if ln.strip()][0])
    big = d["largest_workload"]
    wl = workloads.WORKLOADS[bench.LARGEST]
    assert big["workload"].startswith(bench.LARGEST)
    assert big["algorithmic_bytes_per_step"] == wl.algorithmic_bytes() and big["steps"] == 20
    assert big["kernel_us_avg"] > 0 and big["unit"] == "GB/s"
    assert abs(big["achieved"] - big["algorithmic_bytes_per_step"] / big["kernel_us_avg"] / 1e3) < 1e-3 * big["achieved"]
    assert abs(big["frac"] - big["achieved"] / 8000.0) < 1e-3 and 0 < big["frac"] < 1
    assert 0 < big["value"] <= big["achieved"] * 1.001
    assert d["config"]["workload"].startswith("w4_bs4096_h4096_e4m3_bf16")


@pytest.mark.gpu
@pytest.mark.parametrize("op", ["share", "strided", "all_shares", "quantize"])
def test_overlap_context(gpu, op):
    """--overlap adds a context figure and leaves the rest of the line as it is."""
    wl = "w4_bs4096_h4096_e4m3_bf16"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--op", op, "--workload", wl, "--steps",
                          "20", "--warmup", "10", "--no-cpu-baseline", "--overlap", "--no-largest"], capture_output=True,
                         text=True,
                         timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    d = json.loads([ln for ln in res.stdout.splitlines() if ln.strip()][0])
    o = d["overlap_2streams"]
    assert o["us_per_step"] > 0 and o["sets_per_stream"] >= 1
    assert abs(o["GBps"] - d["config"]["algorithmic_bytes_per_step"] / o["us_per_step"] / 1e3) < 0.01 * o["GBps"]
    assert d["value"] > 0 and d["roofline"]["kernel_us_avg"] > 0


def test_fit_fixed_and_rate_recovers_a_line():
    """The size sweep's fit: points on time = 2.5 us + bytes / 6.5 TB/s give
    back both numbers."""
    pts = [(b, 2.5e-6 + b / 6.5e12) for b in (1.0e7, 4.3e7, 1.7e8, 6.9e8)]
    fixed_us, gbps = bench.fit_fixed_and_rate(pts)
    assert abs(fixed_us - 2.5) < 1e-6 and abs(gbps - 6500.0) < 1e-6


@pytest.mark.gpu
def test_size_sweep_context(gpu):
    """--size-sweep's points: the share kernel and the stream copy timed at
    each size, times growing with the bytes, and the fit over them."""
    import argparse

    import torch

    import quantized_collective_reduction_amd as qrs

    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"]
    args = argparse.Namespace(steps=50, layout="pitched")
    rows = (1024, 2048, 4096)  # device-bound sizes: each launch outlasts its enqueue
    d = bench.size_sweep(wl, args, dev, qrs, workloads, torch, sweep_rows=rows)
    assert [p["rows_per_slice"] for p in d["points"]] == list(rows)
    assert [p["bytes"] for p in d["points"]] == [wl.with_(bs=r * 8).algorithmic_bytes() for r in rows]
    for a, b in zip(d["points"], d["points"][1:]):
        assert b["kernel_us"] > a["kernel_us"] and b["copy_us"] > a["copy_us"]
    for k in ("kernel", "copy"):
        assert d["fit"][k]["GBps"] > 0 and d["fit"][k]["fixed_us"] > 0
