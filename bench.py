"""Benchmark: achieved HBM bandwidth of one GPU's share of the quantized
reduce-scatter (dequant + rank-ordered reduce) on MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--op OP] [--layout L]
                    [--hot] [--overlap] [--size-sweep] [--no-cpu-baseline] [--no-largest]
                    [--gpus 1]

A step is one launch of the whole hot path (decode, scale, rank-ordered fp32
fold, convert, store) over one batch: W rank slices of the workload, already
resident in HBM, placed in one buffer at the pitch qrs_slice_pitch recommends
(--layout). Several identical input/output sets are allocated and the steps
rotate through them, so the working set of consecutive steps (well over the
256 MB Infinity Cache) is not served from that cache.

Prints ONE JSON line on stdout:
  value            whole-job throughput: algorithmic bytes x K / wall time of
                   the K timed steps (GB/s);
  roofline         for the reduce kernel: algorithmic bytes per launch /
                   average launch duration (HIP events recorded on the launch
                   stream at both ends of the K timed launches, divided by
                   K), against the 8 TB/s HBM peak. For --op all_shares one
                   step is one qrs_run_all_shares call: one launch, or W
                   (one per share) for uncapped layouts past about 300 MB per
                   share, so kernel_us_avg is per call;
                   traffic = measured HBM bytes per launch from committed
                   rocprofv3 counter summaries, when they match this kernel
                   source (else null);
  cpu_baseline     the CPU oracle timed on the host (single thread) on the
                   same workload;
  cpu_baseline_all_cores
                   the same oracle calls on row blocks of the share, spread
                   over the host's cores (at most 16 threads; the result does
                   not depend on the blocking);
  device_memory    the HBM bus width and memory clock the HIP runtime
                   reports, and the peak they imply, beside the published
                   8 TB/s that roofline.peak uses;
  copy_calibration the plain 16-byte stream copy of the same bytes, timed the
                   same way as the steps (rotating buffers, back to back);
  hot              with --hot, context only: K more launches on one
                   input/output set (no rotation, so a working set under
                   256 MB may be served from the Infinity Cache); else null;
  overlap_2streams with --overlap, context only: K more steps alternated
                   over two streams of the default priority (independent
                   batches, each stream on its own rotating sets), wall
                   time per step; else null.
  size_sweep       with --size-sweep (--op share), context only: the share
                   kernel and the stream copy timed at 1024 to 8192 rows per
                   slice of the workload's W, H and types (events over
                   back-to-back rotating launches, like the steps), and the
                   least-squares fit time = fixed + bytes / rate of each;
                   else null.
  largest_workload with --op share (the default), unless --no-largest: the
                   largest workload (W=8, BS=65536, H=5120, MX E5M2 -> fp32)
                   timed the same way in the same run, after the headline
                   workload's buffers are freed (W warm-up launches, K timed
                   launches between HIP events, wall clock around them):
                   kernel_us_avg, achieved GB/s and frac of the 8 TB/s peak,
                   and its whole-run GB/s; no CPU leg. Null when the
                   headline workload is itself that one.
Diagnostics go to stderr.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "achieved HBM GB/s and % of peak for dequant+reduce at W=8, H=8192"
# Source file of the kernel each op times (a traffic summary is valid only
# for the source it was measured on).
KERNEL_SOURCES = {
    "share": "quantized_collective_reduction_amd/csrc/qrs_kernels.hip",
    "strided": "quantized_collective_reduction_amd/csrc/qrs_kernels.hip",
    "all_shares": "quantized_collective_reduction_amd/csrc/qrs_kernels.hip",
    "quantize": "quantized_collective_reduction_amd/csrc/qrs_quantize.hip",
}
MALL_BYTES = 256 << 20


def workloads_names():
    import workloads

    return workloads.WORKLOADS.keys()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest(op):
    with open(os.path.join(ROOT, KERNEL_SOURCES[op]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic(workload_name, op):
    """HBM bytes per launch from profiles/traffic_<op>_<workload>.txt, if
    that summary was taken on the current kernel source; else None."""
    stem = "reduce" if op == "share" else op
    path = os.path.join(ROOT, "profiles", f"traffic_{stem}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest(op):
        log(f"[bench] {path} was taken on another kernel source: traffic = null")
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, xs, ss, min_seconds=10.0, min_reps=3):
    """Time the oracle (as it stands) on the host, single-threaded."""
    import oracle

    times = []
    t_start = time.perf_counter()
    while len(times) < min_reps or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    med = statistics.median(times)
    return {
        "value": round(wl.algorithmic_bytes() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole {wl.name} share ({wl.rows}x{wl.h} outputs from {wl.world_size} rank slices), "
                  f"median of {len(times)} runs, {med:.3f} s each, numpy single thread on {host_cpu_model()}",
    }


def _host_threads():
    """Host cores this process may use, at most 16 (the host CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_all_cores(wl, xs, ss, min_seconds=5.0, min_reps=3, block_rows=64):
    """Time the oracle over row blocks of the share on a thread pool: the
    oracle computes every output element from its own row only, so the blocks
    are independent (numpy releases the GIL inside its array operations)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    workers = _host_threads()
    starts = range(0, wl.rows, block_rows)

    def block(s):
        return oracle.reduce_scatter_share([x[s:s + block_rows] for x in xs], [c[s:s + block_rows] for c in ss],
                                           wl.x_format, wl.scale_layout, wl.out_dtype)

    times = []
    with ThreadPoolExecutor(workers) as ex:
        t_start = time.perf_counter()
        while len(times) < min_reps or time.perf_counter() - t_start < min_seconds:
            t0 = time.perf_counter()
            list(ex.map(block, starts))
            times.append(time.perf_counter() - t0)
            if len(times) >= 50:
                break
    med = statistics.median(times)
    return {
        "value": round(wl.algorithmic_bytes() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"whole {wl.name} share in {block_rows}-row blocks on {workers} threads, "
                  f"median of {len(times)} runs, {med:.3f} s each, on {host_cpu_model()}",
    }


def device_memory_props():
    """The HBM figures the HIP runtime reports for device 0 (memory clock in
    kHz, bus width in bits) and the peak they imply, next to the published
    8 TB/s used for the roofline. The runtime reports HBM3E's memory clock as
    a quarter of the per-pin data rate (2 GHz on MI355X, whose pins run at
    8 Gb/s), so the implied peak is bus bytes x clock x 4. Read with
    hipDeviceGetAttribute from the HIP runtime torch has loaded."""
    import ctypes

    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        return None
    hip = ctypes.CDLL(path)
    attr_bus_width, attr_mem_clock = 59, 60  # hipDeviceAttributeMemoryBusWidth, ...MemoryClockRate
    vals = {}
    for name, attr in (("memory_bus_width_bits", attr_bus_width), ("memory_clock_khz", attr_mem_clock)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) != 0:
            return None
        vals[name] = v.value
    vals["hbm_gbps_implied"] = round(vals["memory_bus_width_bits"] / 8 * vals["memory_clock_khz"] * 1e3 * 4 / 1e9, 1)
    vals["hbm_gbps_published"] = HBM_PEAK_GBPS
    return vals


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def place_inputs(p, xs, ss, dev, qrs, torch, layout, full_inputs=False):
    """Device copies of the W rank inputs in the requested placement:
    "pitched" - one x buffer and one scale buffer, slices at the pitch
                qrs_slice_pitch recommends (the default);
    "packed"  - one [W, rows, H] x buffer and one scale buffer, slices back
                to back;
    "separate" - one allocation per slice."""
    if layout == "pitched":
        dx, ds = qrs.alloc_slices(p, device=dev, full_inputs=full_inputs)
        for t, a in zip(dx, xs):
            t.copy_(torch.from_numpy(a))
        for t, a in zip(ds, ss):
            t.copy_(torch.from_numpy(a))
        return dx, ds
    if layout == "packed":
        bx = torch.from_numpy(np.stack(xs)).to(dev)
        bs_ = torch.from_numpy(np.stack(ss)).to(dev)
        return [bx[r] for r in range(len(xs))], [bs_[r] for r in range(len(ss))]
    return [torch.from_numpy(a).to(dev) for a in xs], [torch.from_numpy(a).to(dev) for a in ss]


def setup_share(wl, dev, qrs, workloads, torch, layout):
    """This GPU's share (qrs_run): W slices [rows, H] -> [rows, H]."""
    alg_bytes = wl.algorithmic_bytes()
    t0 = time.perf_counter()
    xs, ss = workloads.generate(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    n_sets = max(2, -(-4 * MALL_BYTES // alg_bytes))
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.out_dtype]
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    stream = torch.cuda.current_stream(dev)
    launches, outs = [], []
    for _ in range(n_sets):
        dx, ds = place_inputs(p, xs, ss, dev, qrs, torch, layout)
        out = torch.empty((wl.rows, wl.h), dtype=out_dt, device=dev)
        launches.append(qrs.Launch(p, dx, ds, out, stream=stream))
        outs.append([out])
    return alg_bytes, launches, outs, (xs, ss)


def setup_strided(wl, dev, qrs, workloads, torch, layout):
    """This GPU's share from a row-interleaved receive buffer
    (qrs_run_strided): codes [rows, W, H] and scales [rows, W, H/G], so each
    rank slice is a row-strided view; output [rows, H]."""
    alg_bytes = wl.algorithmic_bytes()
    t0 = time.perf_counter()
    xs, ss = workloads.generate(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    n_sets = max(2, -(-4 * MALL_BYTES // alg_bytes))
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.out_dtype]
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    stream = torch.cuda.current_stream(dev)
    bx0 = torch.from_numpy(np.ascontiguousarray(np.stack(xs, axis=1))).to(dev)
    bs0 = torch.from_numpy(np.ascontiguousarray(np.stack(ss, axis=1))).to(dev)
    launches, outs = [], []
    for k in range(n_sets):
        bx = bx0 if k == 0 else bx0.clone()
        bs_ = bs0 if k == 0 else bs0.clone()
        out = torch.empty((wl.rows, wl.h), dtype=out_dt, device=dev)
        launches.append(qrs.StridedLaunch(p, [bx[:, r] for r in range(wl.world_size)],
                                          [bs_[:, r] for r in range(wl.world_size)], out, stream=stream))
        outs.append([out])
    return alg_bytes, launches, outs, (xs, ss)


def setup_all_shares(wl, dev, qrs, workloads, torch, layout):
    """The group's whole reduce-scatter on this GPU (qrs_run_all_shares):
    W inputs [BS, H] -> W shares [BS/W, H], the all-to-all by addressing."""
    alg_bytes = wl.world_size * wl.algorithmic_bytes()
    t0 = time.perf_counter()
    xs, ss = workloads.generate_full(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    n_sets = max(2, -(-4 * MALL_BYTES // alg_bytes))
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.out_dtype]
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    stream = torch.cuda.current_stream(dev)
    launches, outs = [], []
    for _ in range(n_sets):
        dx, ds = place_inputs(p, xs, ss, dev, qrs, torch, layout, full_inputs=True)
        o = [torch.empty((wl.rows, wl.h), dtype=out_dt, device=dev) for _ in range(wl.world_size)]
        launches.append(qrs.AllSharesLaunch(p, dx, ds, o, stream=stream))
        outs.append(o)
    return alg_bytes, launches, outs, None


def setup_quantize(wl, dev, qrs, workloads, torch, layout):
    """Producer-side quantization (qrs_quantize) of one rank's bf16
    activations [BS, H] into the workload's x format and scale layout."""
    n = wl.bs * wl.h
    scale_bytes = n // 128 * 4 if wl.scale_layout == "f32_group128" else n // 32
    alg_bytes = 2 * n + n + scale_bytes
    t0 = time.perf_counter()
    bits = workloads.generate_activations(wl, 0)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    n_sets = max(2, -(-4 * MALL_BYTES // alg_bytes))
    x0 = torch.from_numpy(bits.view("int16")).view(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream(dev)
    g = 128 if wl.scale_layout == "f32_group128" else 32
    sdt = torch.float32 if wl.scale_layout == "f32_group128" else torch.uint8
    launches, outs = [], []
    for k in range(n_sets):
        x = x0 if k == 0 else x0.clone()
        codes = torch.empty((wl.bs, wl.h), dtype=torch.uint8, device=dev)
        scales = torch.empty((wl.bs, wl.h // g), dtype=sdt, device=dev)
        launches.append(qrs.QuantizeLaunch(x, codes, scales, wl.x_format, wl.scale_layout, stream=stream))
        outs.append([codes, scales])
    return alg_bytes, launches, outs, None


OPS = {"share": setup_share, "strided": setup_strided, "all_shares": setup_all_shares, "quantize": setup_quantize}


LARGEST = "w8_bs65536_h5120_mx_e5m2_f32"


def time_steps(launches, warmup, steps, stream, torch):
    """W untimed launches, then K timed ones rotating over the sets: HIP
    events on the launch stream at both ends, wall clock around them (with a
    synchronize on both sides). Returns (wall seconds, seconds per launch)."""
    n_sets = len(launches)
    for i in range(warmup):
        launches[i % n_sets]()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    order = [launches[(warmup + i) % n_sets] for i in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for launch in order:
        launch()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / 1e3 / steps


def time_largest(args, dev, qrs, workloads, torch):
    """The largest workload's share, timed like the headline steps."""
    wl = workloads.WORKLOADS[LARGEST]
    log(f"[bench] largest workload {wl.name}: W={wl.world_size} BS={wl.bs} H={wl.h} rows={wl.rows}")
    alg_bytes, launches, outs, _ = setup_share(wl, dev, qrs, workloads, torch, args.layout)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    wall, per_launch = time_steps(launches, args.warmup, args.steps, stream, torch)
    achieved = alg_bytes / per_launch / 1e9
    log(f"[bench] largest workload: {args.steps} steps in {wall * 1e3:.2f} ms wall; HIP events: "
        f"{per_launch * 1e6:.2f} us per launch = {achieved:.0f} GB/s")
    del launches, outs
    torch.cuda.empty_cache()
    return {
        "workload": f"{wl.name}: W={wl.world_size} BS={wl.bs} H={wl.h} x={wl.x_format} scales={wl.scale_layout} "
                    f"out={wl.out_dtype}",
        "algorithmic_bytes_per_step": alg_bytes,
        "steps": args.steps,
        "warmup": args.warmup,
        "kernel_us_avg": round(per_launch * 1e6, 3),
        "achieved": round(achieved, 2),
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "value": round(alg_bytes * args.steps / wall / 1e9, 2),
        "ms_per_step": round(wall * 1e3 / args.steps, 6),
    }


# Rows per slice of the size sweep. Below about 1024 rows a launch at W = 8
# takes less device time than the host needs to enqueue it (about 5-8 us
# through the binding), so smaller points would measure the host.
SWEEP_ROWS = (1024, 1536, 2048, 3072, 4096, 6144, 8192)


def time_copy(nbytes, n_sets, warmup, steps, dev, qrs, torch, stream):
    """The plain 16-byte stream copy moving nbytes (half read, half
    written), rotating over n_sets buffer pairs, timed like the steps.
    Returns seconds per copy."""
    half = (nbytes // 2) // 16 * 16
    src = torch.empty(half * n_sets, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    pairs = [(src[k * half:(k + 1) * half], dst[k * half:(k + 1) * half]) for k in range(n_sets)]
    launches = [lambda a=a, b=b: qrs.stream_copy(a, b, stream=stream) for a, b in pairs]
    _, per = time_steps(launches, warmup, steps, stream, torch)
    del src, dst, pairs, launches
    return per


def fit_fixed_and_rate(points):
    """Least-squares line time = fixed + bytes / rate over (bytes, seconds)
    points: returns (fixed microseconds, rate in GB/s)."""
    b = np.array([p[0] for p in points], dtype=np.float64)
    t = np.array([p[1] for p in points], dtype=np.float64)
    slope, intercept = np.polyfit(b, t, 1)
    return intercept * 1e6, 1.0 / slope / 1e9


def size_sweep(wl, args, dev, qrs, workloads, torch, sweep_rows=SWEEP_ROWS):
    """The share kernel and the stream copy at sweep_rows rows per slice
    (ascending) of the workload's shape (W, H, types), inputs sliced from one
    generated set of the largest size and placed at the recommended pitch."""
    stream = torch.cuda.current_stream(dev)
    big = wl.with_(bs=sweep_rows[-1] * wl.world_size)
    xs_big, ss_big = workloads.generate(big)
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.out_dtype]
    steps = max(50, min(args.steps, 1000))
    points, kernel_pts, copy_pts = [], [], []
    for rows in sweep_rows:
        sub = wl.with_(bs=rows * wl.world_size)
        alg = sub.algorithmic_bytes()
        xs = [np.ascontiguousarray(x[:rows]) for x in xs_big]
        ss = [np.ascontiguousarray(x[:rows]) for x in ss_big]
        n_sets = max(2, -(-4 * MALL_BYTES // alg))
        p = qrs.plan(sub.world_size, sub.bs, sub.h, sub.x_format, sub.scale_layout, sub.out_dtype)
        launches = []
        for _ in range(n_sets):
            dx, ds = place_inputs(p, xs, ss, dev, qrs, torch, args.layout)
            out = torch.empty((rows, sub.h), dtype=out_dt, device=dev)
            launches.append(qrs.Launch(p, dx, ds, out, stream=stream))
        _, k_s = time_steps(launches, 20, steps, stream, torch)
        del launches
        torch.cuda.empty_cache()
        c_s = time_copy(alg, n_sets, 20, steps, dev, qrs, torch, stream)
        torch.cuda.empty_cache()
        points.append({"rows_per_slice": rows, "bytes": alg, "kernel_us": round(k_s * 1e6, 3),
                       "copy_us": round(c_s * 1e6, 3)})
        kernel_pts.append((alg, k_s))
        copy_pts.append((alg, c_s))
        log(f"[bench] size sweep: {rows} rows per slice, {alg} bytes: kernel {k_s * 1e6:.2f} us, "
            f"copy {c_s * 1e6:.2f} us")
    kf, kr = fit_fixed_and_rate(kernel_pts)
    cf, cr = fit_fixed_and_rate(copy_pts)
    return {
        "shape": f"W={wl.world_size} H={wl.h} x={wl.x_format} scales={wl.scale_layout} out={wl.out_dtype}",
        "steps_per_point": steps,
        "points": points,
        "fit": {"kernel": {"fixed_us": round(kf, 3), "GBps": round(kr, 1)},
                "copy": {"fixed_us": round(cf, 3), "GBps": round(cr, 1)}},
        "note": "context only: least-squares time = fixed + bytes / rate over the points",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="w8_bs16384_h8192_mx_e4m3_bf16", choices=sorted(workloads_names()),
                    help="default: the W=8, BS=16384, H=8192 MX E4M3FN -> bf16 share")
    ap.add_argument("--op", default="share", choices=sorted(OPS),
                    help="share: this GPU's share (the hot path, default); strided: the same share from a "
                         "row-interleaved receive buffer [rows, W, H] through qrs_run_strided; all_shares: every "
                         "rank's share from the inputs before the all-to-all, in one launch; quantize: the "
                         "producer-side quantization of one rank's bf16 activations [BS, H]")
    ap.add_argument("--layout", default="pitched", choices=["pitched", "packed", "separate"],
                    help="placement of the W rank slices: pitched (one buffer, the pitch qrs_slice_pitch "
                         "recommends; default), packed (one buffer, back to back), separate (one allocation each)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timings (cpu_baseline and cpu_baseline_all_cores = null)")
    ap.add_argument("--hot", action="store_true",
                    help="also time K launches on one input/output set, without rotation (context only)")
    ap.add_argument("--overlap", action="store_true",
                    help="also time K independent steps alternated over two streams (context only)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="also time the share kernel and the stream copy at 1024 to 8192 rows per slice and fit "
                         "time = fixed + bytes / rate (context only; --op share)")
    ap.add_argument("--no-largest", action="store_true",
                    help="skip the largest workload's extra timing (largest_workload = null)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share on one GPU only: run it with --gpus 1 "
              "(the all-to-all between GPUs is outside this library)", file=sys.stderr)
        sys.exit(2)
    if args.steps <= 0 or args.warmup < 0:
        sys.exit("--steps must be positive and --warmup non-negative")

    import torch

    import quantized_collective_reduction_amd as qrs
    import workloads

    qrs.load_library()
    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    log(f"[bench] {args.op} on {wl.name}: W={wl.world_size} BS={wl.bs} H={wl.h} rows={wl.rows} "
        f"{wl.x_format}/{wl.scale_layout}->{wl.out_dtype}")
    alg_bytes, launches, outs, host_inputs = OPS[args.op](wl, dev, qrs, workloads, torch, args.layout)
    n_sets = len(launches)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    log(f"[bench] {alg_bytes} algorithmic bytes per step; {n_sets} rotating input/output sets on "
        f"{torch.cuda.get_device_name(dev)}")

    # Timed region: K back-to-back launches after W warm-up ones, HIP events
    # on the launch stream at both ends, wall clock around it.
    wall, avg_launch_s = time_steps(launches, args.warmup, args.steps, stream, torch)
    # All sets hold identical inputs, so every set that ran must hold the same bits.
    if args.warmup + args.steps >= n_sets:
        for o in outs[1:]:
            for a, b in zip(o, outs[0]):
                if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
                    sys.exit("rotating sets disagree: the kernel is not deterministic")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"[bench] {args.steps} steps in {wall * 1e3:.2f} ms wall; HIP events over the region: "
        f"{avg_launch_s * 1e6:.2f} us per launch")

    hot_s = None
    if args.hot:
        # Context: the same launches on one set, no rotation. Opt-in, so that
        # a kernel trace of the default command averages rotated launches only.
        hot = launches[0]
        for _ in range(min(args.warmup, 20)):
            hot()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            hot()
        ev1.record(stream)
        torch.cuda.synchronize()
        hot_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
        log(f"[bench] hot (one set, no rotation): {hot_s * 1e6:.2f} us per launch")

    overlap = None
    if args.overlap:
        # Context: independent steps alternated over two streams (both of
        # the default priority), so that one launch's ramp-up overlaps the
        # previous one's drain. Each stream keeps to its own input/output
        # sets (an even number of them), so no two launches in flight share
        # a buffer. Wall time over the K steps, like value.
        s2 = torch.cuda.Stream(device=dev)
        n_even = n_sets - n_sets % 2
        pair = [launches[k] if k % 2 == 0 else launches[k].on_stream(s2) for k in range(n_even)]
        for i in range(min(args.warmup, 20) + n_even):
            pair[i % n_even]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            pair[i % n_even]()
        torch.cuda.synchronize()
        wall2 = time.perf_counter() - t0
        overlap = {"us_per_step": round(wall2 / args.steps * 1e6, 3),
                   "GBps": round(alg_bytes * args.steps / wall2 / 1e9, 2),
                   "sets_per_stream": n_even // 2,
                   "note": "context only: independent steps alternated over two default-priority streams; "
                           "value and roofline describe one launch at a time"}
        log(f"[bench] two streams: {overlap['us_per_step']:.2f} us per step = {overlap['GBps']:.0f} GB/s")
        del pair, s2

    # Calibration: the plain 16-byte stream copy of the same read+write
    # volume, rotating over n_sets buffer pairs and timed like the steps.
    copy_bytes = (alg_bytes // 2) // 16 * 16
    src = torch.empty(copy_bytes * n_sets, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copies = [(src[k * copy_bytes:(k + 1) * copy_bytes], dst[k * copy_bytes:(k + 1) * copy_bytes])
              for k in range(n_sets)]
    n_copies = max(50, min(args.steps, 1000))
    for i in range(10):
        qrs.stream_copy(*copies[i % n_sets], stream=stream)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(n_copies):
        qrs.stream_copy(*copies[i % n_sets], stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_s = ev0.elapsed_time(ev1) / 1e3 / n_copies
    copy_gbps = 2 * copy_bytes / copy_s / 1e9
    log(f"[bench] stream-copy calibration: {2 * copy_bytes} bytes moved in {copy_s * 1e6:.2f} us = {copy_gbps:.0f} GB/s")
    del src, dst, copies

    largest = None
    sweep = None
    if args.op == "share" and (args.size_sweep or (not args.no_largest and wl.name != LARGEST)):
        del launches, outs
        torch.cuda.empty_cache()
        if not args.no_largest and wl.name != LARGEST:
            largest = time_largest(args, dev, qrs, workloads, torch)
        if args.size_sweep:
            sweep = size_sweep(wl, args, dev, qrs, workloads, torch)

    achieved = alg_bytes / avg_launch_s / 1e9
    value = alg_bytes * args.steps / wall / 1e9
    result = {
        "metric": {"share": METRIC, "strided": METRIC + " (row-interleaved receive buffer)",
                   "all_shares": METRIC + " (all W shares in one launch)",
               "quantize": "achieved HBM GB/s and % of peak for the producer-side quantization"}[args.op],
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: W={wl.world_size} BS={wl.bs} H={wl.h} x={wl.x_format} "
                        f"scales={wl.scale_layout} out={wl.out_dtype}"
                        + {"share": "", "strided": ", slices row-interleaved in one [rows, W, H] buffer",
                           "all_shares": ", all W shares from the pre-all-to-all inputs",
                           "quantize": f", quantize one rank's bf16 [{wl.bs}, {wl.h}]"}[args.op],
            "op": args.op,
            "layout": {"quantize": None, "strided": "row-interleaved"}.get(args.op, args.layout),
            "world_size": wl.world_size,
            "bs": wl.bs,
            "rows": wl.rows,
            "h": wl.h,
            "algorithmic_bytes_per_step": alg_bytes,
            "rotating_sets": n_sets,
            # dtype above is the arithmetic type (the fp32 products and fold);
            # these are the element types the step reads and writes.
            "element_types": {"x": wl.x_format, "scales": {"f32_group128": "f32", "e8m0_block32": "e8m0"}[wl.scale_layout],
                              "out": wl.out_dtype} if args.op != "quantize" else
                             {"in": "bf16", "codes": wl.x_format,
                              "scales": {"f32_group128": "f32", "e8m0_block32": "e8m0"}[wl.scale_layout]},
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic(wl.name, args.op),
            "kernel_us_avg": round(avg_launch_s * 1e6, 3),
        },
        "device_memory": device_memory_props(),
        "copy_calibration": {"bytes_moved": 2 * copy_bytes, "us": round(copy_s * 1e6, 3),
                             "GBps": round(copy_gbps, 1)},
        "overlap_2streams": overlap,
        "largest_workload": largest,
        "size_sweep": sweep,
        "hot": None if hot_s is None else {
            "kernel_us_avg": round(hot_s * 1e6, 3), "GBps": round(alg_bytes / hot_s / 1e9, 2),
            "note": "context only: one input/output set, no rotation"},
        "cpu_baseline": None,
        "cpu_baseline_all_cores": None,
    }
    if not args.no_cpu_baseline and host_inputs is not None:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(wl, *host_inputs)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(wl, *host_inputs)
        log(f"[bench] cpu baseline, all cores: {result['cpu_baseline_all_cores']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
