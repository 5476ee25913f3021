"""Every entry point that launches the reduce or the quantize kernels, run with
a small launch bound (QRS_MAX_LAUNCH_ELEMS, set by the caller) so that each
call becomes several launches over consecutive element or row ranges, and
checked against the oracle bit for bit. Run as a child process by
tests/test_gpu_launch_parts.py; exits non-zero on the first mismatch."""

import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import quantized_collective_reduction_amd as qrs  # noqa: E402
import workloads  # noqa: E402
from gpu_util import OUT_TORCH, assert_parity, log, oracle_bits, out_bits, to_device  # noqa: E402
from oracle.quantize import quantize as oracle_quantize  # noqa: E402

BOUND = int(os.environ["QRS_MAX_LAUNCH_ELEMS"])


def _parts(n, m):
    return -(-n // m)


def _workload(w, rows, h, x_format, scale_layout, out_dtype, seed):
    return workloads.Workload("parts", w, rows * w, h, x_format, scale_layout, out_dtype,
                              x_dist="int_uniform" if x_format == "int8" else "normal",
                              x_param=127 if x_format == "int8" else 30,
                              scale_lo=-10 if scale_layout == "f32_group128" else 110,
                              scale_hi=2 if scale_layout == "f32_group128" else 140, seed=seed)


def contiguous(w, rows, h, x_format, scale_layout, out_dtype, seed):
    what = f"contiguous W={w} rows={rows} H={h} {x_format}/{scale_layout}->{out_dtype}"
    log(f"[parts] {what}")
    xs, ss = workloads.generate(_workload(w, rows, h, x_format, scale_layout, out_dtype, seed))
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    launches = qrs.run_launch_info(p)["launches"]
    assert launches == _parts(rows * h, BOUND) > 1, (what, launches)
    dx, ds = to_device(xs, ss)
    out = torch.full((rows, h), float("nan"), dtype=OUT_TORCH[out_dtype], device="cuda")
    qrs.run(p, dx, ds, out)
    torch.cuda.synchronize()
    assert_parity(out_bits(out), want, out_dtype, what)
    out.fill_(float("nan"))
    step = qrs.Launch(p, dx, ds, out)
    step()
    torch.cuda.synchronize()
    assert_parity(out_bits(out), want, out_dtype, what + " (prepared launch)")
    return launches


def strided(w, rows, h, x_format, scale_layout, out_dtype, seed):
    what = f"strided W={w} rows={rows} H={h} {x_format}/{scale_layout}->{out_dtype}"
    log(f"[parts] {what}")
    g = 128 if scale_layout == "f32_group128" else 32
    c0, extra = 256, 512  # column window [c0, c0 + h) of [rows, h + extra] tensors
    xs_full, ss_full = workloads.generate(_workload(w, rows, h + extra, x_format, scale_layout, out_dtype, seed))
    xs = [np.ascontiguousarray(x[:, c0:c0 + h]) for x in xs_full]
    ss = [np.ascontiguousarray(s[:, c0 // g:(c0 + h) // g]) for s in ss_full]
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
    dx_full, ds_full = to_device(xs_full, ss_full)
    dx = [t[:, c0:c0 + h] for t in dx_full]
    ds = [t[:, c0 // g:(c0 + h) // g] for t in ds_full]
    oc0 = 64
    out_full = torch.full((rows, h + 192), float("nan"), dtype=OUT_TORCH[out_dtype], device="cuda")
    out = out_full[:, oc0:oc0 + h]
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    qrs.run_strided(p, dx, ds, out)
    torch.cuda.synchronize()
    assert_parity(out_bits(out.contiguous()), want, out_dtype, what)
    full = out_bits(out_full)
    sentinel = out_bits(torch.full((1, 1), float("nan"), dtype=OUT_TORCH[out_dtype]))[0, 0]
    assert np.all(full[:, :oc0] == sentinel) and np.all(full[:, oc0 + h:] == sentinel), what + ": wrote outside"


def all_shares(w, rows, h, x_format, scale_layout, out_dtype, seed):
    what = f"all shares W={w} rows={rows} H={h} {x_format}/{scale_layout}->{out_dtype}"
    log(f"[parts] {what}")
    xf, sf = workloads.generate_full(_workload(w, rows, h, x_format, scale_layout, out_dtype, seed))
    want = oracle.all_shares(xf, sf, x_format, scale_layout, out_dtype)
    dx, ds = to_device(xf, sf)
    outs = [torch.full((rows, h), float("nan"), dtype=OUT_TORCH[out_dtype], device="cuda") for _ in range(w)]
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    qrs.run_all_shares(p, dx, ds, outs)
    torch.cuda.synchronize()
    for j in range(w):
        assert_parity(out_bits(outs[j]), oracle_bits(want[j], out_dtype), out_dtype, f"{what}, share {j}")


def quantize(tokens, h, x_format, scale_layout, seed):
    what = f"quantize [{tokens}, {h}] -> {x_format}/{scale_layout}"
    log(f"[parts] {what}")
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((tokens, h)).astype(np.float32) * np.exp2(rng.integers(-20, 20, size=(tokens, 1)))
    bits = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_c, want_s = oracle_quantize(bits, x_format, scale_layout)
    g = 128 if scale_layout == "f32_group128" else 32
    x = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    codes = torch.full((tokens, h), 0xAA, dtype=torch.uint8, device="cuda")
    if scale_layout == "f32_group128":
        scales = torch.full((tokens, h // g), float("nan"), dtype=torch.float32, device="cuda")
    else:
        scales = torch.full((tokens, h // g), 0xAA, dtype=torch.uint8, device="cuda")
    qrs.quantize(x, codes, scales, x_format, scale_layout)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), want_c), what + ": codes"
    got_s = scales.cpu().numpy()
    if got_s.dtype == np.float32:
        assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), what + ": scales"
    else:
        assert np.array_equal(got_s, want_s), what + ": scales"


def _capture(fn):
    """fn run once eagerly on a side stream, then captured in a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def share_in_a_graph(w, rows, h, x_format, scale_layout, out_dtype, seed):
    what = f"graph of a split share W={w} rows={rows} H={h} {x_format}/{scale_layout}->{out_dtype}"
    log(f"[parts] {what}")
    xs, ss = workloads.generate(_workload(w, rows, h, x_format, scale_layout, out_dtype, seed))
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    assert qrs.run_launch_info(p)["launches"] > 1
    dx, ds = to_device(xs, ss)
    out = torch.empty((rows, h), dtype=OUT_TORCH[out_dtype], device="cuda")
    g = _capture(lambda: qrs.run(p, dx, ds, out))
    for rep in range(3):
        out.fill_(float("nan"))  # eager work between replays: every element must be rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(out_bits(out), want, out_dtype, f"{what}, replay {rep}")


def pipeline_in_a_graph(w, rows, h, seed):
    # Every rank's quantize, then the group's all shares, each split into
    # several launches, in one graph.
    what = f"graph of split quantizations and all shares W={w} rows={rows} H={h}"
    log(f"[parts] {what}")
    bs = w * rows
    rng = np.random.default_rng(seed)
    acts = []
    for _ in range(w):
        v = rng.standard_normal((bs, h)).astype(np.float32) * np.float32(4.0)
        acts.append(torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    q = [oracle_quantize(a, "e4m3fn", "e8m0_block32") for a in acts]
    want = oracle.all_shares([c for c, _ in q], [s for _, s in q], "e4m3fn", "e8m0_block32", "bf16")
    xin = [torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda() for a in acts]
    p = qrs.plan(w, bs, h, "e4m3fn", "e8m0_block32", "bf16")
    codes = [torch.empty((bs, h), dtype=torch.uint8, device="cuda") for _ in range(w)]
    scales = [torch.empty((bs, h // 32), dtype=torch.uint8, device="cuda") for _ in range(w)]
    outs = [torch.empty((rows, h), dtype=torch.bfloat16, device="cuda") for _ in range(w)]

    def pipeline():
        for r in range(w):
            qrs.quantize(xin[r], codes[r], scales[r], "e4m3fn", "e8m0_block32")
        qrs.run_all_shares(p, codes, scales, outs)

    g = _capture(pipeline)
    for rep in range(3):
        for t in codes + scales:
            t.fill_(0xAA)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j in range(w):
            assert_parity(out_bits(outs[j]), oracle_bits(want[j], "bf16"), "bf16", f"{what}, replay {rep}, share {j}")


def main():
    assert BOUND == 4096, "the cases below are sized for a bound of 4096 elements"
    # 42,624 elements: ten full launches and a ragged eleventh (1,664).
    contiguous(8, 37, 1152, "e4m3fn", "e8m0_block32", "bf16", 1)   # 8-element pieces
    contiguous(2, 37, 1152, "int8", "f32_group128", "f32", 2)      # 16-element chunks, fp32 staging
    contiguous(4, 24, 2048, "e5m2", "e8m0_block32", "f32", 3)      # fp32 pieces, twelve full launches
    contiguous(8, 37, 1152, "e5m2", "f32_group128", "f16", 4)
    # Rows of 1152: twelve launches of 3 rows, then one of a single row.
    strided(8, 37, 1152, "e4m3fn", "e8m0_block32", "f16", 5)
    strided(4, 37, 1152, "e5m2", "f32_group128", "bf16", 6)
    # Rows longer than the bound: one row per launch (each a one-row share).
    strided(2, 5, 8192, "int8", "f32_group128", "bf16", 7)
    # All shares advance together through one split launch over the group
    # (MX at W = 8, capped), or the small group's single launch is split.
    all_shares(8, 37, 1152, "e4m3fn", "e8m0_block32", "bf16", 8)
    all_shares(2, 37, 1152, "int8", "f32_group128", "f32", 9)
    all_shares(4, 24, 2048, "e5m2", "e8m0_block32", "f16", 10)
    quantize(37, 1152, "e4m3fn", "e8m0_block32", 11)
    quantize(37, 1152, "int8", "f32_group128", 12)
    # Captured in HIP graphs: every launch of the split is a node.
    share_in_a_graph(8, 37, 1152, "e4m3fn", "e8m0_block32", "bf16", 13)
    pipeline_in_a_graph(4, 37, 1152, 14)
    # Seeded random shapes: every mode, W and output type, sizes from a few
    # launches to a few dozen.
    rng = np.random.default_rng(2024)
    modes = [("int8", "f32_group128"), ("e4m3fn", "f32_group128"), ("e5m2", "f32_group128"),
             ("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32")]
    for i in range(12):
        w = int(rng.choice([2, 4, 8]))
        x_format, scale_layout = modes[int(rng.integers(len(modes)))]
        out_dtype = str(rng.choice(["f32", "bf16", "f16"]))
        h = 128 * int(rng.integers(8, 65))
        rows = int(rng.integers(-(-2 * BOUND // h), 60))
        kind = i % 3
        if kind == 0:
            contiguous(w, rows, h, x_format, scale_layout, out_dtype, 100 + i)
        elif kind == 1:
            strided(w, rows, h, x_format, scale_layout, out_dtype, 100 + i)
        else:
            all_shares(w, rows, h, x_format, scale_layout, out_dtype, 100 + i)
    print("[parts] all cases match the oracle", flush=True)


if __name__ == "__main__":
    main()
