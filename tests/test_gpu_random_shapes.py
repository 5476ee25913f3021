"""GPU parity on seeded random shapes: every mode, world size, output dtype,
H drawn from all legal widths (multiples of 128 in [1024, 8192]) and row
counts from 1 to 40, through qrs_run, qrs_run_strided (padded rows) and
qrs_run_all_shares. The case list is fixed by a seed, so failures reproduce."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import OUT_TORCH, assert_parity, log, oracle_bits, out_bits, run_gpu

pytestmark = pytest.mark.gpu

MODES = [("int8", "f32_group128"), ("e4m3fn", "f32_group128"), ("e5m2", "f32_group128"),
         ("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32")]


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        xf, sl = MODES[rng.integers(len(MODES))]
        out.append(dict(w=int(rng.choice([2, 4, 8])), rows=int(rng.integers(1, 41)),
                        h=int(128 * rng.integers(8, 65)), x_format=xf, scale_layout=sl,
                        out_dtype=str(rng.choice(["f32", "bf16", "f16"])), seed=1000 + k))
    return out


def _workload(c, rows_per_rank):
    return workloads.Workload(
        "rand", c["w"], c["w"] * rows_per_rank, c["h"], c["x_format"], c["scale_layout"], c["out_dtype"],
        x_dist="int_uniform" if c["x_format"] == "int8" else "normal",
        x_param=127 if c["x_format"] == "int8" else 60,
        scale_lo=-12 if c["scale_layout"] == "f32_group128" else 112,
        scale_hi=2 if c["scale_layout"] == "f32_group128" else 140, seed=c["seed"])


CASES = _cases(24, 2024)


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"W{c['w']}-r{c['rows']}-h{c['h']}-{c['x_format']}-"
                                                  f"{c['scale_layout']}-{c['out_dtype']}")
def test_random_shape(gpu, c):
    log(f"[random] {c}")
    wl = _workload(c, c["rows"])
    xs, ss = workloads.generate(wl)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype),
                       wl.out_dtype)
    # qrs_run on contiguous slices
    got = run_gpu(wl.world_size, wl.rows, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype, xs, ss)
    assert_parity(got, want, wl.out_dtype, "run")
    # qrs_run_strided: each slice and the output padded by 128 elements per row
    g = wl.group
    dx = [torch.zeros((wl.rows, wl.h + 128), dtype=torch.uint8, device="cuda") for _ in xs]
    ds = [torch.zeros((wl.rows, (wl.h + 128) // g), dtype=torch.from_numpy(ss[0]).dtype, device="cuda")
          for _ in ss]
    for t, x in zip(dx, xs):
        t[:, :wl.h].copy_(torch.from_numpy(x))
    for t, s in zip(ds, ss):
        t[:, :wl.h // g].copy_(torch.from_numpy(s))
    out_full = torch.full((wl.rows, wl.h + 128), float("nan"), dtype=OUT_TORCH[wl.out_dtype], device="cuda")
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    qrs.run_strided(p, [t[:, :wl.h] for t in dx], [t[:, :wl.h // g] for t in ds], out_full[:, :wl.h])
    torch.cuda.synchronize()
    assert_parity(out_bits(out_full[:, :wl.h].contiguous()), want, wl.out_dtype, "run_strided")
    assert torch.isnan(out_full[:, wl.h:].float()).all(), "run_strided wrote outside the output rows"


@pytest.mark.parametrize("c", CASES[:12], ids=lambda c: f"W{c['w']}-r{c['rows']}-h{c['h']}-{c['x_format']}-"
                                                       f"{c['scale_layout']}-{c['out_dtype']}")
def test_random_shape_all_shares(gpu, c):
    wl = _workload(c, c["rows"])
    xs, ss = workloads.generate_full(wl)
    want = oracle.all_shares(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx = [torch.from_numpy(x).cuda() for x in xs]
    ds = [torch.from_numpy(s).cuda() for s in ss]
    outs = [torch.empty((wl.rows, wl.h), dtype=OUT_TORCH[wl.out_dtype], device="cuda") for _ in range(wl.world_size)]
    qrs.run_all_shares(p, dx, ds, outs)
    torch.cuda.synchronize()
    for j in range(wl.world_size):
        assert_parity(out_bits(outs[j]), oracle_bits(want[j], wl.out_dtype), wl.out_dtype, f"share {j}")


def _window_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        xf, sl = MODES[rng.integers(len(MODES))]
        g = 128 if sl == "f32_group128" else 32
        out.append(dict(w=int(rng.choice([2, 4, 8])), rows=int(rng.integers(100, 1201)),
                        h=int(128 * rng.integers(8, 65)), x_format=xf, scale_layout=sl,
                        out_dtype=str(rng.choice(["f32", "bf16", "f16"])), seed=5000 + k,
                        c0=int(g * rng.integers(0, 17)), extra=int(g * rng.integers(0, 9)) + 128))
    return out


WINDOW_CASES = _window_cases(24, 77)


@pytest.mark.parametrize("c", WINDOW_CASES, ids=lambda c: f"W{c['w']}-r{c['rows']}-h{c['h']}-c{c['c0']}-"
                                                         f"{c['x_format']}-{c['scale_layout']}-{c['out_dtype']}")
def test_random_column_windows(gpu, c):
    """Larger grids (100 to 1200 rows: up to thousands of blocks) read
    through column windows of wider tensors, so x rows, scale rows and
    output rows start anywhere: for MX scales a window start that is not a
    multiple of 128 columns puts the scale rows off their lines, which gives
    each XCD runs of blocks over whole rows. qrs_run_strided must give the
    bytes qrs_run gives on contiguous copies, sampled rows must match the
    oracle, and nothing outside the output window may change."""
    log(f"[window] {c}")
    w, rows, h, c0 = c["w"], c["rows"], c["h"], c["c0"]
    ht = h + c0 + c["extra"]
    wl = workloads.Workload("win", w, w * rows, ht, c["x_format"], c["scale_layout"], c["out_dtype"],
                            x_dist="int_uniform" if c["x_format"] == "int8" else "normal",
                            x_param=127 if c["x_format"] == "int8" else 60,
                            scale_lo=-12 if c["scale_layout"] == "f32_group128" else 112,
                            scale_hi=2 if c["scale_layout"] == "f32_group128" else 140, seed=c["seed"])
    xs_full, ss_full = workloads.generate(wl)
    g = wl.group
    dx_full = [torch.from_numpy(x).cuda() for x in xs_full]
    ds_full = [torch.from_numpy(s).cuda() for s in ss_full]
    dx = [t[:, c0:c0 + h] for t in dx_full]
    ds = [t[:, c0 // g:(c0 + h) // g] for t in ds_full]
    p = qrs.plan(w, w * rows, h, c["x_format"], c["scale_layout"], c["out_dtype"])
    oc0 = c0 % 256
    out_full = torch.full((rows, h + 512), float("nan"), dtype=OUT_TORCH[c["out_dtype"]], device="cuda")
    qrs.run_strided(p, dx, ds, out_full[:, oc0:oc0 + h])
    ref = torch.empty((rows, h), dtype=OUT_TORCH[c["out_dtype"]], device="cuda")
    qrs.run(p, [t.contiguous() for t in dx], [t.contiguous() for t in ds], ref)
    torch.cuda.synchronize()
    got = out_full[:, oc0:oc0 + h].contiguous()
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), "run_strided differs from run"
    assert torch.isnan(out_full[:, :oc0].float()).all() and torch.isnan(out_full[:, oc0 + h:].float()).all()
    sample = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(c["seed"]).integers(0, rows, 4)]))
    want = oracle.reduce_scatter_share([np.ascontiguousarray(x[sample, c0:c0 + h]) for x in xs_full],
                                       [np.ascontiguousarray(s[sample, c0 // g:(c0 + h) // g]) for s in ss_full],
                                       c["x_format"], c["scale_layout"], c["out_dtype"])
    assert_parity(out_bits(got)[sample], oracle_bits(want, c["out_dtype"]), c["out_dtype"], "sampled rows")
