"""Largest shapes: an fp32 output past 4 GiB (byte offsets beyond 2^32) from
1 GiB input slices, checked against the oracle on a repeating row block."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("x_format,scale_layout", [("e5m2", "e8m0_block32"), ("int8", "f32_group128")])
def test_output_beyond_4gib(gpu, x_format, scale_layout):
    w, h, rows, blk = 2, 8192, 133120, 64  # output 4.06 GiB: byte offsets past 2^32
    wl = workloads.Workload("large", w, w * blk, h, x_format, scale_layout, "f32",
                            x_dist="int_uniform" if x_format == "int8" else "normal",
                            x_param=127 if x_format == "int8" else 300,
                            scale_lo=-8 if scale_layout == "f32_group128" else 110,
                            scale_hi=0 if scale_layout == "f32_group128" else 140, seed=31)
    xs, ss = workloads.generate(wl)  # one block of 64 rows per rank
    want = oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, "f32").view(np.int32)
    log(f"[large] {x_format}/{scale_layout}: {rows} x {h} fp32 output ({rows * h * 4 / 2**30:.2f} GiB)")
    reps = rows // blk
    dx = [torch.from_numpy(x).cuda().repeat(reps, 1) for x in xs]
    ds = [torch.from_numpy(s).cuda().repeat(reps, 1) for s in ss]
    out = torch.empty((rows, h), dtype=torch.float32, device="cuda")
    assert out.numel() * 4 > 2**32
    p = qrs.plan(w, w * rows, h, x_format, scale_layout, "f32")
    qrs.run(p, dx, ds, out)
    torch.cuda.synchronize()
    del dx, ds
    want_t = torch.from_numpy(want).cuda()
    got = out.view(torch.int32).view(reps, blk, h)
    assert torch.equal(got, want_t.unsqueeze(0).expand(reps, blk, h))
    # The very last rows, on the host as well.
    tail = out[-blk:].cpu().view(torch.int32).numpy()
    assert np.array_equal(tail, want)


def test_all_shares_inputs_beyond_4gib(gpu):
    # Each rank's whole input (both shares' row blocks) is just over 4 GiB and
    # each share's output too, so the shares run as one launch each (large
    # shares) on the 64-bit-offset kernel, at row-block offsets past 2^32.
    # Every rank's input is one 64-row block repeated, so every share is the
    # oracle's result for those blocks, repeated.
    w, h, rows, blk = 2, 8192, 262208, 64  # w * rows * h = 4.296e9 > 2^32
    wl = workloads.Workload("large_all", w, w * blk, h, "e4m3fn", "e8m0_block32", "bf16",
                            x_dist="normal", x_param=40, scale_lo=110, scale_hi=140, seed=41)
    xs, ss = workloads.generate(wl)  # one [64, H] block per rank
    want = oracle.reduce_scatter_share(xs, ss, "e4m3fn", "e8m0_block32", "bf16")
    log(f"[large] all shares: W={w}, each rank's input [{w * rows}, {h}] ({w * rows * h / 2**30:.2f} GiB)")
    reps = w * rows // blk
    dx = [torch.from_numpy(x).cuda().repeat(reps, 1) for x in xs]
    ds = [torch.from_numpy(s).cuda().repeat(reps, 1) for s in ss]
    assert dx[0].numel() > 2**32
    outs = [torch.empty((rows, h), dtype=torch.bfloat16, device="cuda") for _ in range(w)]
    p = qrs.plan(w, w * rows, h, "e4m3fn", "e8m0_block32", "bf16")
    qrs.run_all_shares(p, dx, ds, outs)
    torch.cuda.synchronize()
    del dx, ds
    want_t = torch.from_numpy(want.view(np.int16)).cuda()
    for j, o in enumerate(outs):
        got = o.view(torch.int16).view(rows // blk, blk, h)
        assert torch.equal(got, want_t.unsqueeze(0).expand(rows // blk, blk, h)), f"share {j}"


def test_bf16_output_beyond_4gib(gpu):
    # A 16-bit output past 4 GiB takes the 64-bit-offset flat kernel; with
    # fp32 group scales that kernel pairs pieces across the wave's halves
    # before storing. One 64-row block repeated, checked as above.
    w, h, rows, blk = 2, 8192, 262208, 64  # output rows * h * 2 bytes = 4.0005 GiB
    wl = workloads.Workload("large16", w, w * blk, h, "int8", "f32_group128", "bf16",
                            x_dist="int_uniform", x_param=127, scale_lo=-8, scale_hi=0, seed=37)
    xs, ss = workloads.generate(wl)
    want = oracle.reduce_scatter_share(xs, ss, "int8", "f32_group128", "bf16").view(np.int16)
    log(f"[large] int8/f32_group128 -> bf16: {rows} x {h} ({rows * h * 2 / 2**30:.3f} GiB output)")
    reps = rows // blk
    dx = [torch.from_numpy(x).cuda().repeat(reps, 1) for x in xs]
    ds = [torch.from_numpy(s).cuda().repeat(reps, 1) for s in ss]
    out = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")
    assert out.numel() * 2 > 2**32
    p = qrs.plan(w, w * rows, h, "int8", "f32_group128", "bf16")
    qrs.run(p, dx, ds, out)
    torch.cuda.synchronize()
    del dx, ds
    want_t = torch.from_numpy(want).cuda()
    got = out.view(torch.int16).view(reps, blk, h)
    assert torch.equal(got, want_t.unsqueeze(0).expand(reps, blk, h))
