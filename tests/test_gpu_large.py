"""Largest shapes, checked against the oracle on a repeating row block:
outputs and inputs past 4 GiB (byte offsets beyond 2^32), and shares and
quantizations past 2^34 elements, which run as several launches (a HIP grid
holds fewer than 2^32 work-items along a dimension), up to a row-strided
share past 2^35 elements."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from oracle.quantize import quantize as oracle_quantize
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


def _free_or_skip(need):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < need + (8 << 30):
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free")


def _equal_repeated(got, block, what):
    """got: [reps * blk, W] device tensor (any row stride) that must hold the
    [blk, W] device tensor `block` reps times over; compared a few hundred MB
    at a time."""
    blk, width = block.shape
    reps = got.shape[0] // blk
    g = got.view(reps, blk, width)
    step = max(1, (1 << 28) // (blk * width))
    for i in range(0, reps, step):
        part = g[i:i + step]
        assert torch.equal(part, block.unsqueeze(0).expand_as(part)), f"{what}: rows {i * blk} to {(i + step) * blk}"


def test_strided_share_past_2_35_elements(gpu):
    # rows * H = 2^35 + 2^23 elements. One launch of 8-element pieces would
    # hold more than 2^32 lanes, which a HIP grid cannot; the share runs as
    # launches of whole rows (2^21, 2^21 and 1024 rows). Rows are padded in
    # every tensor; the scale rows (264 bytes apart) are off 128-byte lines.
    w, h, blk = 2, 8192, 64
    rows = (1 << 22) + 1024
    x_ld, s_ld, o_ld = h + 128, h // 32 + 8, h + 64
    _free_or_skip(w * rows * (x_ld + s_ld) + rows * o_ld * 2)
    wl = workloads.Workload("large_strided", w, w * blk, h, "e4m3fn", "e8m0_block32", "bf16",
                            x_dist="normal", x_param=40, scale_lo=110, scale_hi=140, seed=43)
    xs, ss = workloads.generate(wl)  # one [64, H] block per rank
    want = oracle.reduce_scatter_share(xs, ss, "e4m3fn", "e8m0_block32", "bf16").view(np.int16)
    log(f"[large] strided share: W={w}, {rows} x {h} ({rows * h / 2**35:.4f} x 2^35 elements)")
    reps = rows // blk
    dx, ds = [], []
    for x, s in zip(xs, ss):
        xb = torch.empty((rows, x_ld), dtype=torch.uint8, device="cuda")
        xb.view(reps, blk, x_ld)[:, :, :h].copy_(torch.from_numpy(x).cuda().unsqueeze(0).expand(reps, blk, h))
        dx.append(xb[:, :h])
        sb = torch.empty((rows, s_ld), dtype=torch.uint8, device="cuda")
        sb.view(reps, blk, s_ld)[:, :, :h // 32].copy_(
            torch.from_numpy(s).cuda().unsqueeze(0).expand(reps, blk, h // 32))
        ds.append(sb[:, :h // 32])
    ob = torch.full((rows, o_ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = ob[:, :h]
    p = qrs.plan(w, w * rows, h, "e4m3fn", "e8m0_block32", "bf16")
    qrs.run_strided(p, dx, ds, out)
    torch.cuda.synchronize()
    del dx, ds, xb, sb
    _equal_repeated(out.view(torch.int16), torch.from_numpy(want).cuda(), "strided share")
    assert bool(torch.isnan(ob[:, h:]).all()), "wrote outside the output rows"
    del ob, out
    torch.cuda.empty_cache()


def test_share_in_two_launches(gpu):
    # rows * H = 2^34 + 2^19 elements: a launch of 2^34 elements (an output
    # past 4 GiB, 64-bit offsets) and one of 2^19 (8-element pieces), by
    # qrs_run and by a prepared launch.
    w, h, blk = 2, 8192, 64
    rows = (1 << 21) + 64
    _free_or_skip(w * rows * h * 33 // 32 + rows * h * 2)
    wl = workloads.Workload("large_parts", w, w * blk, h, "e5m2", "e8m0_block32", "f16",
                            x_dist="normal", x_param=30, scale_lo=100, scale_hi=125, seed=47)
    xs, ss = workloads.generate(wl)
    want = torch.from_numpy(oracle.reduce_scatter_share(xs, ss, "e5m2", "e8m0_block32", "f16").view(np.int16))
    p = qrs.plan(w, w * rows, h, "e5m2", "e8m0_block32", "f16")
    assert qrs.run_launch_info(p)["launches"] == 2
    log(f"[large] share in two launches: W={w}, {rows} x {h}")
    reps = rows // blk
    dx = [torch.from_numpy(x).cuda().repeat(reps, 1) for x in xs]
    ds = [torch.from_numpy(s).cuda().repeat(reps, 1) for s in ss]
    out = torch.full((rows, h), float("nan"), dtype=torch.float16, device="cuda")
    qrs.run(p, dx, ds, out)
    torch.cuda.synchronize()
    want = want.cuda()
    _equal_repeated(out.view(torch.int16), want, "qrs_run")
    out.fill_(float("nan"))
    log("[large] the same share, prepared launch")
    step = qrs.Launch(p, dx, ds, out)
    step()
    torch.cuda.synchronize()
    _equal_repeated(out.view(torch.int16), want, "prepared launch")
    del step, dx, ds, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("x_format,scale_layout", [("e4m3fn", "e8m0_block32"), ("int8", "f32_group128")])
def test_quantize_in_two_launches(gpu, x_format, scale_layout):
    # tokens * H = 2^34 + 2^19 elements: two launches, the second starting
    # 2^34 elements (2^29 scale bytes) in.
    tokens, h, blk = (1 << 21) + 64, 8192, 64
    g = 128 if scale_layout == "f32_group128" else 32
    _free_or_skip(tokens * h * 3 + tokens * h // 32)
    rng = np.random.default_rng(53)
    v = rng.standard_normal((blk, h)).astype(np.float32) * np.exp2(rng.integers(-30, 30, size=(blk, 1)))
    bits = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_c, want_s = oracle_quantize(bits, x_format, scale_layout)
    log(f"[large] quantize in two launches: [{tokens}, {h}] -> {x_format}/{scale_layout}")
    x = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16).repeat(tokens // blk, 1)
    codes = torch.empty((tokens, h), dtype=torch.uint8, device="cuda")
    if scale_layout == "f32_group128":
        scales = torch.full((tokens, h // g), float("nan"), dtype=torch.float32, device="cuda")
    else:
        scales = torch.full((tokens, h // g), 0xAA, dtype=torch.uint8, device="cuda")
    qrs.quantize(x, codes, scales, x_format, scale_layout)
    torch.cuda.synchronize()
    del x
    _equal_repeated(codes, torch.from_numpy(want_c).cuda(), "codes")
    if scale_layout == "f32_group128":
        _equal_repeated(scales.view(torch.int32), torch.from_numpy(want_s.view(np.int32)).cuda(), "scales")
    else:
        _equal_repeated(scales, torch.from_numpy(want_s).cuda(), "scales")
    del codes, scales
    torch.cuda.empty_cache()


def test_stream_copy_past_2_35_bytes(gpu):
    # The calibration copy runs as launches of 2^35 bytes (2^31 lanes of 16
    # bytes): 2^35 + 2^20 bytes take two, the second starting 32 GiB in.
    n = (1 << 35) + (1 << 20)
    _free_or_skip(2 * n)
    log(f"[large] stream copy of {n} bytes")
    src = torch.arange(n // 8, dtype=torch.int64, device="cuda")
    dst = torch.full_like(src, -1)
    qrs.stream_copy(src, dst)
    torch.cuda.synchronize()
    step = 1 << 27
    for i in range(0, n // 8, step):
        assert torch.equal(dst[i:i + step], src[i:i + step]), f"words {i} to {i + step}"
    del src, dst
    torch.cuda.empty_cache()
