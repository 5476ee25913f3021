"""GPU parity of qrs_run_strided: slices and outputs that are row ranges of
wider buffers (column windows of [rows, H_total] tensors)."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import OUT_TORCH, assert_parity, oracle_bits, out_bits

pytestmark = pytest.mark.gpu

MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


def _case(w, rows, h, x_format, scale_layout, out_dtype, extra_cols, c0, seed):
    g = 128 if scale_layout == "f32_group128" else 32
    ht = h + extra_cols
    wl = workloads.Workload("strided", w, rows * w, ht, x_format, scale_layout, out_dtype,
                            x_dist="int_uniform" if x_format == "int8" else "normal",
                            x_param=127 if x_format == "int8" else 30,
                            scale_lo=-10 if scale_layout == "f32_group128" else 110,
                            scale_hi=2 if scale_layout == "f32_group128" else 140, seed=seed)
    xs_full, ss_full = workloads.generate(wl)  # [rows, ht] per rank
    xs = [x[:, c0:c0 + h] for x in xs_full]
    ss = [s[:, c0 // g:(c0 + h) // g] for s in ss_full]
    want = oracle.reduce_scatter_share([np.ascontiguousarray(x) for x in xs], [np.ascontiguousarray(s) for s in ss],
                                       x_format, scale_layout, out_dtype)
    dx_full = [torch.from_numpy(x).cuda() for x in xs_full]
    ds_full = [torch.from_numpy(s).cuda() for s in ss_full]
    dx = [t[:, c0:c0 + h] for t in dx_full]
    ds = [t[:, c0 // g:(c0 + h) // g] for t in ds_full]
    oc0 = 64
    out_full = torch.full((rows, h + 192), float("nan"), dtype=OUT_TORCH[out_dtype], device="cuda")
    out = out_full[:, oc0:oc0 + h]
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    qrs.run_strided(p, dx, ds, out)
    torch.cuda.synchronize()
    got = out_bits(out.contiguous())
    assert_parity(got, oracle_bits(want, out_dtype), out_dtype, f"W={w} H={h} {x_format}/{scale_layout}->{out_dtype}")
    # Nothing outside the window was written.
    full_bits = out_bits(out_full)
    pad = np.concatenate([full_bits[:, :oc0], full_bits[:, oc0 + h:]], axis=1)
    sentinel = out_bits(torch.full((1, 1), float("nan"), dtype=OUT_TORCH[out_dtype]))[0, 0]
    assert np.all(pad == sentinel)
    # Same bits as qrs_run on contiguous copies.
    out2 = torch.empty((rows, h), dtype=OUT_TORCH[out_dtype], device="cuda")
    qrs.run(p, [t.contiguous() for t in dx], [t.contiguous() for t in ds], out2)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(out2), got)


@pytest.mark.parametrize("x_format,scale_layout", MODES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("w", [2, 8])
def test_column_window(gpu, x_format, scale_layout, out_dtype, w):
    _case(w, 7, 1152, x_format, scale_layout, out_dtype, extra_cols=384, c0=128, seed=w)


@pytest.mark.parametrize("h", [1024, 5120, 8192])
def test_wide_rows_and_equal_stride(gpu, h):
    _case(4, 5, h, "e4m3fn", "e8m0_block32", "f32", extra_cols=256, c0=256, seed=h)
    _case(4, 3, h, "e5m2", "f32_group128", "bf16", extra_cols=0, c0=0, seed=h + 1)  # stride == H


def test_strided_rejects_mismatched_strides(gpu):
    p = qrs.plan(2, 8, 1024, "e4m3fn", "e8m0_block32", "f32")
    a = torch.zeros(4, 2048, dtype=torch.uint8, device="cuda")
    b = torch.zeros(4, 1024 + 512, dtype=torch.uint8, device="cuda")
    s = [torch.zeros(4, 32, dtype=torch.uint8, device="cuda") for _ in range(2)]
    out = torch.zeros(4, 1024, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        qrs.run_strided(p, [a[:, :1024], b[:, :1024]], s, out)


def test_strided_rejects_element_sizes_of_another_mode(gpu):
    # The strides and row lengths are counted in the mode's elements: a view
    # of 1-byte elements as the bf16 output (or as fp32 scales) would make the
    # kernel address twice (four times) the view's rows. Rejected before any
    # launch, as are Launch objects built from them.
    p = qrs.plan(2, 8, 1024, "e4m3fn", "f32_group128", "bf16")
    xs = [torch.zeros(4, 1024, dtype=torch.uint8, device="cuda") for _ in range(2)]
    s32 = [torch.zeros(4, 8, dtype=torch.float32, device="cuda") for _ in range(2)]
    s8 = [torch.zeros(4, 8, dtype=torch.uint8, device="cuda") for _ in range(2)]
    out16 = torch.zeros(4, 1024, dtype=torch.bfloat16, device="cuda")
    out8 = torch.zeros(4, 1024, dtype=torch.uint8, device="cuda")
    x16 = [torch.zeros(4, 1024, dtype=torch.int16, device="cuda") for _ in range(2)]
    for bad in ((xs, s32, out8), (xs, s8, out16), (x16, s32, out16)):
        with pytest.raises(ValueError, match="elements expected"):
            qrs.run_strided(p, *bad)
        with pytest.raises(ValueError, match="elements expected"):
            qrs.StridedLaunch(p, *bad)
    qrs.run_strided(p, xs, s32, out16)  # the matching sizes are accepted
    torch.cuda.synchronize()
    assert torch.count_nonzero(out16.view(torch.int16)) == 0


@pytest.mark.parametrize("h,rows", [(1152, 61), (7168, 9), (5120, 13), (1024, 33)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_rows_crossing_waves_and_blocks(gpu, h, rows, out_dtype):
    # Rows of H/16 chunks that are not a multiple of a wave's 64 chunks or a
    # block's 256: waves and blocks start mid-row and span row ends.
    _case(8, rows, h, "e5m2", "e8m0_block32", out_dtype, extra_cols=128, c0=128, seed=h + rows)
    _case(2, rows, h, "int8", "f32_group128", out_dtype, extra_cols=256, c0=0, seed=h + rows + 1)


@pytest.mark.parametrize("h,rows", [(5120, 37), (7168, 70), (1152, 300), (3200, 150)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_xcd_runs_over_whole_rows(gpu, h, rows, out_dtype):
    # MX scale windows that start mid-line (c0 = 160 columns: 5 bytes into a
    # scale row) make the row-strided piece launch hand each XCD runs of
    # lcm(H/8, 256) / 256 consecutive blocks (5, 7, 9 and 25 here). These
    # grids hold full sets of eight runs plus a tail of blocks left in
    # hardware order: every element must still be written once, correctly.
    _case(8, rows, h, "e4m3fn", "e8m0_block32", out_dtype, extra_cols=256, c0=160, seed=h * 7 + rows)


@pytest.mark.parametrize("name", ["w8_bs65536_h5120_mx_e5m2_f32", "w8_bs8192_h7168_e5m2_bf16"])
def test_full_size_row_interleaved_receive_buffer(gpu, name):
    # The W slices interleaved by row in one [rows, W, H] buffer (and the
    # scales in [rows, W, H/G]): every slice is a row-strided view. Sampled
    # rows against the oracle, the whole output against qrs_run on the same
    # values in contiguous slices.
    wl = workloads.WORKLOADS[name]
    xs, ss = workloads.generate(wl)
    w, rows, h = wl.world_size, wl.rows, wl.h
    bx = torch.empty((rows, w, h), dtype=torch.uint8, device="cuda")
    bs = torch.empty((rows, w) + ss[0].shape[1:], dtype=torch.float32 if ss[0].dtype == np.float32 else torch.uint8,
                     device="cuda")
    for r in range(w):
        bx[:, r, :].copy_(torch.from_numpy(xs[r]))
        bs[:, r, :].copy_(torch.from_numpy(ss[r]))
    p = qrs.plan(w, wl.bs, h, wl.x_format, wl.scale_layout, wl.out_dtype)
    out = torch.empty((rows, h), dtype=OUT_TORCH[wl.out_dtype], device="cuda")
    qrs.run_strided(p, [bx[:, r, :] for r in range(w)], [bs[:, r, :] for r in range(w)], out)
    torch.cuda.synchronize()
    got = out_bits(out)
    # The prepared launch (arguments marshalled once) gives the same bytes.
    out3 = torch.empty_like(out)
    qrs.StridedLaunch(p, [bx[:, r, :] for r in range(w)], [bs[:, r, :] for r in range(w)], out3)()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out3.view(torch.uint8))
    sample = np.unique(np.concatenate([[0, 1, rows - 1], np.random.default_rng(5).integers(0, rows, 13)]))
    want = oracle.reduce_scatter_share([x[sample] for x in xs], [s[sample] for s in ss], wl.x_format,
                                       wl.scale_layout, wl.out_dtype)
    assert_parity(got[sample], oracle_bits(want, wl.out_dtype), wl.out_dtype, name)
    del bx, bs
    dx = [torch.from_numpy(x).cuda() for x in xs]
    ds = [torch.from_numpy(s).cuda() for s in ss]
    out2 = torch.empty_like(out)
    qrs.run(p, dx, ds, out2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
