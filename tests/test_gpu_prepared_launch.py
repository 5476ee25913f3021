"""GPU: the prepared launch (qrs_launch_create / qrs_launch_enqueue) gives
the bytes qrs_run gives, on every launch form qrs_run uses for a share:
8-element pieces with preloaded arguments (MX scales; fp32 output from
W = 4), 16-element chunks (fp32 group scales; MX fp32 output at W = 2),
capped and uncapped grids, ragged tails. The handle keeps what it needs
from the plan, so it still runs after the plan is destroyed."""

import ctypes

import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import assert_parity, empty_out, oracle_bits, out_bits, to_device

pytestmark = pytest.mark.gpu

CASES = [
    (8, 2048, 8192, "e4m3fn", "e8m0_block32", "bf16"),  # pieces, 8192 blocks: capped
    (8, 24, 1152, "e5m2", "e8m0_block32", "f32"),       # fp32 pieces, a partial wave
    (4, 37, 1024, "e4m3fn", "e8m0_block32", "f32"),     # fp32 pieces at W = 4
    (2, 53, 1024, "e5m2", "e8m0_block32", "f32"),       # chunks at W = 2
    (8, 61, 7168, "e5m2", "f32_group128", "bf16"),      # chunks, swapped 16-bit stores
    (2, 4096, 8192, "int8", "f32_group128", "f32"),     # chunks, 8192 blocks: capped
]


@pytest.mark.parametrize("w,rows,h,xf,sl,od", CASES)
def test_prepared_launch_matches_run(gpu, w, rows, h, xf, sl, od):
    wl = workloads.Workload("prepared", w, rows * w, h, xf, sl, od,
                            x_dist="int_uniform" if xf == "int8" else "normal",
                            x_param=127 if xf == "int8" else 40,
                            scale_lo=-10 if sl == "f32_group128" else 110,
                            scale_hi=2 if sl == "f32_group128" else 140, seed=991 + rows)
    xs, ss = workloads.generate(wl)
    dx, ds = to_device(xs, ss)
    p = qrs.plan(w, rows * w, h, xf, sl, od)
    ref = empty_out(rows, h, od)
    qrs.run(p, dx, ds, ref)
    out = empty_out(rows, h, od).fill_(float("nan"))
    launch = qrs.Launch(p, dx, ds, out)
    launch()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
    out.fill_(float("nan"))
    launch()  # the handle is reusable
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
    if rows * h <= (1 << 20):
        want = oracle.reduce_scatter_share(xs, ss, xf, sl, od)
        assert_parity(out_bits(out), oracle_bits(want, od), od, "prepared launch")


def test_prepared_launch_outlives_its_plan(gpu):
    lib = qrs.load_library()
    w, rows, h = 8, 64, 1024
    wl = workloads.Workload("prepared", w, rows * w, h, "e4m3fn", "e8m0_block32", "bf16", x_dist="normal",
                            x_param=40, scale_lo=110, scale_hi=140, seed=5)
    xs, ss = workloads.generate(wl)
    dx, ds = to_device(xs, ss)
    out = empty_out(rows, h, "bf16").fill_(float("nan"))
    plan = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    assert lib.qrs_plan(w, rows * w, h, int(qrs.XDtype.FP8_E4M3FN), int(qrs.ScaleLayout.E8M0_BLOCK32),
                        int(qrs.OutDtype.BF16), ctypes.byref(plan), ctypes.byref(ws)) == qrs.Status.OK
    xa = (ctypes.c_void_p * w)(*[t.data_ptr() for t in dx])
    sa = (ctypes.c_void_p * w)(*[t.data_ptr() for t in ds])
    stream = torch.cuda.current_stream().cuda_stream
    handle = ctypes.c_void_p()
    assert lib.qrs_launch_create(plan, xa, sa, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream),
                                 ctypes.byref(handle)) == qrs.Status.OK
    assert handle.value
    assert lib.qrs_plan_destroy(plan) == qrs.Status.OK
    assert lib.qrs_launch_enqueue(handle) == qrs.Status.OK
    torch.cuda.synchronize()
    assert lib.qrs_launch_destroy(handle) == qrs.Status.OK
    want = oracle.reduce_scatter_share(xs, ss, "e4m3fn", "e8m0_block32", "bf16")
    assert_parity(out_bits(out), oracle_bits(want, "bf16"), "bf16", "after plan destroyed")
