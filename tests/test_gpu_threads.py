"""Host threads: a plan is immutable and a prepared launch read-only after
creation, so several threads may use them at once (the C calls release
Python's lock). Each thread's outputs must be what one thread alone
computes."""

import threading

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import assert_parity, empty_out, oracle_bits, out_bits, to_device

pytestmark = pytest.mark.gpu


def _problem(seed, rows=96):
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * rows, seed=seed)
    xs, ss = workloads.generate(wl)
    return wl, xs, ss


def _run_threads(fns):
    errors = []

    def wrap(f):
        try:
            f()
        except BaseException as e:  # reported on the main thread
            errors.append(e)

    ts = [threading.Thread(target=wrap, args=(f,)) for f in fns]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    if errors:
        raise errors[0]


def test_one_plan_from_several_threads(gpu):
    # 1152 rows: 4608 piece blocks, so every call also takes the residency
    # cap (the cached device sizes and static LDS) while the others do.
    rows = 1152
    wl, _, _ = _problem(1, rows)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    assert qrs.run_launch_info(p)["blocks_per_cu_cap"] > 0
    jobs = []
    for k in range(4):
        _, xs, ss = _problem(100 + k, rows)
        dx, ds = to_device(xs, ss)
        ref = empty_out(wl.rows, wl.h, wl.out_dtype)
        qrs.run(p, dx, ds, ref)  # one thread alone
        jobs.append((xs, ss, dx, ds, empty_out(wl.rows, wl.h, wl.out_dtype), ref, torch.cuda.Stream()))
    torch.cuda.synchronize()

    def worker(job):
        _, _, dx, ds, out, _, s = job
        with torch.cuda.stream(s):
            for _ in range(50):
                qrs.run(p, dx, ds, out)
        s.synchronize()

    _run_threads([lambda j=j: worker(j) for j in jobs])
    torch.cuda.synchronize()
    for xs, ss, _, _, out, ref, _ in jobs:
        assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
        sample = np.array([0, 1, rows // 2, rows - 1])
        want = oracle.reduce_scatter_share([x[sample] for x in xs], [s_[sample] for s_ in ss], wl.x_format,
                                           wl.scale_layout, wl.out_dtype)
        assert_parity(out_bits(out)[sample], oracle_bits(want, wl.out_dtype), wl.out_dtype, "thread")


def test_one_prepared_launch_from_several_threads(gpu):
    wl, xs, ss = _problem(7)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = to_device(xs, ss)
    out = empty_out(wl.rows, wl.h, wl.out_dtype).fill_(float("nan"))
    launch = qrs.Launch(p, dx, ds, out)  # torch's current stream: every enqueue goes there

    def worker():
        for _ in range(50):
            launch()

    _run_threads([worker] * 4)
    torch.cuda.synchronize()
    want = oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
    assert_parity(out_bits(out), oracle_bits(want, wl.out_dtype), wl.out_dtype, "shared handle")
