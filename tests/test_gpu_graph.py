"""The launches allocate nothing, set no memory and synchronise nothing, so
they can be captured in a HIP graph (torch.cuda.CUDAGraph). Each graph is
replayed several times with eager work in between, and every replay is
checked against the eager result."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import assert_parity, empty_out, oracle_bits, out_bits
from oracle.quantize import quantize as oracle_quantize

pytestmark = pytest.mark.gpu


def _replay_and_check(graph, outs, want_bits, fill):
    for rep in range(3):
        for o in outs:
            o.fill_(fill)  # eager work between replays: the replay must rewrite every element
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want_bits):
            assert np.array_equal(o.cpu().view(torch.uint8).numpy(), w), f"replay {rep}"


def test_share_in_a_graph(gpu):
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * 64)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = qrs.alloc_slices(p)
    for t, a in zip(dx, xs):
        t.copy_(torch.from_numpy(a))
    for t, a in zip(ds, ss):
        t.copy_(torch.from_numpy(a))
    out = empty_out(wl.rows, wl.h, wl.out_dtype)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qrs.run(p, dx, ds, out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert_parity(out_bits(out), want, wl.out_dtype, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qrs.run(p, dx, ds, out)
    _replay_and_check(g, [out], [want.view(np.uint8).reshape(wl.rows, -1)], float("nan"))


def test_quantize_then_all_shares_in_one_graph(gpu):
    w, bs, h = 4, 4 * 16, 2048
    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(world_size=w, bs=bs, h=h)
    acts = [workloads.generate_activations(wl, r) for r in range(w)]
    xin = [torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda() for a in acts]
    p = qrs.plan(w, bs, h, "e4m3fn", "e8m0_block32", "f32")
    codes, scales = qrs.alloc_slices(p, full_inputs=True)
    outs = [empty_out(bs // w, h, "f32") for _ in range(w)]
    q = [oracle_quantize(a, "e4m3fn", "e8m0_block32") for a in acts]
    want = oracle.all_shares([c for c, _ in q], [s for _, s in q], "e4m3fn", "e8m0_block32", "f32")
    want_bits = [np.ascontiguousarray(x).view(np.uint8).reshape(bs // w, -1) for x in want]

    def pipeline():
        for r in range(w):
            qrs.quantize(xin[r], codes[r], scales[r], "e4m3fn", "e8m0_block32")
        qrs.run_all_shares(p, codes, scales, outs)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pipeline()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for o, wb in zip(outs, want_bits):
        assert np.array_equal(o.cpu().view(torch.uint8).numpy(), wb), "eager"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline()
    for c in codes:
        c.zero_()  # the replay must also redo the quantization
    _replay_and_check(g, outs, want_bits, float("nan"))


@pytest.mark.parametrize("name", ["w8_bs16384_h8192_mx_e4m3_bf16", "w8_bs65536_h5120_mx_e5m2_f32"])
def test_prepared_launch_in_a_graph(gpu, name):
    """A prepared launch (qrs_launch_create on the capture stream) captured
    twice in one graph: the contiguous piece kernel with preloaded
    arguments, 16-bit and fp32 outputs."""
    wl = workloads.WORKLOADS[name].with_(bs=8 * 48)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = qrs.alloc_slices(p)
    for t, a in zip(dx, xs):
        t.copy_(torch.from_numpy(a))
    for t, a in zip(ds, ss):
        t.copy_(torch.from_numpy(a))
    out = empty_out(wl.rows, wl.h, wl.out_dtype)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    launch = qrs.Launch(p, dx, ds, out, stream=s)
    launch()  # warm-up on the capture stream
    torch.cuda.synchronize()
    assert_parity(out_bits(out), want, wl.out_dtype, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launch()
        launch()
    _replay_and_check(g, [out], [want.view(np.uint8).reshape(wl.rows, -1)], float("nan"))
