"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every output type must match exactly: fp32 bit for bit, and bf16 / fp16
too, since both sides round the same binary32 accumulator to nearest-even (a
1-ulp bound would be the weaker contract). The five workloads run at their
full sizes and are compared element by element and against the stored
digests of the oracle's output; a sweep covers every mode, world size and
several H at small, ragged row counts.
"""

import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_parity, empty_out, log, oracle_bits, out_bits, run_gpu, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "digests.json")

MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_workload_full_size(gpu, name):
    """Every element of each workload at full size, with the slices placed
    as the benchmark places them (one buffer, recommended pitch)."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS[name]
    log(f"[parity] {name}: W={wl.world_size} BS={wl.bs} H={wl.h} {wl.x_format}/{wl.scale_layout}->{wl.out_dtype}")
    xs, ss = workloads.generate(wl)
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = qrs.alloc_slices(p)
    for t, a in zip(dx, xs):
        t.copy_(torch.from_numpy(a))
    for t, a in zip(ds, ss):
        t.copy_(torch.from_numpy(a))
    out = empty_out(wl.rows, wl.h, wl.out_dtype).fill_(float("nan"))
    qrs.Launch(p, dx, ds, out)()  # the call the benchmark times
    torch.cuda.synchronize()
    got = out_bits(out)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    n_diff = assert_parity(got, want, wl.out_dtype, name)
    log(f"[parity] {name}: {got.size} elements, {n_diff} not bit-identical")
    assert n_diff == 0
    with open(GOLDEN) as f:
        digest = json.load(f)["configs"][name]["output_sha256"]
    assert hashlib.sha256(got.tobytes()).hexdigest() == digest


@pytest.mark.parametrize("x_format,scale_layout", MODES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("w", [2, 4, 8])
@pytest.mark.parametrize("h", [1024, 1152, 5120, 8192])
def test_sweep_small_ragged(gpu, x_format, scale_layout, out_dtype, w, h):
    # rows chosen so the element count is not a multiple of a block's span.
    rows = 3 if h == 8192 else 5
    wl = workloads.Workload(
        "sweep", w, rows * w, h, x_format, scale_layout, out_dtype,
        x_dist="int_uniform" if x_format == "int8" else "normal",
        x_param=127 if x_format == "int8" else (64 if x_format == "e4m3fn" else 2048),
        scale_lo=-20 if scale_layout == "f32_group128" else 100,
        scale_hi=4 if scale_layout == "f32_group128" else 150,
        seed=1000 + w * 7 + h,
    )
    xs, ss = workloads.generate(wl)
    got = run_gpu(w, rows, h, x_format, scale_layout, out_dtype, xs, ss)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
    assert_parity(got, want, out_dtype, f"W={w} H={h} {x_format}/{scale_layout}->{out_dtype}")


@pytest.mark.parametrize("rows", [1, 2, 7, 63, 64, 65, 257])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("base", ["w8_bs16384_h8192_mx_e4m3_bf16", "w8_bs8192_h7168_e5m2_bf16"])
def test_row_counts_around_block_edges(gpu, rows, out_dtype, base):
    # H = 1152 is 72 chunks a row: waves and blocks end mid-row and the grid's
    # last wave is partial, for every store path (direct, LDS-staged, swapped).
    wl = workloads.WORKLOADS[base].with_(bs=8 * rows, h=1152, out_dtype=out_dtype)
    xs, ss = workloads.generate(wl)
    got = run_gpu(8, rows, 1152, wl.x_format, wl.scale_layout, out_dtype, xs, ss)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, out_dtype), out_dtype)
    assert_parity(got, want, out_dtype, f"rows={rows}")


def test_non_finite_and_extreme_codes(gpu):
    """Every code including NaN / inf, every E8M0 code including 0 and 255,
    fp32 scales with zeros, negatives, subnormals and huge values."""
    rng = np.random.default_rng(99)
    for x_format, scale_layout in MODES:
        for out_dtype in ("f32", "bf16", "f16"):
            w, rows, h = 4, 16, 1024
            g = 128 if scale_layout == "f32_group128" else 32
            xs = [rng.integers(0, 256, size=(rows, h), dtype=np.uint8) for _ in range(w)]
            if scale_layout == "f32_group128":
                bits = rng.integers(0, 2**32, size=(w, rows, h // g), dtype=np.uint64).astype(np.uint32)
                ss = [b.view(np.float32) for b in bits]
            else:
                ss = [rng.integers(0, 256, size=(rows, h // g), dtype=np.uint8) for _ in range(w)]
            got = run_gpu(w, rows, h, x_format, scale_layout, out_dtype, xs, ss)
            want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
            assert_parity(got, want, out_dtype, f"{x_format}/{scale_layout}->{out_dtype}")


def test_slices_in_separate_allocations_and_one_buffer(gpu):
    """The pointer-array form: separate tensors per rank, or views into one
    [W, rows, H] buffer, give the same bits."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w8_bs8192_h7168_e5m2_bf16"].with_(bs=8 * 40, h=2048)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = to_device(xs, ss)
    o1 = empty_out(wl.rows, wl.h, wl.out_dtype)
    qrs.run(p, dx, ds, o1)
    bx = torch.stack(dx)
    bs_ = torch.stack(ds)
    o2 = empty_out(wl.rows, wl.h, wl.out_dtype)
    qrs.run(p, [bx[r] for r in range(8)], [bs_[r] for r in range(8)], o2)
    # Fresh copies at other addresses: only the pointer array fixes which slice is which rank.
    o3 = empty_out(wl.rows, wl.h, wl.out_dtype)
    qrs.run(p, [t.clone() for t in dx], [t.clone() for t in ds], o3)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(o1), out_bits(o2))
    assert np.array_equal(out_bits(o1), out_bits(o3))


def test_runs_on_the_given_stream(gpu):
    """The kernel is ordered after earlier work on a non-default stream."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(bs=4 * 256)
    xs, ss = workloads.generate(wl)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    p = qrs.plan(4, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    s = torch.cuda.Stream()
    dx = [torch.zeros(wl.rows, wl.h, dtype=torch.uint8, device="cuda") for _ in range(4)]
    ds = [torch.zeros(wl.rows, wl.h // 128, dtype=torch.float32, device="cuda") for _ in range(4)]
    hx = [torch.from_numpy(x).pin_memory() for x in xs]
    hs = [torch.from_numpy(v).pin_memory() for v in ss]
    out = empty_out(wl.rows, wl.h, wl.out_dtype)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        # Big slow-ish work first on the same stream, then the copies, then the run.
        junk = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        for _ in range(4):
            junk.mul_(1.0001)
        for r in range(4):
            dx[r].copy_(hx[r], non_blocking=True)
            ds[r].copy_(hs[r], non_blocking=True)
        qrs.run(p, dx, ds, out)  # current stream is s
    s.synchronize()
    assert_parity(out_bits(out), want, wl.out_dtype, "stream order")


def test_one_plan_on_two_streams_at_once(gpu):
    """A plan is immutable: launches of one plan interleaved on two streams,
    with different inputs, each give their own oracle result."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w8_bs8192_h7168_e5m2_bf16"].with_(bs=8 * 96)
    cases = [workloads.generate(wl), workloads.generate(wl.with_(seed=9))]
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    dev_in = [to_device(xs, ss) for xs, ss in cases]
    outs = [[empty_out(wl.rows, wl.h, wl.out_dtype).fill_(float("nan")) for _ in range(4)] for _ in cases]
    torch.cuda.synchronize()
    for i in range(4):
        for k in range(2):
            qrs.run(p, dev_in[k][0], dev_in[k][1], outs[k][i], stream=streams[k])
    torch.cuda.synchronize()
    for k, (xs, ss) in enumerate(cases):
        want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype),
                           wl.out_dtype)
        for i in range(4):
            assert_parity(out_bits(outs[k][i]), want, wl.out_dtype, f"stream {k} launch {i}")


def test_misaligned_device_pointers_rejected(gpu):
    import quantized_collective_reduction_amd as qrs

    p = qrs.plan(2, 32, 1024, "e4m3fn", "e8m0_block32", "f32")
    x = torch.zeros(2, 16 * 1024 + 16, dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, 16 * 32 + 16, dtype=torch.uint8, device="cuda")  # room for offset views
    out = torch.zeros(16 * 1024 + 4, dtype=torch.float32, device="cuda")
    with pytest.raises(qrs.QrsError) as ei:
        qrs.run(p, [x[0, 8:].data_ptr(), x[1, :16384].data_ptr()], [s[0, :512], s[1, :512]], out[:16384])
    assert ei.value.status == qrs.Status.INVALID_ARG
    with pytest.raises(qrs.QrsError):
        qrs.run(p, [x[0, :16384], x[1, :16384]], [s[0, :512], s[1, :512]], out[1:16385].data_ptr())
    # E8M0 scales have no alignment requirement.
    qrs.run(p, [x[0, :16384], x[1, :16384]], [s[0, 1:].data_ptr(), s[1, 3:].data_ptr()], out[:16384])
    torch.cuda.synchronize()


def test_stream_copy(gpu):
    import quantized_collective_reduction_amd as qrs

    src = torch.randint(0, 255, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    qrs.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_prepared_launch_matches_run(gpu):
    """qrs.Launch (arguments marshalled once) gives the same bits as qrs.run."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w8_bs65536_h5120_mx_e5m2_f32"].with_(bs=8 * 33)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = to_device(xs, ss)
    o1 = empty_out(wl.rows, wl.h, wl.out_dtype)
    o2 = empty_out(wl.rows, wl.h, wl.out_dtype)
    qrs.run(p, dx, ds, o1)
    launch = qrs.Launch(p, dx, ds, o2)
    launch()
    launch()
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(o1), out_bits(o2))
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    assert_parity(out_bits(o2), want, wl.out_dtype, "Launch")


def test_launch_on_another_stream(gpu):
    """Launch.on_stream enqueues the same share on the given stream: the
    output appears there (after that stream's earlier work) with the bits of
    the original launch."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * 21)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx, ds = to_device(xs, ss)
    o1 = empty_out(wl.rows, wl.h, wl.out_dtype)
    launch = qrs.Launch(p, dx, ds, o1)
    launch()
    s = torch.cuda.Stream()
    side = launch.on_stream(s)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o1.view(torch.int16).fill_(-1)  # ordered before the side launch on the same stream
    side()
    s.synchronize()
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    assert_parity(out_bits(o1), want, wl.out_dtype, "Launch.on_stream")


@pytest.mark.parametrize("x_format,scale_layout", [("e4m3fn", "e8m0_block32"), ("e5m2", "f32_group128"),
                                                   ("int8", "f32_group128")])
def test_typed_float8_tensors(gpu, x_format, scale_layout):
    """The binding accepts codes and scales in torch's float8 / int8 / E8M0
    dtypes as well as raw bytes; both give the oracle's bits."""
    import quantized_collective_reduction_amd as qrs

    x_dt = {"int8": torch.int8, "e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[x_format]
    base = {"int8": "w2_bs32_h1024_int8_f32", "e5m2": "w8_bs8192_h7168_e5m2_bf16",
            "e4m3fn": "w8_bs16384_h8192_mx_e4m3_bf16"}[x_format]
    wl = workloads.WORKLOADS[base].with_(world_size=4, bs=4 * 9, h=1024, out_dtype="bf16")
    assert (wl.x_format, wl.scale_layout) == (x_format, scale_layout)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(4, wl.bs, wl.h, x_format, scale_layout, "bf16")
    dx, ds = to_device(xs, ss)
    typed_x = [t.view(x_dt) for t in dx]
    typed_s = [t.view(torch.float8_e8m0fnu) for t in ds] if scale_layout == "e8m0_block32" else ds
    o_raw = empty_out(wl.rows, wl.h, "bf16")
    o_typed = empty_out(wl.rows, wl.h, "bf16")
    qrs.run(p, dx, ds, o_raw)
    qrs.run(p, typed_x, typed_s, o_typed)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(o_raw), out_bits(o_typed))
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, "bf16"), "bf16")
    assert_parity(out_bits(o_typed), want, "bf16", f"typed {x_format}/{scale_layout}")


@pytest.mark.parametrize("full", [False, True])
def test_recommended_slice_placement(gpu, full):
    """Slices placed by qrs.alloc_slices (one buffer, recommended pitch) give
    the oracle's bits, for this GPU's share and for all shares."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * 12, h=2048)
    p = qrs.plan(8, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    xs, ss = workloads.generate_full(wl) if full else workloads.generate(wl)
    dx, ds = qrs.alloc_slices(p, full_inputs=full)
    for t, a in zip(dx, xs):
        t.copy_(torch.from_numpy(a))
    for t, a in zip(ds, ss):
        t.copy_(torch.from_numpy(a))
    xp, sp = qrs.slice_pitch(p, full_inputs=full)
    assert dx[1].data_ptr() - dx[0].data_ptr() == xp and ds[1].data_ptr() - ds[0].data_ptr() == sp
    if full:
        outs = [empty_out(wl.rows, wl.h, wl.out_dtype) for _ in range(8)]
        qrs.run_all_shares(p, dx, ds, outs)
        torch.cuda.synchronize()
        want = oracle.all_shares(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
        for j in range(8):
            assert_parity(out_bits(outs[j]), oracle_bits(want[j], wl.out_dtype), wl.out_dtype, f"share {j}")
    else:
        out = empty_out(wl.rows, wl.h, wl.out_dtype)
        qrs.run(p, dx, ds, out)
        torch.cuda.synchronize()
        want = oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
        assert_parity(out_bits(out), oracle_bits(want, wl.out_dtype), wl.out_dtype, "pitched")


@pytest.mark.parametrize("x_format,scale_layout", [("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32"),
                                                   ("int8", "f32_group128")])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("w,rows,h", [(8, 3, 1152), (4, 7, 1024), (2, 1, 8192)])
def test_share_writes_only_its_output(gpu, x_format, scale_layout, out_dtype, w, rows, h):
    """The output is the head of a larger buffer whose tail holds NaN: the
    tail must survive (ragged element counts, every output type, the MX
    16-bit piece layout included)."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.Workload("guard", w, rows * w, h, x_format, scale_layout, out_dtype,
                            x_dist="int_uniform" if x_format == "int8" else "normal",
                            x_param=127 if x_format == "int8" else 40,
                            scale_lo=-10 if scale_layout == "f32_group128" else 110,
                            scale_hi=2 if scale_layout == "f32_group128" else 140, seed=77 + w + rows)
    xs, ss = workloads.generate(wl)
    p = qrs.plan(w, rows * w, h, x_format, scale_layout, out_dtype)
    dx, ds = to_device(xs, ss)
    n = rows * h
    big = empty_out(1, n + 4096, out_dtype).fill_(float("nan")).view(-1)
    qrs.run(p, dx, ds, big[:n].view(rows, h))
    torch.cuda.synchronize()
    assert torch.isnan(big[n:].float()).all(), "the share wrote past its output"
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype), out_dtype)
    assert_parity(out_bits(big[:n].view(rows, h)), want, out_dtype, "guard")


@pytest.mark.parametrize("w,rows,h", [
    (8, 10, 8192),   # 40 piece blocks: 32 renumbered in pairs, 8 left in order
    (8, 9, 8192),    # 36 blocks: 32 + 4
    (4, 37, 1152),   # 21 blocks, the last one partial
    (2, 64, 8192),   # 256 blocks, every one paired
    (8, 31, 5120),   # 78 blocks, the last one partial
    (8, 37, 1152),   # 21 blocks, the last wave partial; waves straddle rows
])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_piece_grids_with_unpaired_tails(gpu, w, rows, h, out_dtype):
    """MX shares run as 8-element pieces (fp32 outputs from W = 8) with
    blocks renumbered in groups of 16: grids whose block count is not a
    multiple of 16 (and whose last block or wave is partial) must still
    cover every element once, through all three launch forms. fp32 pieces
    trade output units across the half-waves, so a wave past the end of the
    share or straddling two rows must still store each unit at its own
    place."""
    import quantized_collective_reduction_amd as qrs

    wl = workloads.Workload("tails", w, rows * w, h, "e4m3fn", "e8m0_block32", out_dtype, x_dist="normal",
                            x_param=40, scale_lo=112, scale_hi=140, seed=4242 + rows)
    xs, ss = workloads.generate(wl)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, "e4m3fn", "e8m0_block32", out_dtype), out_dtype)
    got = run_gpu(w, rows, h, "e4m3fn", "e8m0_block32", out_dtype, xs, ss)
    assert_parity(got, want, out_dtype, "run")
    # row-strided: each row padded by 256 elements
    p = qrs.plan(w, rows * w, h, "e4m3fn", "e8m0_block32", out_dtype)
    dx = [torch.zeros((rows, h + 256), dtype=torch.uint8, device="cuda") for _ in xs]
    ds = [torch.zeros((rows, (h + 256) // 32), dtype=torch.uint8, device="cuda") for _ in ss]
    for t, x in zip(dx, xs):
        t[:, :h].copy_(torch.from_numpy(x))
    for t, s in zip(ds, ss):
        t[:, :h // 32].copy_(torch.from_numpy(s))
    out_full = empty_out(rows, h + 256, out_dtype).fill_(float("nan"))
    qrs.run_strided(p, [t[:, :h] for t in dx], [t[:, :h // 32] for t in ds], out_full[:, :h])
    torch.cuda.synchronize()
    assert_parity(out_bits(out_full[:, :h].contiguous()), want, out_dtype, "run_strided")
    assert torch.isnan(out_full[:, h:].float()).all(), "run_strided wrote outside the output rows"
    # all shares: each rank's full input is W copies of its slice's rows
    xf = [np.concatenate([x] * w) for x in xs]
    sf = [np.concatenate([s] * w) for s in ss]
    fx, fs = to_device(xf, sf)
    outs = [empty_out(rows, h, out_dtype).fill_(float("nan")) for _ in range(w)]
    qrs.run_all_shares(p, fx, fs, outs)
    torch.cuda.synchronize()
    for j in range(w):
        assert_parity(out_bits(outs[j]), want, out_dtype, f"all shares, share {j}")
