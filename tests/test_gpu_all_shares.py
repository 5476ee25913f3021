"""GPU parity of qrs_run_all_shares (the group's whole reduce-scatter on one
GPU, the all-to-all applied by addressing) against the oracle's all-to-all +
reduce."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import assert_parity, empty_out, log, oracle_bits, out_bits

pytestmark = pytest.mark.gpu

MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


def _run(wl, xs, ss):
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    dx = [torch.from_numpy(x).cuda() for x in xs]
    ds = [torch.from_numpy(s).cuda() for s in ss]
    outs = [empty_out(wl.rows, wl.h, wl.out_dtype).fill_(float("nan")) for _ in range(wl.world_size)]
    qrs.run_all_shares(p, dx, ds, outs)
    torch.cuda.synchronize()
    return [out_bits(o) for o in outs]


@pytest.mark.parametrize("x_format,scale_layout", MODES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("w", [2, 4, 8])
def test_all_shares_small(gpu, x_format, scale_layout, out_dtype, w):
    rows, h = 5, 1152
    wl = workloads.Workload(
        "all", w, rows * w, h, x_format, scale_layout, out_dtype,
        x_dist="int_uniform" if x_format == "int8" else "normal",
        x_param=127 if x_format == "int8" else 40,
        scale_lo=-12 if scale_layout == "f32_group128" else 110,
        scale_hi=2 if scale_layout == "f32_group128" else 140, seed=77 + w,
    )
    xs, ss = workloads.generate_full(wl)
    got = _run(wl, xs, ss)
    want = oracle.all_shares(xs, ss, x_format, scale_layout, out_dtype)
    for j in range(w):
        assert_parity(got[j], oracle_bits(want[j], out_dtype), out_dtype, f"share {j}")


def test_all_shares_full_size_sampled(gpu):
    """The W=8, BS=16384, H=8192 MX group (1 GiB of codes) in the launch the
    benchmark times; every share checked on 24 sampled rows, all columns."""
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"]
    log("[all_shares] generating 8 x [16384, 8192] inputs")
    xs, ss = workloads.generate_full(wl)
    got = _run(wl, xs, ss)
    rng = np.random.default_rng(4)
    rows = np.sort(np.concatenate([[0, wl.rows - 1], rng.choice(wl.rows, 22, replace=False)]))
    for j, (rx, rs) in enumerate(oracle.all_to_all(xs, ss)):
        want = oracle.reduce_scatter_share([x[rows] for x in rx], [s[rows] for s in rs],
                                           wl.x_format, wl.scale_layout, wl.out_dtype)
        assert_parity(got[j][rows], oracle_bits(want, wl.out_dtype), wl.out_dtype, f"share {j}")


def test_all_shares_rejects_overlapping_outputs(gpu):
    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(bs=4 * 8)
    p = qrs.plan(4, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    xs = [torch.zeros(wl.bs, wl.h, dtype=torch.uint8, device="cuda") for _ in range(4)]
    ss = [torch.zeros(wl.bs, wl.h // 128, dtype=torch.float32, device="cuda") for _ in range(4)]
    big = empty_out(wl.rows * 4, wl.h, wl.out_dtype)
    outs = [big[0:wl.rows], big[wl.rows:2 * wl.rows], big[0:wl.rows], big[3 * wl.rows:]]
    with pytest.raises(qrs.QrsError) as ei:
        qrs.run_all_shares(p, xs, ss, outs)
    assert ei.value.status == qrs.Status.INVALID_ARG


def test_all_shares_large_shares_one_launch_each(gpu):
    """Shares of more than about 300 MB are enqueued one launch per share:
    W=2, BS=32768, H=8192 MX E4M3FN -> bf16 is 545 MB per share. Both shares
    checked on 24 sampled rows, all columns; the result must equal the same
    inputs' shares computed by qrs_run on each row block."""
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(world_size=2, bs=32768)
    assert wl.algorithmic_bytes() > 300_000_000  # per share
    log("[all_shares] generating 2 x [32768, 8192] inputs")
    xs, ss = workloads.generate_full(wl)
    got = _run(wl, xs, ss)
    rng = np.random.default_rng(8)
    rows = np.sort(np.concatenate([[0, wl.rows - 1], rng.choice(wl.rows, 22, replace=False)]))
    for j, (rx, rs) in enumerate(oracle.all_to_all(xs, ss)):
        want = oracle.reduce_scatter_share([x[rows] for x in rx], [s[rows] for s in rs],
                                           wl.x_format, wl.scale_layout, wl.out_dtype)
        assert_parity(got[j][rows], oracle_bits(want, wl.out_dtype), wl.out_dtype, f"share {j}")
    p = qrs.plan(wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype)
    for j, (rx, rs) in enumerate(oracle.all_to_all(xs, ss)):
        dx = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in rx]
        ds = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in rs]
        out = empty_out(wl.rows, wl.h, wl.out_dtype)
        qrs.run(p, dx, ds, out)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), got[j]), f"share {j}"


def test_all_shares_large_capped_group_one_launch(gpu):
    """A W=8 MX group runs as one capped launch of 8-element pieces even
    where its shares are large: W=8, BS=24576, H=8192 MX E5M2 -> fp32 is 309
    MB per share (2.5 GB for the group). The inputs are drawn on the GPU
    (finite codes, E8M0 bytes 112..142); every share must equal qrs_run on
    its row blocks, byte for byte, and 16 sampled rows must match the
    oracle."""
    w, rows, h = 8, 3072, 8192
    bs = w * rows
    p = qrs.plan(w, bs, h, "e5m2", "e8m0_block32", "f32")
    per_share = w * rows * h + w * rows * h // 32 + rows * h * 4
    assert per_share > 300_000_000
    gen = torch.Generator(device="cuda").manual_seed(31)
    xs = []
    for _ in range(w):
        mag = torch.randint(0, 124, (bs, h), dtype=torch.int32, device="cuda", generator=gen)
        sign = torch.randint(0, 2, (bs, h), dtype=torch.int32, device="cuda", generator=gen) << 7
        xs.append((mag | sign).to(torch.uint8))
    ss = [torch.randint(112, 143, (bs, h // 32), dtype=torch.int32, device="cuda", generator=gen).to(torch.uint8)
          for _ in range(w)]
    outs = [empty_out(rows, h, "f32").fill_(float("nan")) for _ in range(w)]
    log("[all_shares] one launch over a 2.5 GB W=8 group")
    qrs.run_all_shares(p, xs, ss, outs)
    torch.cuda.synchronize()
    sample = np.sort(np.concatenate([[0, rows - 1], np.random.default_rng(3).choice(rows, 14, replace=False)]))
    ref = empty_out(rows, h, "f32")
    for j in range(w):
        qrs.run(p, [x[j * rows:(j + 1) * rows] for x in xs], [s[j * rows:(j + 1) * rows] for s in ss], ref)
        torch.cuda.synchronize()
        assert torch.equal(outs[j].view(torch.uint8), ref.view(torch.uint8)), f"share {j}"
        rx = [x[j * rows:(j + 1) * rows][sample].cpu().numpy() for x in xs]
        rs = [s[j * rows:(j + 1) * rows][sample].cpu().numpy() for s in ss]
        want = oracle.reduce_scatter_share(rx, rs, "e5m2", "e8m0_block32", "f32")
        assert_parity(out_bits(outs[j])[sample], oracle_bits(want, "f32"), "f32", f"share {j} sampled rows")


def _gpu_codes(x_format, shape, gen):
    """Random finite codes of the format, drawn on the GPU."""
    b = torch.randint(0, 256, shape, dtype=torch.int32, device="cuda", generator=gen)
    if x_format == "e4m3fn":
        b = torch.where((b & 0x7F) == 0x7F, b - 1, b)  # no NaN
    elif x_format == "e5m2":
        b = torch.where((b & 0x7F) >= 0x7C, b & 0x83, b)  # no inf or NaN
    return b.to(torch.uint8)


def _gpu_scales(scale_layout, shape, gen):
    if scale_layout == "e8m0_block32":
        return torch.randint(112, 143, shape, dtype=torch.int32, device="cuda", generator=gen).to(torch.uint8)
    e = torch.randint(-14, 3, shape, dtype=torch.int32, device="cuda", generator=gen).float()
    m = 1.0 + torch.rand(shape, device="cuda", generator=gen)
    return (m * torch.exp2(e)).to(torch.float32)


def _large_group_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        xf, sl = MODES[rng.integers(len(MODES))]
        out.append(dict(w=int(rng.choice([2, 4, 8])), rows=int(rng.integers(100, 701)),
                        h=int(128 * rng.integers(8, 65)), x_format=xf, scale_layout=sl,
                        out_dtype=str(rng.choice(["f32", "bf16", "f16"]))))
    return out


LARGE_GROUP_CASES = _large_group_cases(12, 515) + [
    dict(w=8, rows=400, h=4096, x_format="e4m3fn", scale_layout="e8m0_block32", out_dtype="bf16"),  # capped
    dict(w=8, rows=300, h=7168, x_format="e5m2", scale_layout="e8m0_block32", out_dtype="f32"),  # capped
]


@pytest.mark.parametrize("c", LARGE_GROUP_CASES,
                         ids=lambda c: f"W{c['w']}-r{c['rows']}-h{c['h']}-{c['x_format']}-{c['scale_layout']}-"
                                       f"{c['out_dtype']}")
def test_all_shares_random_larger_groups(gpu, c):
    """Groups of 100 to 700 rows per share (at W = 8 past three generations
    of capped blocks, so the capped launch runs), inputs drawn on the GPU:
    every share equals qrs_run on its row blocks, byte for byte, and
    sampled rows of two shares match the oracle."""
    w, rows, h = c["w"], c["rows"], c["h"]
    xf, sl, od = c["x_format"], c["scale_layout"], c["out_dtype"]
    g = 128 if sl == "f32_group128" else 32
    gen = torch.Generator(device="cuda").manual_seed(rows * 131 + h)
    xs = [_gpu_codes(xf, (w * rows, h), gen) for _ in range(w)]
    ss = [_gpu_scales(sl, (w * rows, h // g), gen) for _ in range(w)]
    p = qrs.plan(w, w * rows, h, xf, sl, od)
    outs = [empty_out(rows, h, od).fill_(float("nan")) for _ in range(w)]
    qrs.run_all_shares(p, xs, ss, outs)
    ref = empty_out(rows, h, od)
    sample = np.array([0, rows // 3, rows - 1])
    for j in range(w):
        qrs.run(p, [x[j * rows:(j + 1) * rows] for x in xs], [s[j * rows:(j + 1) * rows] for s in ss], ref)
        torch.cuda.synchronize()
        assert torch.equal(outs[j].view(torch.uint8), ref.view(torch.uint8)), f"share {j}"
        if j in (0, w - 1):
            rx = [x[j * rows:(j + 1) * rows][sample].cpu().numpy() for x in xs]
            rs = [s[j * rows:(j + 1) * rows][sample].cpu().numpy() for s in ss]
            want = oracle.reduce_scatter_share(rx, rs, xf, sl, od)
            assert_parity(out_bits(outs[j])[sample], oracle_bits(want, od), od, f"share {j} sampled rows")
