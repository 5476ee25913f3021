"""GPU parity of the producer-side quantization (qrs_quantize) against the
oracle: codes and scales bit for bit. Also every in-range bf16 value through
the hardware conversions, and the producer -> reduce-scatter pipeline."""

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_reduction_amd as qrs
import workloads
from gpu_util import assert_parity, empty_out, oracle_bits, out_bits
from oracle.quantize import quantize as oracle_quantize
from test_oracle_quantize_examples import AMAX_COL, V_COL, example_input, load_examples

pytestmark = pytest.mark.gpu

MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


def _gpu_quantize(bits, x_format, scale_layout):
    t, h = bits.shape
    g = 128 if scale_layout == "f32_group128" else 32
    x = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    codes = torch.full((t, h), 0xAA, dtype=torch.uint8, device="cuda")
    if scale_layout == "f32_group128":
        scales = torch.full((t, h // g), float("nan"), dtype=torch.float32, device="cuda")
    else:
        scales = torch.full((t, h // g), 0xAA, dtype=torch.uint8, device="cuda")
    qrs.quantize(x, codes, scales, x_format, scale_layout)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()
    return codes.cpu().numpy(), (s.view(np.uint32) if s.dtype == np.float32 else s)


def _want(bits, x_format, scale_layout):
    c, s = oracle_quantize(bits, x_format, scale_layout)
    return c, (s.view(np.uint32) if s.dtype == np.float32 else s)


def _activations(t, h, seed, zero_groups=True):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((t, h)).astype(np.float32) * np.exp2(rng.integers(-40, 40, size=(t, 1))).astype(np.float32)
    if zero_groups:
        v[0, :256] = 0.0
        v[-1, -128:] = -0.0
        v[t // 2, 128:256] *= np.float32(2.0 ** -100)  # tiny groups (bf16 subnormals appear)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("x_format,scale_layout", MODES)
@pytest.mark.parametrize("t,h", [(1, 1024), (3, 1152), (17, 8192), (5, 5120)])
def test_quantize_matches_oracle(gpu, x_format, scale_layout, t, h):
    bits = _activations(t, h, seed=t * 1000 + h)
    gc, gs = _gpu_quantize(bits, x_format, scale_layout)
    wc, ws = _want(bits, x_format, scale_layout)
    assert np.array_equal(gs, ws), "scales differ"
    bad = np.argwhere(gc != wc)
    assert bad.size == 0, (bad[:5], gc[tuple(bad[0])], wc[tuple(bad[0])])


@pytest.mark.parametrize("x_format,scale_layout", MODES)
def test_every_in_range_bf16_value_converts_like_the_oracle(gpu, x_format, scale_layout):
    """Groups whose maximum makes the multiplier exactly 1 (per-group: amax =
    qmax; MX: amax in the format's top binade), filled with every bf16 value
    in range: the hardware conversion sees each of them, ties included."""
    qmax = {"int8": 127.0, "e4m3fn": 448.0, "e5m2": 57344.0}[x_format]
    g = 128 if scale_layout == "f32_group128" else 32
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_fp32(allbits)
    keep = allbits[np.isfinite(vals) & (np.abs(vals) <= qmax)]
    per = g - 1
    n_groups = -(-keep.size // per)
    h = 1024 * 8
    groups_per_row = h // g
    rows = -(-n_groups // groups_per_row)
    pad = np.zeros(rows * groups_per_row * per, dtype=np.uint16)
    pad[: keep.size] = keep
    body = pad.reshape(rows, groups_per_row, per)
    top = oracle.fp32_to_bf16_bits(np.array([qmax], dtype=np.float32))[0]
    bits = np.concatenate([np.full((rows, groups_per_row, 1), top, dtype=np.uint16), body], axis=2).reshape(rows, h)
    gc, gs = _gpu_quantize(bits, x_format, scale_layout)
    wc, ws = _want(bits, x_format, scale_layout)
    assert np.array_equal(gs, ws)
    bad = np.argwhere(gc != wc)
    assert bad.size == 0, [(int(bits[tuple(b)]), int(gc[tuple(b)]), int(wc[tuple(b)])) for b in bad[:8]]


@pytest.mark.parametrize("x_format,scale_layout", [("e4m3fn", "e8m0_block32"), ("int8", "f32_group128")])
def test_quantize_full_size_sampled(gpu, x_format, scale_layout):
    """One rank's [16384, 8192] activations, the launch the benchmark times;
    256 sampled tokens compared bit for bit."""
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"]
    bits = workloads.generate_activations(wl, 0)
    gc, gs = _gpu_quantize(bits, x_format, scale_layout)
    rows = np.sort(np.random.default_rng(9).choice(wl.bs, 256, replace=False))
    wc, ws = _want(bits[rows], x_format, scale_layout)
    assert np.array_equal(gs[rows], ws)
    assert np.array_equal(gc[rows], wc)


@pytest.mark.parametrize("x_format,scale_layout,out_dtype", [("e4m3fn", "e8m0_block32", "bf16"),
                                                             ("int8", "f32_group128", "f32"),
                                                             ("e5m2", "f32_group128", "f32")])
def test_producer_to_reduce_scatter_pipeline(gpu, x_format, scale_layout, out_dtype):
    """bf16 activations of W ranks -> qrs_quantize on each -> qrs_run_all_shares:
    bit-exact with the oracle's quantize -> all_shares, and close to the exact
    reduce-scatter of the unquantized values."""
    w, bs, h = 4, 4 * 6, 2048
    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(world_size=w, bs=bs, h=h)
    acts = [workloads.generate_activations(wl, r) for r in range(w)]
    g = 128 if scale_layout == "f32_group128" else 32
    dx, ds = [], []
    for a in acts:
        x = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
        c = torch.empty((bs, h), dtype=torch.uint8, device="cuda")
        s = torch.empty((bs, h // g), dtype=torch.float32 if scale_layout == "f32_group128" else torch.uint8,
                        device="cuda")
        qrs.quantize(x, c, s, x_format, scale_layout)
        dx.append(c)
        ds.append(s)
    p = qrs.plan(w, bs, h, x_format, scale_layout, out_dtype)
    outs = [empty_out(bs // w, h, out_dtype) for _ in range(w)]
    qrs.run_all_shares(p, dx, ds, outs)
    torch.cuda.synchronize()
    q = [oracle_quantize(a, x_format, scale_layout) for a in acts]
    want = oracle.all_shares([c for c, _ in q], [s for _, s in q], x_format, scale_layout, out_dtype)
    for j in range(w):
        assert_parity(out_bits(outs[j]), oracle_bits(want[j], out_dtype), out_dtype, f"share {j}")
    # Close to the reduce-scatter of the original values: each rank's
    # element is off by at most rel * |v| + step * amax of its group (the
    # format's relative half-step, the MX clamp of the block maximum, and the
    # absolute half-step of the smallest codes), plus the fold and output
    # rounding.
    rows = bs // w
    rel = {"int8": 0.0, "e4m3fn": 2.0 ** -3, "e5m2": 2.0 ** -2}[x_format]
    step = {"int8": 0.5 / 127, "e4m3fn": 2.0 ** -9, "e5m2": 2.0 ** -16}[x_format]
    out_rel = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -23
    for j in range(w):
        blocks = [oracle.bf16_bits_to_fp32(a[j * rows:(j + 1) * rows]).astype(np.float64) for a in acts]
        exact = sum(blocks)
        bound = np.zeros_like(exact)
        for b in blocks:
            amax = np.repeat(np.abs(b).reshape(rows, -1, g).max(axis=2), g, axis=1)
            bound += rel * np.abs(b) + step * amax * (1 + 2.0 ** -10)
        got = outs[j].float().cpu().numpy().astype(np.float64)
        mag = sum(np.abs(b) for b in blocks)
        assert np.all(np.abs(got - exact) <= bound + out_rel * np.abs(got) + w * 2.0 ** -23 * (mag + bound))


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_hand_derived_group_examples(gpu, ex):
    """The hand-derived midpoint groups of tests/golden/quantize_examples.json
    through the kernel: the code of v, of amax and the group's scale."""
    bits = np.repeat(example_input(ex), 3, axis=0)
    gc, gs = _gpu_quantize(bits, ex["x_format"], "f32_group128")
    qmax_code = {"int8": 0x7F, "e4m3fn": 0x7E, "e5m2": 0x7B}[ex["x_format"]]
    assert np.all(gc[:, V_COL] == int(ex["expected_code"], 16)), (ex["name"], hex(int(gc[0, V_COL])))
    assert np.all(gc[:, AMAX_COL] == qmax_code)
    assert np.all(gs[:, 0] == int(ex["expected_scale_bits"], 16))
    wc, ws = _want(bits, ex["x_format"], "f32_group128")
    assert np.array_equal(gc, wc) and np.array_equal(gs, ws)
