"""Pins for the oracle from closed forms, invariants and hand-worked examples.

Each test fixes something a plausible mistake in the oracle would break: the
fold order and start (worked examples), the group size and the axis groups
run along (scale locality, cross-layout equivalence), the decode of each
code (single-rank identity against torch's cast), the product and sum
rounding (exact integer sums, the recursive-summation error bound), sign
handling (cancellation), and IEEE propagation of NaN and infinity.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import exact
from oracle.decode import GROUP_SIZE, decode_table, scale_decode_table
from oracle.reduce import fp32_to_bf16_bits, reduce_scatter_share

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def load_worked_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def build_example(ex, rows=1, h=256):
    """Broadcast a single-element worked example over ``[rows, h]``."""
    g = GROUP_SIZE[ex["scale_layout"]]
    xs = [np.full((rows, h), int(c, 16), dtype=np.uint8) for c in ex["x_codes"]]
    if ex["scale_layout"] == "f32_group128":
        ss = [np.full((rows, h // g), int(s, 16), dtype=np.uint32).view(np.float32) for s in ex["scales"]]
    else:
        ss = [np.full((rows, h // g), int(s, 16), dtype=np.uint8) for s in ex["scales"]]
    return xs, ss


@pytest.mark.parametrize("ex", load_worked_examples(), ids=lambda e: e["name"])
def test_worked_example(ex):
    xs, ss = build_example(ex)
    out = reduce_scatter_share(xs, ss, ex["x_format"], ex["scale_layout"], ex["out_dtype"])
    want = int(ex["expected_bits"], 16)
    got = out.view(np.uint32) if ex["out_dtype"] == "f32" else out
    assert np.all(got == want), (ex["name"], hex(int(got.ravel()[0])), hex(want))


# ------------------------------------------------------------ exact sums


@pytest.mark.parametrize("w", [2, 4, 8])
def test_int8_power_of_two_scales_give_exact_integer_sums(w):
    """INT8 data, fp32 scales 2^k with k in a span of 10: every product is
    exact and every partial sum needs at most 8 + 10 + 3 bits, so the result
    is the exact sum, whatever the summation order."""
    rng = np.random.default_rng(w)
    rows, h = 8, 1024
    xs = [rng.integers(-128, 128, size=(rows, h), dtype=np.int8).view(np.uint8) for _ in range(w)]
    ks = [rng.integers(-14, -4, size=(rows, h // 128)) for _ in range(w)]
    ss = [np.ldexp(np.float32(1.0), k).astype(np.float32) for k in ks]
    out = reduce_scatter_share(xs, ss, "int8", "f32_group128", "f32")
    # Exact value in units of 2^-14, from Python integers.
    kmin = -14
    want = np.zeros((rows, h), dtype=object)
    for x, k in zip(xs, ks):
        xi = x.view(np.int8).astype(object)
        want += xi * (2 ** (np.repeat(k, 128, axis=1) - kmin)).astype(object)
    want_f = np.vectorize(lambda v: math.ldexp(float(v), kmin))(want).astype(np.float32)
    assert np.array_equal(_bits(out), _bits(want_f))
    # ... and therefore invariant under any permutation of the ranks.
    perm = rng.permutation(w)
    out_p = reduce_scatter_share([xs[p] for p in perm], [ss[p] for p in perm], "int8", "f32_group128", "f32")
    assert np.array_equal(_bits(out), _bits(out_p))


@pytest.mark.parametrize("x_format,tdt", [("int8", torch.int8), ("e4m3fn", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
@pytest.mark.parametrize("scale_layout", ["f32_group128", "e8m0_block32"])
def test_single_rank_is_decode_times_power_of_two(x_format, tdt, scale_layout):
    """W = 1: the output is rank 0's dequantized slice. With a power-of-two
    scale 2^k the product is exact, so it equals torch's decode of the codes
    times 2^k (np.ldexp, exact here)."""
    if x_format == "int8" and scale_layout == "e8m0_block32":
        pytest.skip("INT8 is paired with fp32 scales only")
    g = GROUP_SIZE[scale_layout]
    codes = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(2, 1024)
    k = np.array([[-3, 0, 2, 5, -1, 1, 4, -2] * (1024 // g // 8)] * 2)
    if scale_layout == "f32_group128":
        s = np.ldexp(np.float32(1.0), k).astype(np.float32)
    else:
        s = (k + 127).astype(np.uint8)
    out = reduce_scatter_share([codes], [s], x_format, scale_layout, "f32")
    dec = torch.from_numpy(codes.copy()).view(tdt).to(torch.float32).numpy()
    want = np.ldexp(dec, np.repeat(k, g, axis=1)).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(_bits(out)[~nan], _bits(want)[~nan])


def _negate_codes(x, x_format):
    if x_format == "int8":
        return (-(x.view(np.int8).astype(np.int16))).astype(np.int8).view(np.uint8)
    return x ^ np.uint8(0x80)


@pytest.mark.parametrize("x_format,scale_layout", [("int8", "f32_group128"), ("e4m3fn", "e8m0_block32"), ("e5m2", "f32_group128")])
def test_opposite_rank_pairs_cancel_to_positive_zero(x_format, scale_layout):
    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(world_size=2, bs=8, h=1024, x_format=x_format, scale_layout=scale_layout,
                                       x_dist="int_uniform" if x_format == "int8" else "normal",
                                       x_param=127 if x_format == "int8" else 16,
                                       scale_lo=100 if scale_layout == "e8m0_block32" else -6,
                                       scale_hi=150 if scale_layout == "e8m0_block32" else 6)
    a, sa = workloads.generate_rank(wl, 0)
    b, sb = workloads.generate_rank(wl, 1)
    xs = [a, _negate_codes(a, x_format), b, _negate_codes(b, x_format)]
    ss = [sa, sa, sb, sb]
    out = reduce_scatter_share(xs, ss, x_format, scale_layout, "f32")
    assert np.all(_bits(out) == 0)  # +0, not -0


# ------------------------------------------------------------ structure


def test_scale_influence_is_local_to_its_group():
    """Changing S_r[i, k] may change only columns [kG, (k+1)G) of row i, and
    does change some of them."""
    for scale_layout in ("f32_group128", "e8m0_block32"):
        g = GROUP_SIZE[scale_layout]
        wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=4 * 6, world_size=4, h=1024, scale_layout=scale_layout,
                                           scale_lo=-4 if scale_layout == "f32_group128" else 120,
                                           scale_hi=4 if scale_layout == "f32_group128" else 134, out_dtype="f32")
        xs, ss = workloads.generate(wl)
        base = reduce_scatter_share(xs, ss, wl.x_format, scale_layout, "f32")
        i, k, r = 3, 5, 2
        ss2 = [s.copy() for s in ss]
        if scale_layout == "f32_group128":
            ss2[r][i, k] = ss2[r][i, k] * np.float32(4.0)
        else:
            ss2[r][i, k] = ss2[r][i, k] + 2
        changed = _bits(reduce_scatter_share(xs, ss2, wl.x_format, scale_layout, "f32")) != _bits(base)
        allowed = np.zeros_like(changed)
        allowed[i, k * g:(k + 1) * g] = True
        assert not np.any(changed & ~allowed), scale_layout
        assert changed[i, k * g:(k + 1) * g].sum() >= g // 2, scale_layout


def test_mx_and_group_layouts_agree_on_equal_scales():
    """E8M0 codes constant over each 128 columns give the same output as fp32
    scales 2^(code-127) per 128-group: the two layouts index the same
    columns."""
    rng = np.random.default_rng(3)
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * 4, h=2048)
    xs, _ = workloads.generate(wl)
    codes128 = [rng.integers(110, 145, size=(wl.rows, wl.h // 128), dtype=np.uint8) for _ in range(8)]
    mx = [np.repeat(c, 4, axis=1) for c in codes128]
    f32 = [np.ldexp(np.float32(1.0), c.astype(np.int32) - 127).astype(np.float32) for c in codes128]
    a = reduce_scatter_share(xs, mx, "e4m3fn", "e8m0_block32", "f32")
    b = reduce_scatter_share(xs, f32, "e4m3fn", "f32_group128", "f32")
    assert np.array_equal(_bits(a), _bits(b))


def test_rows_are_independent():
    wl = workloads.WORKLOADS["w8_bs8192_h7168_e5m2_bf16"].with_(bs=8 * 16, h=1024)
    xs, ss = workloads.generate(wl)
    perm = np.random.default_rng(0).permutation(wl.rows)
    a = reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, "f32")
    b = reduce_scatter_share([x[perm] for x in xs], [s[perm] for s in ss], wl.x_format, wl.scale_layout, "f32")
    assert np.array_equal(_bits(a[perm]), _bits(b))


def test_non_finite_propagation():
    h = 128
    one = np.full((1, h // 32), 127, dtype=np.uint8)
    x = lambda code: np.full((1, h), code, dtype=np.uint8)  # noqa: E731
    f = lambda xs, ss, fmt: reduce_scatter_share(xs, ss, fmt, "e8m0_block32", "f32")[0, 0]  # noqa: E731
    assert math.isnan(f([x(0x38), x(0x7F)], [one, one], "e4m3fn"))  # E4M3FN NaN code
    assert math.isnan(f([x(0x7C), x(0xFC)], [one, one], "e5m2"))  # +inf + -inf
    assert f([x(0x7C), x(0x3C)], [one, one], "e5m2") == math.inf
    assert f([x(0x3C), x(0xFC)], [one, one], "e5m2") == -math.inf
    nan_scale = np.full((1, h // 32), 255, dtype=np.uint8)
    assert math.isnan(f([x(0x3C), x(0x3C)], [one, nan_scale], "e5m2"))
    # A zero element times a NaN scale is NaN, times an infinite result is NaN.
    assert math.isnan(f([x(0x00), x(0x00)], [nan_scale, one], "e5m2"))


def test_16bit_outputs_are_rounded_fp32_output():
    wl = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"].with_(bs=4 * 8)
    xs, ss = workloads.generate(wl)
    f = reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, "f32")
    b = reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, "bf16")
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, fp32_to_bf16_bits(f))
    assert np.array_equal(b, tb)
    h = reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, "f16")
    assert np.array_equal(h, f.astype(np.float16).view(np.uint16))


# ------------------------------------------------------------ error bound


@pytest.mark.parametrize("name", ["w2_bs32_h1024_int8_f32", "w4_bs4096_h4096_e4m3_bf16", "w8_bs8192_h7168_e5m2_bf16", "w8_bs16384_h8192_mx_e4m3_bf16", "w8_bs65536_h5120_mx_e5m2_f32"])
def test_error_bound_against_exact_sum(name):
    """|Y - sum_r x_r s_r| <= gamma_W * sum_r |x_r s_r|, gamma_W = W u/(1 - W u),
    u = 2^-24 (recursive summation of W rounded products; Higham, Accuracy and
    Stability of Numerical Algorithms, the dot-product bound of ch. 3). Checked
    on sampled elements of a few rows of each workload's distribution."""
    wl = workloads.WORKLOADS[name]
    wl = wl.with_(bs=wl.world_size * 4)
    xs, ss = workloads.generate(wl)
    y = reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, "f32")
    g = wl.group
    xt = decode_table(wl.x_format)
    st = scale_decode_table()
    u = Fraction(1, 2**24)
    gamma = wl.world_size * u / (1 - wl.world_size * u)
    rng = np.random.default_rng(1)
    worst = Fraction(0)
    for _ in range(400):
        i = int(rng.integers(0, wl.rows))
        c = int(rng.integers(0, wl.h))
        xv = [float(xt[x[i, c]]) for x in xs]
        if wl.scale_layout == "f32_group128":
            sv = [float(s[i, c // g]) for s in ss]
        else:
            sv = [float(st[s[i, c // g]]) for s in ss]
        s_exact = exact.exact_sum(xv, sv)
        mag = sum(abs(Fraction(a) * Fraction(b)) for a, b in zip(xv, sv))
        err = abs(Fraction(float(y[i, c])) - s_exact)
        assert err <= gamma * mag, (name, i, c)
        if mag:
            worst = max(worst, err / mag)
    assert worst <= gamma
