"""Pins for the oracle's arithmetic: numpy oracle == exact-rational brute force.

First the brute force's own rounding routine is pinned to a library routine
(numpy's float64 -> float32 conversion, which rounds to nearest-even). Then
``oracle.reduce_scatter_share`` must equal, bit for bit, a fold of exact
rational products and sums each rounded by that routine, on random tiny
inputs of every (x format, scale layout) and on every pair of x codes.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import exact
from oracle.decode import GROUP_SIZE, decode_table, scale_decode_table
from oracle.reduce import reduce_scatter_share

MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


def _f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


# ---------------------------------------------------------------- rounding


def test_round_to_binary32_matches_numpy_conversion():
    rng = np.random.default_rng(11)
    # Doubles spread over the whole binary32 range, its subnormals, and past
    # the overflow threshold.
    mant = rng.uniform(1.0, 2.0, size=6000)
    exps = rng.integers(-152, 130, size=6000)
    signs = rng.choice([-1.0, 1.0], size=6000)
    vals = signs * np.ldexp(mant, exps)
    # Exact ties: binary32 values plus half an ulp, in normal and subnormal range.
    base = np.ldexp(rng.integers(2**23, 2**24, size=500).astype(np.float64), rng.integers(-140, 100, size=500))
    ulp_exp = np.floor(np.log2(np.abs(base))) - 23
    ties = base + np.ldexp(0.5, ulp_exp.astype(int))
    sub_ties = np.ldexp(rng.integers(0, 2**23, size=300).astype(np.float64) + 0.5, -149)
    edge = np.array([3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2**-25), 2.0**128 * (1 - 2**-25), 2.0**-150, 2.0**-151, 3 * 2.0**-151])
    allv = np.concatenate([vals, ties, sub_ties, edge, -edge])
    with np.errstate(over="ignore"):
        want = allv.astype(np.float32)
    for d, w in zip(allv, want):
        got = exact.round_to_binary32(Fraction(float(d)))
        assert _f32_bits(got) == int(np.array([w]).view(np.uint32)[0]), (d, got, w)


def test_signed_zero_rules():
    assert math.copysign(1.0, exact.add_binary32(-0.0, -0.0)) < 0
    assert math.copysign(1.0, exact.add_binary32(-0.0, 0.0)) > 0
    assert math.copysign(1.0, exact.add_binary32(1.5, -1.5)) > 0
    assert math.copysign(1.0, exact.mul_binary32(-0.0, 3.0)) < 0
    assert math.copysign(1.0, exact.mul_binary32(-2.0**-100, 2.0**-100)) < 0  # underflow keeps sign


# ---------------------------------------------------------------- brute force


def _random_tiny(rng, x_format, scale_layout, w, rows, h):
    g = GROUP_SIZE[scale_layout]
    table = decode_table(x_format)
    finite = np.nonzero(np.isfinite(table))[0].astype(np.uint8)
    xs = [rng.choice(finite, size=(rows, h)) for _ in range(w)]
    if scale_layout == "f32_group128":
        # Random significands (so products round) over a wide exponent span.
        ss = [
            (rng.uniform(1.0, 2.0, size=(rows, h // g)) * np.exp2(rng.integers(-30, 10, size=(rows, h // g)))
             * rng.choice([-1.0, 1.0], size=(rows, h // g))).astype(np.float32)
            for _ in range(w)
        ]
    else:
        # E8M0 codes low enough that no product overflows (57344 * 2^111 < 2^127).
        ss = [rng.integers(0, 239, size=(rows, h // g), dtype=np.uint8) for _ in range(w)]
    return xs, ss


def _brute_force(xs, ss, x_format, scale_layout):
    g = GROUP_SIZE[scale_layout]
    xt = decode_table(x_format)
    st = scale_decode_table()
    rows, h = xs[0].shape
    out = np.empty((rows, h), dtype=np.float32)
    for i in range(rows):
        for c in range(h):
            xv = [float(xt[x[i, c]]) for x in xs]
            if scale_layout == "f32_group128":
                sv = [float(s[i, c // g]) for s in ss]
            else:
                sv = [float(st[s[i, c // g]]) for s in ss]
            out[i, c] = exact.share_element(xv, sv)
    return out


@pytest.mark.parametrize("x_format,scale_layout", MODES)
@pytest.mark.parametrize("w", [1, 2, 3, 4, 8])
def test_oracle_equals_brute_force_random(x_format, scale_layout, w):
    rng = np.random.default_rng([w, len(x_format), len(scale_layout)])
    rows, h = 2, 256
    xs, ss = _random_tiny(rng, x_format, scale_layout, w, rows, h)
    got = reduce_scatter_share(xs, ss, x_format, scale_layout, "f32")
    want = _brute_force(xs, ss, x_format, scale_layout)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("x_format,scale_layout", MODES)
def test_oracle_equals_brute_force_all_code_pairs(x_format, scale_layout):
    """Every (rank-0 code, rank-1 code) pair at W=2: 64 rows x 1024 columns.

    Pairs with a non-finite code are left to the closed-form tests (the brute
    force is finite-only); the rest must agree bit for bit.
    """
    rng = np.random.default_rng(5)
    g = GROUP_SIZE[scale_layout]
    codes = np.arange(256 * 256)
    x0 = (codes // 256).astype(np.uint8).reshape(64, 1024)
    x1 = (codes % 256).astype(np.uint8).reshape(64, 1024)
    xs = [x0, x1]
    _, ss = _random_tiny(rng, x_format, scale_layout, 2, 64, 1024)
    got = reduce_scatter_share(xs, ss, x_format, scale_layout, "f32")
    table = decode_table(x_format)
    finite = np.isfinite(table[x0]) & np.isfinite(table[x1])
    xt = table
    st = scale_decode_table()
    idx = np.argwhere(finite)
    # Every finite pair is checked (up to 65536 elements).
    for i, c in idx:
        xv = [float(xt[x0[i, c]]), float(xt[x1[i, c]])]
        if scale_layout == "f32_group128":
            sv = [float(ss[0][i, c // g]), float(ss[1][i, c // g])]
        else:
            sv = [float(st[ss[0][i, c // g]]), float(st[ss[1][i, c // g]])]
        want = exact.share_element(xv, sv)
        assert _f32_bits(float(got[i, c])) == _f32_bits(want), (i, c, xv, sv)
