"""GPU probes of the conversions and the fold, through the real kernels.

* Every x code of every format, alone in rank 0 with a unit scale: the
  output must be the code's exact value (catches a wrong fp8 flavour, NaN,
  infinity or subnormal handling in the hardware conversions).
* Every E8M0 code as the scale of x = 1: the output is the scale's value
  (catches the 2^-127 subnormal and the NaN code).
* The hand-derived worked examples (tests/golden/worked_examples.json):
  the kernel must reproduce the expected bits, which fix the fold order, the
  fold's start, the separate rounding of product and sum, and bf16 ties.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_parity, oracle_bits, run_gpu
from test_oracle_closed_forms import build_example, load_worked_examples

pytestmark = pytest.mark.gpu

ONE_CODE = {"int8": 0x01, "e4m3fn": 0x38, "e5m2": 0x3C}


@pytest.mark.parametrize(
    "x_format,scale_layout",
    [("int8", "f32_group128"), ("e4m3fn", "f32_group128"), ("e5m2", "f32_group128"),
     ("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32")],
)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_every_x_code_decodes_exactly(gpu, x_format, scale_layout, out_dtype):
    rows, h = 2, 1024
    codes = np.tile(np.arange(256, dtype=np.uint8), rows * h // 256).reshape(rows, h)
    zero = np.zeros_like(codes)
    g = 128 if scale_layout == "f32_group128" else 32
    if scale_layout == "f32_group128":
        unit = np.ones((rows, h // g), dtype=np.float32)
    else:
        unit = np.full((rows, h // g), 127, dtype=np.uint8)
    got = run_gpu(2, rows, h, x_format, scale_layout, out_dtype, [codes, zero], [unit, unit])
    want = oracle_bits(oracle.reduce_scatter_share([codes, zero], [unit, unit], x_format, scale_layout, out_dtype),
                       out_dtype)
    assert_parity(got, want, out_dtype, f"{x_format} codes")
    if out_dtype == "f32":
        table = oracle.decode_table(x_format)
        vals = got.view(np.float32).reshape(-1)[:256]
        nan = np.isnan(table)
        assert np.array_equal(np.isnan(vals), nan)
        # x + 0: exact except that -0 + +0 = +0.
        expect = np.where(table == 0, np.float32(0.0), table)
        assert np.array_equal(vals[~nan].view(np.uint32), expect[~nan].view(np.uint32))


@pytest.mark.parametrize("x_format", ["e4m3fn", "e5m2"])
def test_every_e8m0_code(gpu, x_format):
    rows, h = 1, 8192  # 256 scale blocks in one row
    one = np.full((rows, h), ONE_CODE[x_format], dtype=np.uint8)
    zero = np.zeros_like(one)
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    unit = np.full((1, 256), 127, dtype=np.uint8)
    got = run_gpu(2, rows, h, x_format, "e8m0_block32", "f32", [one, zero], [codes, unit])
    want = oracle_bits(oracle.reduce_scatter_share([one, zero], [codes, unit], x_format, "e8m0_block32", "f32"), "f32")
    assert_parity(got, want, "f32", "e8m0 codes")
    vals = got.view(np.float32).reshape(256, 32)[:, 0]
    st = oracle.scale_decode_table()
    assert np.isnan(vals[255])
    assert np.array_equal(vals[:255].view(np.uint32), st[:255].view(np.uint32))
    assert vals[0].view(np.uint32) == 0x00400000  # 2^-127 kept as a subnormal


@pytest.mark.parametrize("ex", load_worked_examples(), ids=lambda e: e["name"])
def test_worked_example_on_gpu(gpu, ex):
    rows, h = 2, 1024
    xs, ss = build_example(ex, rows=rows, h=h)
    got = run_gpu(len(xs), rows, h, ex["x_format"], ex["scale_layout"], ex["out_dtype"], xs, ss)
    want = int(ex["expected_bits"], 16)
    assert np.all(got == want), (ex["name"], hex(int(got.ravel()[0])), hex(want))


@pytest.mark.parametrize("w", [2, 8])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("x_format", ["e4m3fn", "e5m2"])
def test_every_code_times_every_e8m0_code(gpu, x_format, out_dtype, w):
    # All 256 x 256 (x code, E8M0 code) pairs through the MX kernels: element
    # i holds x code i % 256 under scale code i // 256. The other ranks add
    # -0 (code 0x80), which leaves every product unchanged, so the output is
    # the product itself: the IEEE binary32 product of the two decoded
    # values, bit for bit (2^-127 for code 0, NaN for 255, overflow to
    # infinity, subnormal results, signed zeros). fp32 outputs take the
    # scaled fp8 conversions, 16-bit outputs decode and multiply: both are
    # checked, at W = 2 (fp32: 16-element chunks) and W = 8 (8-element
    # pieces for both outputs).
    rows, h = 8, 8192
    codes = np.tile(np.arange(256, dtype=np.uint8), rows * h // 256).reshape(rows, h)
    neg_zero = np.full((rows, h), 0x80, dtype=np.uint8)
    r_idx, b_idx = np.meshgrid(np.arange(rows), np.arange(h // 32), indexing="ij")
    scale_codes = (r_idx * (h // 256) + b_idx // 8).astype(np.uint8)  # element i -> i // 256
    unit = np.full((rows, h // 32), 127, dtype=np.uint8)
    xs = [codes] + [neg_zero] * (w - 1)
    ss = [scale_codes] + [unit] * (w - 1)
    got = run_gpu(w, rows, h, x_format, "e8m0_block32", out_dtype, xs, ss)
    want_o = oracle_bits(oracle.reduce_scatter_share(xs, ss, x_format, "e8m0_block32", out_dtype), out_dtype)
    assert_parity(got, want_o, out_dtype, f"{x_format} x E8M0 -> {out_dtype}")
    if out_dtype != "f32":
        return
    xt = oracle.decode_table(x_format)
    st = oracle.scale_decode_table()
    i = np.arange(rows * h)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (xt[i % 256] * st[i // 256]).astype(np.float32)
    g = got.reshape(-1)
    nan = np.isnan(prod)
    assert np.array_equal((g & 0x7FFFFFFF) > 0x7F800000, nan)
    assert np.array_equal(g[~nan], prod[~nan].view(np.uint32))
