"""Pins for the oracle's producer-side quantization.

The element encoders are pinned to library routines (torch's float8 casts,
Python's round-half-even) and to a brute-force nearest-code search; the
quantizer to closed forms (re-quantizing an already quantized block
reproduces it, the group maximum maps to the format's maximum, zero groups,
hand-derived MX shared exponents) and to a round-trip error bound.
"""

import math

import numpy as np
import pytest
import torch

from oracle.decode import decode_table, scale_decode_table
from oracle.quantize import EMAX_ELEM, QMAX, encode_fp8_rne, encode_int8_rne, quantize
from oracle.reduce import bf16_bits_to_fp32, fp32_to_bf16_bits

_TORCH = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
_LAST = {"e4m3fn": 0x7E, "e5m2": 0x7B}


def _torch_encode(q, fmt):
    return torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(_TORCH[fmt]).view(torch.uint8).numpy()


def _encoder_probe_values(fmt, rng):
    vals = decode_table(fmt)[: _LAST[fmt] + 1].astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties (float32-representable)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    down = np.nextafter(mids32, np.float32(0))
    lim = np.float32(vals[-1])
    rand = (rng.uniform(-1, 1, 20000) * lim).astype(np.float32)
    tiny = (rng.uniform(-1, 1, 2000) * vals[3]).astype(np.float32)
    allv = np.concatenate([vals.astype(np.float32), mids32, up, down, rand, tiny, [0.0, -0.0]]).astype(np.float32)
    allv = np.concatenate([allv, -allv])
    return allv[np.abs(allv) <= lim]


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_encoder_matches_torch_cast(fmt):
    q = _encoder_probe_values(fmt, np.random.default_rng(2))
    got = encode_fp8_rne(q, fmt)
    want = _torch_encode(q, fmt)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (q[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_encoder_matches_brute_force_nearest(fmt):
    table = decode_table(fmt).astype(np.float64)
    finite = [c for c in range(256) if math.isfinite(table[c])]
    rng = np.random.default_rng(3)
    q = _encoder_probe_values(fmt, rng)[::7]
    got = encode_fp8_rne(q, fmt)
    for v, c in zip(q.astype(np.float64), got):
        # nearest value; ties to the even code; zero keeps the sign of v
        best = min(finite, key=lambda k: (abs(table[k] - v), k & 1, (k >> 7) != (1 if math.copysign(1, v) < 0 else 0)))
        assert table[c] == table[best] and (c & 1) == (best & 1) or (table[c] == 0 and table[best] == 0), (v, c, best)
        assert (c >> 7) == (1 if math.copysign(1.0, v) < 0 else 0)


def test_int8_encoder_is_round_half_even():
    rng = np.random.default_rng(4)
    q = np.concatenate([rng.uniform(-127, 127, 5000), np.arange(-127, 127) + 0.5, np.arange(-127, 128)]).astype(np.float32)
    got = encode_int8_rne(q).view(np.int8)
    want = np.array([round(float(v)) for v in q], dtype=np.int8)  # Python round: half to even
    assert np.array_equal(got, want)


def _bf16(values_f32):
    return fp32_to_bf16_bits(np.asarray(values_f32, dtype=np.float32))


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_mx_requantizing_a_quantized_block_is_exact(fmt):
    """Blocks built as code value * 2^X with the block maximum in the top
    binade of the format quantize back to the same codes and scale X+127."""
    rng = np.random.default_rng(5)
    table = decode_table(fmt)
    emax = EMAX_ELEM[fmt]
    finite = np.nonzero(np.isfinite(table))[0]
    top = [c for c in finite if 2.0 ** emax <= abs(table[c]) < 2.0 ** (emax + 1)]
    t, nb = 6, 8
    codes = rng.choice(finite, size=(t, nb * 32)).astype(np.uint8)
    for i in range(t):
        for b in range(nb):
            codes[i, b * 32 + rng.integers(0, 32)] = rng.choice(top)
    xexp = rng.integers(-60, 60, size=(t, nb))
    vals = table[codes].astype(np.float64) * np.exp2(np.repeat(xexp, 32, axis=1))
    bits = _bf16(vals.astype(np.float32))
    assert np.array_equal(bf16_bits_to_fp32(bits).astype(np.float64), vals)  # exactly representable
    got_codes, got_scales = quantize(bits, fmt, "e8m0_block32")
    assert np.array_equal(got_scales.astype(np.int64), xexp + 127)
    # -0 and +0 codes both decode to zero; compare values
    assert np.array_equal(table[got_codes], table[codes])


@pytest.mark.parametrize("fmt,amax,code", [("e4m3fn", 1.0, 119), ("e4m3fn", 448.0, 127), ("e5m2", 0.75, 111),
                                           ("e5m2", 2.0 ** -100, 127 - 100 - 15), ("e4m3fn", 1.5 * 2.0 ** 127, 246),
                                           ("e4m3fn", 2.0 ** -130, 0)])
def test_mx_shared_exponent_examples(fmt, amax, code):
    """floor(log2(amax)) - emax_elem + 127, limited to [0, 254] (2^-130 is a
    bf16 subnormal whose exponent falls below the E8M0 range)."""
    v = np.zeros((1, 32), dtype=np.float32)
    v[0, 5] = -amax
    _, s = quantize(_bf16(v), fmt, "e8m0_block32")
    assert int(s[0, 0]) == code


@pytest.mark.parametrize("fmt,layout", [("int8", "f32_group128"), ("e4m3fn", "f32_group128"), ("e5m2", "f32_group128"),
                                        ("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32")])
def test_zero_groups_and_group_maximum(fmt, layout):
    rng = np.random.default_rng(6)
    g = 128 if layout == "f32_group128" else 32
    v = (rng.standard_normal((4, 1024)) * 3).astype(np.float32)
    v[1, :g] = 0.0
    v[2, g:2 * g] = -0.0
    codes, scales = quantize(_bf16(v), fmt, layout)
    table = decode_table(fmt)
    assert np.all(table[codes[1, :g]] == 0) and np.all(table[codes[2, g:2 * g]] == 0)
    if layout == "f32_group128":
        assert scales[1, 0] == np.float32(2.0 ** -126) and scales[2, 1] == np.float32(2.0 ** -126)
        # the element of largest magnitude in each nonzero group maps to +-qmax
        vb = bf16_bits_to_fp32(_bf16(v)).reshape(4, -1, g)
        idx = np.argmax(np.abs(vb), axis=2)
        cb = table[codes].reshape(4, -1, g)
        for i in range(4):
            for k in range(vb.shape[1]):
                if np.any(vb[i, k] != 0):
                    assert abs(cb[i, k, idx[i, k]]) == QMAX[fmt]
    else:
        assert scales[1, 0] == 0 and scales[2, 1] == 0


@pytest.mark.parametrize("fmt,layout", [("int8", "f32_group128"), ("e4m3fn", "f32_group128"), ("e5m2", "f32_group128"),
                                        ("e4m3fn", "e8m0_block32"), ("e5m2", "e8m0_block32")])
def test_round_trip_error_bound(fmt, layout):
    """|v - decode(code) * scale| is at most half the spacing of the element
    format at the scaled value (plus the rounding of the scaling itself), in
    units of the scale. In MX mode a scaled value may exceed the format's
    largest normal (the shared exponent only fixes the binade of the block
    maximum) and is clamped to it: that excess adds to the bound."""
    rng = np.random.default_rng(7)
    g = 128 if layout == "f32_group128" else 32
    v = (rng.standard_normal((8, 2048)) * np.exp2(rng.integers(-20, 20, size=(8, 1)))).astype(np.float32)
    bits = _bf16(v)
    v = bf16_bits_to_fp32(bits).astype(np.float64)
    codes, scales = quantize(bits, fmt, layout)
    table = decode_table(fmt).astype(np.float64)
    s = scales.astype(np.float64) if layout == "f32_group128" else scale_decode_table()[scales].astype(np.float64)
    s_full = np.repeat(s, g, axis=1)
    deq = table[codes] * s_full
    vals = np.sort(np.unique(np.abs(table[np.isfinite(table)])))
    spacing = np.diff(vals)
    q = np.abs(v) / s_full
    k = np.clip(np.searchsorted(vals, q) - 1, 0, len(spacing) - 1)
    half_step = 0.5 * spacing[k] * s_full
    clamp_excess = np.maximum(q - QMAX[fmt], 0) * s_full
    err = np.abs(v - deq)
    assert np.all(err <= (half_step + clamp_excess) * (1 + 2.0 ** -20) + np.abs(v) * 2.0 ** -22)
    if layout == "f32_group128":
        assert np.all(clamp_excess <= np.abs(v) * 2.0 ** -22)


@pytest.mark.parametrize("fmt", ["int8", "e4m3fn", "e5m2"])
def test_tiny_groups_use_the_smallest_normal_scale(fmt):
    """amax / qmax below 2^-126: scale 2^-126, codes = RNE(v * 2^126) (exact
    products); above it the ordinary rule applies."""
    v = np.zeros((2, 1024), dtype=np.float32)
    v[0, :128] = np.float32(2.0 ** -130) * np.arange(128, dtype=np.float32) / 128  # bf16-exact
    v[1, :128] = np.float32(2.0 ** -110)
    bits = _bf16(v)
    vv = bf16_bits_to_fp32(bits)
    codes, scales = quantize(bits, fmt, "f32_group128")
    assert scales[0, 0] == np.float32(2.0 ** -126)
    want = encode_int8_rne(vv[0, :128] * np.float32(2.0 ** 126)) if fmt == "int8" else \
        encode_fp8_rne(vv[0, :128] * np.float32(2.0 ** 126), fmt)
    assert np.array_equal(codes[0, :128], want)
    assert scales[1, 0] == np.float32(2.0 ** -110) / np.float32(QMAX[fmt])
    assert np.all(decode_table(fmt)[codes[1, :128]] == QMAX[fmt])
