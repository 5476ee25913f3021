"""Pins for the per-token-per-group quantizer's reading: which binary32
operations form a code from v, the group maximum amax and qmax.

The page "aclnnQuantReduceScatter" (Constraints) fixes the per-group mode
(128 columns, FLOAT scales, INT8 / E4M3FN / E5M2 codes) but not how a
producer forms the codes. The oracle multiplies each element by one
per-group multiplier fl(qmax / amax); dividing by the stored scale
fl(amax / qmax) is the other plausible reading, and it rounds differently on
real inputs. tests/golden/quantize_examples.json holds hand-derived groups
whose exact value v * qmax / amax is a rounding midpoint, so the binary32
roundings decide the code: the oracle must give the derived codes, and a
copy of the quantizer with the other reading (or another plausible slip)
planted in it must fail at least one of them.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.decode import decode_table
from oracle.quantize import QMAX, encode_fp8_rne, encode_int8_rne, quantize
from oracle.reduce import bf16_bits_to_fp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_examples.json")
AMAX_COL, V_COL = 5, 77  # both in the first 128-column group


def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def example_input(ex, h=1024):
    """One bf16 row [1, h]: amax and v in group 0, every other element 0."""
    bits = np.zeros((1, h), dtype=np.uint16)
    bits[0, AMAX_COL] = int(ex["amax_bf16"], 16)
    bits[0, V_COL] = int(ex["v_bf16"], 16)
    return bits


def _check(codes, scales, ex):
    qmax_code = {"int8": 0x7F, "e4m3fn": 0x7E, "e5m2": 0x7B}[ex["x_format"]]
    scale_bits = np.ascontiguousarray(scales, dtype=np.float32).view(np.uint32)
    return (int(codes[0, V_COL]) == int(ex["expected_code"], 16)
            and int(codes[0, AMAX_COL]) == qmax_code
            and int(scale_bits[0, 0]) == int(ex["expected_scale_bits"], 16))


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_oracle_gives_the_derived_code(ex):
    codes, scales = quantize(example_input(ex), ex["x_format"], "f32_group128")
    assert _check(codes, scales, ex), (ex["name"], hex(int(codes[0, V_COL])), hex(int(scales.view(np.uint32)[0, 0])))
    # every other element of the row is 0 -> code of zero
    rest = np.delete(codes[0], [AMAX_COL, V_COL])
    assert np.all(decode_table(ex["x_format"])[rest] == 0)


def _rne32(q: Fraction) -> Fraction:
    """Nearest binary32 of an exact rational that float64 holds exactly
    (checked), via numpy's float64 -> float32 conversion (IEEE RNE)."""
    d = float(q)
    assert Fraction(d) == q, "not exact in float64"
    return Fraction(float(np.float32(d)))


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_derivation_numbers_are_the_binary32_roundings(ex):
    """The multiplier and product a derivation states are the binary32
    roundings of the exact quotient and product, the exact value is a
    midpoint of two neighbouring codes, and the stated other-reading code
    is what dividing by the rounded scale gives."""
    fmt = ex["x_format"]
    amax = Fraction(float(bf16_bits_to_fp32(np.array([int(ex["amax_bf16"], 16)], dtype=np.uint16))[0]))
    v = Fraction(float(bf16_bits_to_fp32(np.array([int(ex["v_bf16"], 16)], dtype=np.uint16))[0]))
    qmax = Fraction(int(QMAX[fmt]))
    m, k = ex["multiplier"]
    mul = Fraction(m) * Fraction(2) ** k
    assert m < 2 ** 24
    # qmax / amax is not exact in float64 in general: bracket it instead.
    exact_q = qmax / amax
    ulp = Fraction(2) ** k
    assert abs(mul - exact_q) <= ulp / 2
    pm, pk = ex["product"]
    prod = Fraction(pm) * Fraction(2) ** pk
    assert pm < 2 ** 24 and _rne32(v * mul) == prod
    # the exact value sits on a midpoint of the format's neighbouring values
    target = v * qmax / amax
    table = decode_table(fmt).astype(np.float64)
    finite = sorted({Fraction(float(t)) for t in table if np.isfinite(t)})
    lo = max(t for t in finite if t < target)
    hi = min(t for t in finite if t > target)
    assert target == (lo + hi) / 2
    # the other readings, from the rounded scale fl(amax / qmax), then the
    # same encoder: v / scale, and v * fl(1 / scale)
    scale = np.float32(np.float64(amax) / np.float64(qmax))
    assert int(scale.view(np.uint32)) == int(ex["expected_scale_bits"], 16)
    v32 = np.float32(float(v))
    divided = np.float32(np.float64(v32) / np.float64(scale))
    recip = np.float32(np.float64(np.float32(1.0)) / np.float64(scale))
    times_recip = np.float32(np.float64(v32) * np.float64(recip))
    enc = encode_int8_rne if fmt == "int8" else (lambda q: encode_fp8_rne(q, fmt))
    other = ex["other_readings"]
    assert int(enc(np.array([divided], dtype=np.float32))[0]) == int(other["divide_by_scale"], 16)
    assert int(enc(np.array([times_recip], dtype=np.float32))[0]) == int(other["multiply_by_reciprocal_of_scale"], 16)
    assert any(c != ex["expected_code"] for c in other.values()), "the case separates no other reading"


def test_each_other_reading_is_separated_twice():
    seen = {}
    for ex in load_examples():
        for name, c in ex["other_readings"].items():
            seen[name] = seen.get(name, 0) + (c != ex["expected_code"])
    assert seen and all(n >= 2 for n in seen.values()), seen


# ------------------------------------------------------------ planted mistakes


def _group_quantize(bits, fmt, *, divide_by_scale=False, reciprocal_of_scale=False, wide_product=False,
                    ties_away=False):
    """A configurable re-statement of the per-group quantizer, used only to
    plant mistakes (each flag is one plausible slip)."""
    v = bf16_bits_to_fp32(bits)
    t, h = v.shape
    blocks = v.reshape(t, h // 128, 128)
    amax = np.max(np.abs(blocks), axis=2)
    qmax = np.float32(QMAX[fmt])
    scale = (amax / qmax).astype(np.float32)
    small = scale < np.float32(2.0 ** -126)
    safe = np.where(small, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(small, np.float32(2.0 ** -126), scale).astype(np.float32)
    if divide_by_scale:
        q = (blocks / scale[:, :, None]).astype(np.float32)
    elif reciprocal_of_scale:
        q = (blocks * (np.float32(1.0) / scale)[:, :, None].astype(np.float32)).astype(np.float32)
    elif wide_product:
        q = (blocks.astype(np.float64) * (np.float64(qmax) / safe.astype(np.float64))[:, :, None])
        q = np.where(small[:, :, None], blocks.astype(np.float64) * 2.0 ** 126, q)
    else:
        mul = np.where(small, np.float32(2.0 ** 126), qmax / safe).astype(np.float32)
        q = (blocks * mul[:, :, None]).astype(np.float32)
    q = np.clip(q, -float(qmax), float(qmax)).reshape(t, h)
    if ties_away:
        q64 = np.asarray(q, dtype=np.float64)
        if fmt == "int8":
            return (np.sign(q64) * np.floor(np.abs(q64) + 0.5)).astype(np.int8).view(np.uint8), scale
        codes = encode_fp8_rne(q.astype(np.float32), fmt)
        last = {"e4m3fn": 0x7E, "e5m2": 0x7B}[fmt]
        vals = decode_table(fmt)[: last + 1].astype(np.float64)
        a = np.abs(q64)
        hi = np.minimum(np.searchsorted(vals, a, side="left"), last)
        lo = np.maximum(hi - 1, 0)
        tie = (a - vals[lo] == vals[hi] - a) & (a != vals[hi])
        away = np.where(np.signbit(q64), hi | 0x80, hi).astype(np.uint8)
        return np.where(tie, away, codes).astype(np.uint8), scale
    q = q.astype(np.float32)
    codes = encode_int8_rne(q) if fmt == "int8" else encode_fp8_rne(q, fmt)
    return codes, scale


MUTANTS = {
    "divide_by_the_scale": dict(divide_by_scale=True),
    "multiply_by_the_reciprocal_of_the_scale": dict(reciprocal_of_scale=True),
    "unrounded_multiplier_and_product": dict(wide_product=True),
    "ties_away_from_zero": dict(ties_away=True),
}


def _examples_pass(fn):
    for ex in load_examples():
        codes, scales = fn(example_input(ex), ex["x_format"])
        if not _check(codes, scales, ex):
            return False
    return True


def test_unmutated_restatement_is_the_oracle():
    rng = np.random.default_rng(11)
    for fmt in ("int8", "e4m3fn", "e5m2"):
        v = (rng.standard_normal((16, 1024)) * 3).astype(np.float32)
        v[3, :128] = 0.0
        v[4, 128:256] *= np.float32(2.0 ** -120)
        bits = (np.ascontiguousarray(v).view(np.uint32) >> 16).astype(np.uint16)
        want_c, want_s = quantize(bits, fmt, "f32_group128")
        got_c, got_s = _group_quantize(bits, fmt)
        assert np.array_equal(got_c, want_c) and np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    assert _examples_pass(lambda b, f: _group_quantize(b, f))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_quantizer_mistake_is_caught(name):
    kw = MUTANTS[name]
    assert not _examples_pass(lambda b, f: _group_quantize(b, f, **kw)), f"no example rejects {name}"


@pytest.mark.parametrize("reading,kw", [("divide_by_scale", dict(divide_by_scale=True)),
                                         ("multiply_by_reciprocal_of_scale", dict(reciprocal_of_scale=True))])
def test_restated_other_readings_give_the_stated_codes(reading, kw):
    """The planted readings, run as quantizers, give the codes each
    derivation states for them."""
    for ex in load_examples():
        codes, _ = _group_quantize(example_input(ex), ex["x_format"], **kw)
        assert int(codes[0, V_COL]) == int(ex["other_readings"][reading], 16), (reading, ex["name"])
