"""Pins for the oracle's decode tables (all 256 codes of every format).

The tables are built from bit fields (oracle/decode.py); here they are checked
against an independent library routine (torch's CPU float8 / int8 casts) and
against named code points read off the OCP format specifications
(tests/golden/format_specials.json).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.decode import decode_table, scale_decode_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_specials.json")

_TORCH_DTYPES = {
    "int8": torch.int8,
    "e4m3fn": torch.float8_e4m3fn,
    "e5m2": torch.float8_e5m2,
}


def _torch_table(dt):
    return torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float32).numpy()


def _same_values(a, b):
    """Bitwise equality with any NaN equal to any NaN; signed zeros must match."""
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    if not np.array_equal(nan_a, nan_b):
        return False
    ok = ~nan_a
    return np.array_equal(a[ok].view(np.uint32), b[ok].view(np.uint32))


@pytest.mark.parametrize("fmt", ["int8", "e4m3fn", "e5m2"])
def test_x_table_matches_torch_cast(fmt):
    assert _same_values(decode_table(fmt), _torch_table(_TORCH_DTYPES[fmt]))


def test_e8m0_table_matches_torch_cast():
    assert _same_values(scale_decode_table(), _torch_table(torch.float8_e8m0fnu))


def _parse(v: str) -> float:
    if v.startswith("2^"):
        return math.ldexp(1.0, int(v[2:]))
    return float(v)


@pytest.mark.parametrize("fmt", ["int8", "e4m3fn", "e5m2", "e8m0"])
def test_named_code_points(fmt):
    with open(GOLDEN) as f:
        specials = json.load(f)[fmt]
    table = scale_decode_table() if fmt == "e8m0" else decode_table(fmt)
    for code_s, val_s in specials.items():
        got = float(table[int(code_s, 16)])
        want = _parse(val_s)
        if math.isnan(want):
            assert math.isnan(got), (fmt, code_s)
        else:
            assert got == want, (fmt, code_s, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), (fmt, code_s)


@pytest.mark.parametrize("fmt,last_finite", [("e4m3fn", 0x7E), ("e5m2", 0x7B)])
def test_float8_codes_are_monotone_and_symmetric(fmt, last_finite):
    """Positive codes increase strictly; code | 0x80 is the negation.

    A wrong bias, field width or subnormal rule breaks monotonicity or the
    ratio of neighbouring binades.
    """
    t = decode_table(fmt).astype(np.float64)
    pos = t[: last_finite + 1]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80 : 0x80 + last_finite + 1], -pos)
    mbits = 3 if fmt == "e4m3fn" else 2
    step = 1 << mbits
    # Between normal binades the value doubles.
    for c in range(step, last_finite + 1 - step):
        assert t[c + step] == 2 * t[c]


def test_e8m0_is_power_of_two_ladder():
    t = scale_decode_table().astype(np.float64)
    assert np.array_equal(t[1:255] / t[:254], np.full(254, 2.0))
    assert t[127] == 1.0
