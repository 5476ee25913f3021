"""Pins for the oracle's fp32 -> binary16 rounding, against numpy's float32
-> float16 conversion (a library routine that rounds to nearest-even), plus
hand-checked edges."""

import numpy as np

from oracle.reduce import fp32_to_f16_bits


def _check(x):
    got = fp32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    g = got[nan]
    assert np.all((g & 0x7C00) == 0x7C00) and np.all((g & 0x0200) != 0)


def test_random_bit_patterns():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(over="ignore"):
        _check(bits.view(np.float32))


def test_binary16_range_dense():
    """Every fp32 pattern whose exponent lies in or near binary16's range,
    sampled densely, with exact ties and their neighbours."""
    rng = np.random.default_rng(6)
    exps = rng.integers(127 - 26, 127 + 17, size=400_000).astype(np.uint32)
    mant = rng.integers(0, 2**23, size=400_000).astype(np.uint32)
    sign = rng.integers(0, 2, size=400_000).astype(np.uint32)
    bits = (sign << 31) | (exps << 23) | mant
    # force ties: low 13 bits = 0x1000 (halfway for normals)
    ties = (bits & ~np.uint32(0x1FFF)) | np.uint32(0x1000)
    with np.errstate(over="ignore"):
        _check(np.concatenate([bits, ties, ties + 1, ties - 1]).view(np.float32))


def test_edges():
    # 2^-25 is half the smallest subnormal (tie -> 0); 3 * 2^-25 is 1.5 quanta (tie -> 2).
    x = np.array([65504.0, 65519.99, 65520.0, 1e30, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
                  2.0 ** -14, 0.0, -0.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    got = fp32_to_f16_bits(x)
    assert list(got[:13]) == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0xFC00, 0x0001, 0x0000, 0x0002,
                              0x0400, 0x0000, 0x8000, 0x7C00, 0xFC00]
    assert (got[13] & 0x7E00) == 0x7E00
