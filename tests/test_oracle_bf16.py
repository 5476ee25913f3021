"""Pins for the oracle's fp32 -> bf16 rounding (integer round-to-nearest-even).

Checked against torch's CPU float32 -> bfloat16 cast, a library routine that
rounds to nearest-even, on random bit patterns, constructed ties, the
overflow edge, subnormals and specials.
"""

import numpy as np
import torch

from oracle.reduce import bf16_bits_to_fp32, fp32_to_bf16_bits


def _torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _check(x_f32):
    got = fp32_to_bf16_bits(x_f32)
    want = _torch_bf16_bits(x_f32)
    nan = np.isnan(x_f32)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN (quiet), with its sign.
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x007F) != 0)
    assert np.all((g & 0x0040) != 0)
    assert np.array_equal(g >> 15, x_f32[nan].view(np.uint32) >> 31)


def test_random_bit_patterns():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    _check(bits.view(np.float32))


def test_constructed_ties_and_neighbours():
    rng = np.random.default_rng(7)
    hi = rng.integers(0, 2**16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16
    lows = np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    _check(bits.view(np.float32))


def test_documented_ties():
    x = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000], dtype=np.uint32).view(np.float32)
    assert list(fp32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF80, 0xBF82]


def test_overflow_subnormal_and_specials():
    bits = np.array(
        [
            0x7F7FFFFF,  # fp32 max -> rounds past bf16 max to +inf
            0x7F7F7FFF,  # just below the midpoint above bf16 max -> bf16 max
            0x7F7F8000,  # exactly the midpoint above bf16 max (odd) -> +inf
            0xFF7FFFFF,
            0x7F800000,
            0xFF800000,
            0x00000001,  # smallest subnormal -> +0
            0x00008000,  # tie at the smallest bf16 subnormal's half -> 0
            0x00018000,  # tie between subnormals 1 and 2 -> 2
            0x80000000,
            0x00000000,
            0x7FC00000,
            0xFFC00001,
            0x7F800001,  # signalling NaN -> quiet NaN
        ],
        dtype=np.uint32,
    ).view(np.float32)
    _check(bits)


def test_widening_is_exact_inverse_on_bf16_values():
    all_bf16 = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_fp32(all_bf16)
    back = fp32_to_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], all_bf16[~nan])
