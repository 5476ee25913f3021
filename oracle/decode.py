"""Decode tables: each byte code of an element or scale format -> its value.

TEST INFRASTRUCTURE (part of the CPU oracle; see ``oracle/__init__.py``).

Formats (page "aclnnQuantReduceScatter", Constraints): x is INT8,
FLOAT8_E4M3FN or FLOAT8_E5M2; scales are FLOAT (binary32) in the
per-token-per-group mode with a group of 128 columns, or FLOAT8_E8M0 in the
MX mode. The page names the formats without defining them; the bit layouts
used here are the OCP 8-bit floating point formats (E4M3 in its "FN" form:
no infinities, one NaN mantissa pattern per sign) and the OCP Microscaling
v1.0 shared-scale format E8M0. The page also lists HIFLOAT8 for x but never
defines it, so it has no table here.

The MX block size of 32 follows from the page's MX scales size, one byte per
32 elements of x (Constraints, the HCCL_BUFFSIZE sizing rule); the per-group
size of 128 is stated with the per-token-per-group mode.

Every table entry is computed from integer bit fields with ``math.ldexp``.
All values are exactly representable in binary32, so storing them as
``np.float32`` loses nothing.
"""

import math

import numpy as np

X_FORMATS = ("int8", "e4m3fn", "e5m2")
SCALE_LAYOUTS = ("f32_group128", "e8m0_block32")
OUT_DTYPES = ("f32", "bf16", "f16")

# Elements of one row that share one scale, per scale layout.
GROUP_SIZE = {"f32_group128": 128, "e8m0_block32": 32}


def decode_int8(code: int) -> float:
    """Two's complement byte: codes 0..127 are themselves, 128..255 are code-256."""
    return float(code if code < 128 else code - 256)


def decode_e4m3fn(code: int) -> float:
    """OCP FP8 E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 15 with mantissa 7 is NaN (keeping the code's sign bit);
    there is no infinity, so the rest of exponent 15 are ordinary numbers up
    to 448. Exponent field 0 is subnormal: m * 2^(1-7-3).
    """
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return math.copysign(math.nan, sign)
    if e == 0:
        mag = math.ldexp(m, 1 - 7 - 3)
    else:
        mag = math.ldexp(8 + m, e - 7 - 3)
    return math.copysign(mag, sign)


def decode_e5m2(code: int) -> float:
    """OCP FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits.

    Exponent field 31 is infinity (mantissa 0) or NaN (mantissa != 0), as in
    IEEE 754. Exponent field 0 is subnormal: m * 2^(1-15-2).
    """
    s, e, m = code >> 7, (code >> 2) & 0x1F, code & 0x3
    sign = -1.0 if s else 1.0
    if e == 0x1F:
        return math.copysign(math.inf if m == 0 else math.nan, sign)
    if e == 0:
        mag = math.ldexp(m, 1 - 15 - 2)
    else:
        mag = math.ldexp(4 + m, e - 15 - 2)
    return math.copysign(mag, sign)


def decode_e8m0(code: int) -> float:
    """OCP MX E8M0 scale: an unsigned biased exponent, 2^(code-127).

    Code 255 is NaN. Code 0 is 2^-127, a binary32 subnormal, kept as such.
    """
    if code == 0xFF:
        return math.nan
    return math.ldexp(1.0, code - 127)


_X_DECODERS = {"int8": decode_int8, "e4m3fn": decode_e4m3fn, "e5m2": decode_e5m2}


def decode_table(x_format: str) -> np.ndarray:
    """256-entry float32 table: table[code] is the value of byte ``code``."""
    dec = _X_DECODERS[x_format]
    return np.array([dec(c) for c in range(256)], dtype=np.float32)


def scale_decode_table() -> np.ndarray:
    """256-entry float32 table for E8M0 scale bytes."""
    return np.array([decode_e8m0(c) for c in range(256)], dtype=np.float32)
