"""Producer-side quantization: the "quant" in front of the exchange.

TEST INFRASTRUCTURE (part of the CPU oracle; see ``oracle/__init__.py``).

Page "aclnnQuantReduceScatter" takes x already quantized, with its scales,
in one of two modes (Constraints): per-token-per-group (group of 128
columns, fp32 scales; x INT8, FP8 E4M3FN or FP8 E5M2) or MX (blocks of 32,
E8M0 scales; x FP8). The page does not say how a producer chooses the
scales. The readings taken here:

* MX mode follows the conversion of the OCP Microscaling (MX) v1.0
  specification: the shared exponent of a block is floor(log2(amax)) minus
  the largest exponent of the element format (8 for E4M3, 15 for E5M2),
  limited to the E8M0 range [-127, 127]; each element is divided by the
  shared scale (a power of two, so exactly) and rounded to the element
  format, nearest-even, with values beyond the largest normal clamped to it.
  A block of zeros gets the smallest scale, code 0.
* Per-token-per-group mode uses the absolute maximum of the group:
  scale = amax / qmax (one fp32 division) with qmax = 127, 448 or 57344;
  each element is multiplied by qmax / amax (one fp32 division per group,
  one fp32 multiplication per element), clamped to [-qmax, qmax] and
  rounded nearest-even to the element format. The scale is kept at or above
  the smallest normal binary32, 2^-126: a group whose amax / qmax falls below
  it (all-zero groups included) gets scale 2^-126 and multiplier 2^126, so
  the multiplier never overflows.

Inputs are bf16 values (uint16 bit patterns), finite. Every operation is a
single binary32 operation with round-to-nearest-even, so numpy float32 is the
definition written out.
"""

import numpy as np

from .decode import GROUP_SIZE, decode_table
from .reduce import bf16_bits_to_fp32

QMAX = {"int8": 127.0, "e4m3fn": 448.0, "e5m2": 57344.0}
# Largest binade exponent of the element format's normals: 448 = 1.75 * 2^8,
# 57344 = 1.75 * 2^15 (OCP MX v1.0, emax of the FP8 element types).
EMAX_ELEM = {"e4m3fn": 8, "e5m2": 15}
_LAST_FINITE = {"e4m3fn": 0x7E, "e5m2": 0x7B}


def encode_fp8_rne(q, x_format):
    """float32 values within the format's finite range -> codes, nearest
    representable value with ties to the even code.

    Written from the definition: the non-negative finite values of the format
    in code order (they increase with the code) are the candidates; the two
    neighbours of |q| are compared exactly (in float64, which holds every
    float32 and every float8 value exactly); a tie goes to the code whose
    last bit is 0. The sign of q (including -0) sets bit 7.
    """
    q = np.asarray(q, dtype=np.float32)
    last = _LAST_FINITE[x_format]
    vals = decode_table(x_format)[: last + 1].astype(np.float64)
    a = np.abs(q.astype(np.float64))
    if np.any(~np.isfinite(a)) or np.any(a > vals[-1]):
        raise ValueError("encode_fp8_rne needs finite values within the format's range")
    hi = np.searchsorted(vals, a, side="left")  # vals[hi] >= a
    hi = np.minimum(hi, last)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == vals[hi], hi, code).astype(np.uint8)  # exact hits
    neg = np.signbit(q)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def encode_int8_rne(q):
    """float32 values in [-127, 127] -> two's complement codes, nearest
    integer with ties to even."""
    q = np.asarray(q, dtype=np.float32)
    r = np.rint(q)  # IEEE round-to-nearest-even
    return r.astype(np.int8).view(np.uint8)


def quantize(x_bf16_bits, x_format, scale_layout):
    """bf16 ``[tokens, H]`` (uint16 bit patterns) -> (codes uint8
    ``[tokens, H]``, scales ``[tokens, H/G]``: float32 or E8M0 uint8)."""
    if scale_layout == "e8m0_block32" and x_format == "int8":
        raise ValueError("INT8 is paired with fp32 per-group scales only")
    g = GROUP_SIZE[scale_layout]
    v = bf16_bits_to_fp32(x_bf16_bits)
    t, h = v.shape
    if h % g:
        raise ValueError(f"H={h} is not a multiple of {g}")
    if not np.all(np.isfinite(v)):
        raise ValueError("quantize takes finite inputs")
    blocks = v.reshape(t, h // g, g)
    amax = np.max(np.abs(blocks), axis=2)  # exact
    if scale_layout == "f32_group128":
        qmax = np.float32(QMAX[x_format])
        floor = np.float32(2.0 ** -126)
        scale = (amax / qmax).astype(np.float32)
        small = scale < floor
        safe = np.where(small, np.float32(1.0), amax).astype(np.float32)  # avoids 0-division warnings
        mul = np.where(small, np.float32(2.0 ** 126), qmax / safe).astype(np.float32)
        scale = np.where(small, floor, scale).astype(np.float32)
        q = (blocks * mul[:, :, None]).astype(np.float32)
        q = np.clip(q, -qmax, qmax).astype(np.float32)
        q = q.reshape(t, h)
        codes = encode_int8_rne(q) if x_format == "int8" else encode_fp8_rne(q, x_format)
        return codes, scale
    # MX (OCP MX v1.0 conversion)
    emax = EMAX_ELEM[x_format]
    _, e2 = np.frexp(amax)  # amax = m * 2^e2 with m in [0.5, 1): floor(log2(amax)) = e2 - 1
    shared = np.where(amax == 0, -127, e2.astype(np.int32) - 1 - emax)
    shared = np.clip(shared, -127, 127).astype(np.int32)
    inv_scale = np.ldexp(np.float32(1.0), -shared).astype(np.float32)  # 2^-shared, exact
    q = (blocks * inv_scale[:, :, None]).astype(np.float32)
    lim = np.float32(QMAX[x_format])
    q = np.clip(q, -lim, lim).astype(np.float32).reshape(t, h)
    codes = encode_fp8_rne(q, x_format)
    return codes, (shared + 127).astype(np.uint8)
