"""Brute force with exact rationals, for pinning ``oracle.reduce`` on tiny inputs.

TEST INFRASTRUCTURE (part of the CPU oracle; see ``oracle/__init__.py``).

Each product and each partial sum of the definition (page
"aclnnQuantReduceScatter", Function description; readings as in
``oracle.reduce``) is formed exactly as a ``fractions.Fraction`` and then
rounded to binary32 by ``round_to_binary32``, which is written from the IEEE
754 definition of round-to-nearest, ties-to-even: pick the quantum of the
binade the exact value falls in (or the subnormal quantum 2^-149 below
2^-126), round the exact quotient to the nearest integer with ties to even,
and overflow to infinity at or beyond the midpoint between the largest finite
value and 2^128. Signed zeros follow IEEE 754: a product's zero takes the
xor of the operand signs; an exact zero sum of two operands is +0 unless
both are -0.

Nothing here touches numpy arithmetic; inputs are Python floats (exact
copies of the decoded binary32 values). Non-finite inputs are rejected: the
brute force covers finite arithmetic only.
"""

import math
from fractions import Fraction

_MIN_NORMAL_EXP = -126
_SUBNORMAL_QUANTUM = Fraction(1, 2**149)
_MANTISSA_BITS = 24
# Largest finite binary32 is (2^24 - 1) * 2^104; the midpoint to 2^128 is
# (2^24 - 1/2) * 2^104. At or above it, round-to-nearest-even gives infinity.
_OVERFLOW_THRESHOLD = (Fraction(2**24) - Fraction(1, 2)) * 2**104


def _floor_log2(a: Fraction) -> int:
    """The integer E with 2^E <= a < 2^(E+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # The bit-length difference is E or E+1; settle it exactly.
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    return e


def round_to_binary32(q: Fraction, zero_sign: float = 1.0) -> float:
    """The binary32 value nearest to q, ties to even, as a Python float.

    ``zero_sign`` gives the sign of the result when q is exactly zero (IEEE
    754 fixes that sign from the operation, not from q).
    """
    if q == 0:
        return math.copysign(0.0, zero_sign)
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    if a >= _OVERFLOW_THRESHOLD:
        return math.copysign(math.inf, sign)
    e = _floor_log2(a)
    if e < _MIN_NORMAL_EXP:
        quantum = _SUBNORMAL_QUANTUM
    else:
        quantum = Fraction(2) ** (e - (_MANTISSA_BITS - 1))
    n = a / quantum
    whole = n.numerator // n.denominator
    frac = n - whole
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    # Results that underflow to zero keep the sign of the exact value.
    return math.copysign(float(whole * quantum), sign)


def _check_finite(v: float):
    if not math.isfinite(v):
        raise ValueError("exact brute force handles finite inputs only")


def mul_binary32(a: float, b: float) -> float:
    """fp32(a * b) for binary32 a, b: exact product, one rounding."""
    _check_finite(a)
    _check_finite(b)
    zero_sign = -1.0 if (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0 else 1.0
    return round_to_binary32(Fraction(a) * Fraction(b), zero_sign)


def add_binary32(a: float, b: float) -> float:
    """fp32(a + b) for binary32 a, b: exact sum, one rounding.

    An exact zero sum is +0 in round-to-nearest, except (-0) + (-0) = -0.
    """
    _check_finite(a)
    _check_finite(b)
    both_neg_zero = a == 0 and b == 0 and math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0
    return round_to_binary32(Fraction(a) + Fraction(b), -1.0 if both_neg_zero else 1.0)


def share_element(x_values, scale_values) -> float:
    """One output element: rank-ordered fold of the rounded products.

    ``x_values[r]`` and ``scale_values[r]`` are the decoded binary32 values of
    rank r's element and of its scale.
    """
    if len(x_values) == 0 or len(x_values) != len(scale_values):
        raise ValueError("need W >= 1 values and as many scales")
    acc = mul_binary32(x_values[0], scale_values[0])
    for xv, sv in zip(x_values[1:], scale_values[1:]):
        acc = add_binary32(acc, mul_binary32(xv, sv))
    return acc


def exact_sum(x_values, scale_values) -> Fraction:
    """The mathematically exact sum of x_r * s_r, with no rounding at all."""
    total = Fraction(0)
    for xv, sv in zip(x_values, scale_values):
        _check_finite(xv)
        _check_finite(sv)
        total += Fraction(xv) * Fraction(sv)
    return total
