"""The plain definition of one GPU's share of the quantized reduce-scatter.

TEST INFRASTRUCTURE (part of the CPU oracle; see ``oracle/__init__.py``).

Page "aclnnQuantReduceScatter", Function description: the output is a
reduction, across the data coming from the different ranks, of the product of
the all-to-all'ed scales with the all-to-all'ed quantized x. After the
all-to-all, rank slice r holds ``[rows, H]`` codes of x and the matching
scales; the reduce-scatter output of this GPU is ``[rows, H]``.

For row i, column c, and G the group size of the scale layout (128 columns in
the per-token-per-group mode, 32 in the MX mode, Constraints):

    p_r     = fp32( decode_x(X_r[i, c]) * decode_s(S_r[i, c // G]) )   one rounding
    acc     = p_0
    acc     = fp32( acc + p_r )            for r = 1 .. W-1, in that order
    Y[i, c] = acc                          fp32 output
    Y[i, c] = bf16_rne(acc)                bf16 output
    Y[i, c] = f16_rne(acc)                 fp16 output

Readings of what the page leaves open (each is listed with its reason in the
design notes): the reduction is a left fold in rank order 0..W-1; the fold
starts from p_0 rather than from +0; products and sums are separate binary32
operations, each rounded to nearest-even, with no fused multiply-add and no
wider accumulator; bf16 output rounds the fp32 accumulator to nearest-even;
the scale tensor of a slice is row-major ``[rows, H/G]`` with each group
running along H inside one token; NaN and infinity propagate as in IEEE 754;
subnormals are kept.

numpy float32 ``*`` and ``+`` are single IEEE operations with round-to-
nearest-even, so the explicit loop below is the definition written out.
``np.sum`` is deliberately not used: it may sum pairwise.
"""

import numpy as np

from .decode import GROUP_SIZE, decode_table, scale_decode_table


def _check_shapes(x_slices, scale_slices, scale_layout):
    if len(x_slices) == 0 or len(x_slices) != len(scale_slices):
        raise ValueError("need W >= 1 x slices and as many scale slices")
    g = GROUP_SIZE[scale_layout]
    rows, h = x_slices[0].shape
    if h % g:
        raise ValueError(f"H={h} is not a multiple of the group size {g}")
    for x, s in zip(x_slices, scale_slices):
        if x.shape != (rows, h) or x.dtype != np.uint8:
            raise ValueError("every x slice must be uint8 [rows, H]")
        if s.shape != (rows, h // g):
            raise ValueError(f"every scale slice must be [rows, H/{g}]")
        want = np.float32 if scale_layout == "f32_group128" else np.uint8
        if s.dtype != want:
            raise ValueError(f"scale slices for {scale_layout} must be {np.dtype(want)}")
    return rows, h, g


def dequantize_rank(x_codes, scales, x_format, scale_layout):
    """p_r: decoded x times its decoded scale, one fp32 rounding per element.

    ``x_codes`` is uint8 ``[rows, H]``; ``scales`` is float32 ``[rows, H/128]``
    for "f32_group128" or uint8 E8M0 codes ``[rows, H/32]`` for
    "e8m0_block32". Returns float32 ``[rows, H]``.
    """
    g = GROUP_SIZE[scale_layout]
    xv = decode_table(x_format)[x_codes]
    if scale_layout == "f32_group128":
        sv = np.asarray(scales, dtype=np.float32)
    else:
        sv = scale_decode_table()[scales]
    # Group k covers columns [k*G, (k+1)*G) of the same row: repeat each
    # scale G times along H (a copy, no arithmetic).
    sv_full = np.repeat(sv, g, axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        return (xv * sv_full).astype(np.float32, copy=False)


def fp32_to_bf16_bits(acc):
    """Round binary32 values to bfloat16 (nearest, ties to even); uint16 bits.

    Integer arithmetic on the bit pattern u: adding 0x7FFF plus the lowest
    kept bit and truncating the low 16 bits rounds to nearest with ties to
    even, and carries into the exponent where needed (which also turns values
    past the bf16 maximum into infinity). NaN maps to a quiet NaN of the
    same sign.
    """
    u = np.ascontiguousarray(acc, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    quiet = (u >> 16) | 0x0040
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def fp32_to_f16_bits(acc):
    """Round binary32 values to IEEE binary16 (nearest, ties to even); uint16
    bits. binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; normals
    from 2^-14, subnormal quantum 2^-24, largest finite 65504.

    Written out: in float64 (which holds every binary32 value and every
    quotient below exactly) take the binade E = floor(log2 |v|), the quantum
    2^(max(E, -14) - 10) of binary16 at that magnitude, round |v| / quantum
    to the nearest integer with ties to even, and multiply back. A result
    above 65504 (that is, |v| >= 65520) is infinity. NaN maps to a quiet NaN
    of the same sign.
    """
    with np.errstate(invalid="ignore"):  # signalling NaN patterns widen to quiet NaNs
        v = np.ascontiguousarray(acc, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        _, e2 = np.frexp(a)  # a = m * 2^e2, m in [0.5, 1)
        binade = np.maximum(e2 - 1, -14)
        quantum = np.ldexp(1.0, binade - 10)
        r = np.rint(a / quantum) * quantum  # exact scaling, RNE to an integer
        r = np.where(r > 65504.0, np.inf, r)
        r = np.where(np.isinf(a), np.inf, r)
    mag = np.where(np.isnan(a), 0.0, r).astype(np.float16)  # exact: r is a binary16 value or inf
    bits = mag.view(np.uint16)
    sign = (np.signbit(v).astype(np.uint16) << 15).astype(np.uint16)
    nan_bits = (np.uint16(0x7E00) | sign).astype(np.uint16)
    return np.where(np.isnan(v), nan_bits, bits | sign).astype(np.uint16)


def bf16_bits_to_fp32(bits):
    """Widen bf16 bit patterns (uint16) to float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def reduce_scatter_share(x_slices, scale_slices, x_format, scale_layout, out_dtype):
    """One GPU's share of the quantized reduce-scatter, by definition.

    ``x_slices[r]``: uint8 ``[rows, H]`` codes from rank r, r = 0..W-1.
    ``scale_slices[r]``: that rank's scales (layout as in ``dequantize_rank``).
    Returns float32 ``[rows, H]`` for ``out_dtype == "f32"`` and the uint16
    bit patterns of bf16 or binary16 ``[rows, H]`` for ``out_dtype`` "bf16"
    or "f16".
    """
    if x_format not in ("int8", "e4m3fn", "e5m2"):
        raise ValueError(f"unknown x format {x_format!r}")
    if scale_layout not in GROUP_SIZE:
        raise ValueError(f"unknown scale layout {scale_layout!r}")
    if out_dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown output dtype {out_dtype!r}")
    _check_shapes(x_slices, scale_slices, scale_layout)

    acc = dequantize_rank(x_slices[0], scale_slices[0], x_format, scale_layout)
    with np.errstate(invalid="ignore", over="ignore"):
        for r in range(1, len(x_slices)):
            p = dequantize_rank(x_slices[r], scale_slices[r], x_format, scale_layout)
            acc = acc + p  # float32 + float32: one RNE rounding per element
    assert acc.dtype == np.float32
    if out_dtype == "f32":
        return acc
    if out_dtype == "f16":
        return fp32_to_f16_bits(acc)
    return fp32_to_bf16_bits(acc)


def all_to_all(x_full, scale_full):
    """The all-to-all in front of the reduce (page "aclnnQuantReduceScatter",
    Function description: both the data and the scales are all-to-all'ed).

    ``x_full[r]`` is rank r's ``[BS, H]`` codes and ``scale_full[r]`` its
    scales for all BS rows. Each rank splits its rows into W equal row blocks
    and sends block j to rank j; rank j receives the blocks in rank order.
    Returns, for each rank j, the list of received (x, scales) slices.
    """
    w = len(x_full)
    if w == 0 or len(scale_full) != w:
        raise ValueError("need W >= 1 inputs and as many scale tensors")
    bs = x_full[0].shape[0]
    if bs % w:
        raise ValueError(f"BS={bs} is not a multiple of W={w}")
    rows = bs // w
    received = []
    for j in range(w):
        xs = [x_full[r][j * rows:(j + 1) * rows] for r in range(w)]
        ss = [scale_full[r][j * rows:(j + 1) * rows] for r in range(w)]
        received.append((xs, ss))
    return received


def all_shares(x_full, scale_full, x_format, scale_layout, out_dtype):
    """Every rank's share of the quantized reduce-scatter: the all-to-all,
    then on each rank the reduce of ``reduce_scatter_share``."""
    return [
        reduce_scatter_share(xs, ss, x_format, scale_layout, out_dtype)
        for xs, ss in all_to_all(x_full, scale_full)
    ]
