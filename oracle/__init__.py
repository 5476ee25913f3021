"""CPU oracle for one GPU's share of the quantized reduce-scatter.

TEST INFRASTRUCTURE ONLY. This package is the checker the GPU path is
compared against. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The product path (``quantized_collective_reduction_amd``) never imports it
and has no CPU fallback.

What it computes (page "aclnnQuantReduceScatter", Function description):
the output is the reduction over ranks of the elementwise product of the
exchanged scales with the exchanged quantized data. On one GPU the exchange
is already done: the caller hands in W rank slices ``[rows, H]``.

Modules:

* ``decode`` -- 256-entry decode tables for INT8, FP8 E4M3FN, FP8 E5M2 and
  E8M0, built from the bit fields of each code.
* ``reduce`` -- the plain numpy definition: decode, multiply by the group or
  block scale with one fp32 rounding, left fold over ranks 0..W-1 in fp32,
  optional round-to-nearest-even to bf16 done in integer arithmetic.
* ``reduce.all_to_all`` / ``reduce.all_shares`` -- the all-to-all index map
  (rank r's row block j goes to rank j, received in rank order) followed by
  the reduce on every rank: the whole group's reduce-scatter on one host.
* ``exact`` -- brute force with ``fractions.Fraction``: exact products and
  sums, each rounded to binary32 by a rounding routine written from the
  IEEE 754 definition. Used to pin ``reduce`` on tiny inputs.
* ``quantize`` -- the producer side: bf16 activations to codes and scales,
  MX by the OCP Microscaling conversion, per-token-per-group by one fp32
  multiplier qmax / amax per group and one rounded product per element.

Pins (tests marked "not gpu"): every decode table entry against torch's CPU
float8 casts; bf16 rounding against torch's CPU cast; ``reduce`` against
``exact`` on random tiny inputs and on all 256x256 code pairs; closed forms
(exact integer sums under power-of-two scales, rank-permutation invariance
where every partial sum is exact, single-rank identity, cancellation of
opposite ranks, the recursive-summation error bound); hand-derived worked
examples that fix the fold order (three orders told apart by two W = 4
cases) and the absence of fused multiply-add. ``quantize``: its fp8 encoder
against torch's casts and a brute-force nearest-code search, INT8 against
round-half-even, re-quantizing quantized MX blocks, hand-derived shared
exponents, zero and tiny groups, a round-trip error bound, and hand-derived
per-group cases at rounding midpoints that fix the multiplier reading
against dividing by the stored scale or multiplying by its reciprocal.
"""

from .decode import (
    X_FORMATS,
    SCALE_LAYOUTS,
    OUT_DTYPES,
    GROUP_SIZE,
    decode_table,
    scale_decode_table,
)
from .reduce import (
    all_shares,
    all_to_all,
    dequantize_rank,
    reduce_scatter_share,
    fp32_to_bf16_bits,
    fp32_to_f16_bits,
    bf16_bits_to_fp32,
)

__all__ = [
    "X_FORMATS",
    "SCALE_LAYOUTS",
    "OUT_DTYPES",
    "GROUP_SIZE",
    "decode_table",
    "scale_decode_table",
    "all_shares",
    "all_to_all",
    "dequantize_rank",
    "reduce_scatter_share",
    "fp32_to_bf16_bits",
    "fp32_to_f16_bits",
    "bf16_bits_to_fp32",
]
