"""Seeded synthetic inputs for the quantized reduce-scatter share.

Shared by the tests, the benchmark and the smoke check. This module only
draws random numbers and encodes them into the input formats (with torch's
CPU float8 casts); it holds none of the arithmetic the reduction performs:
no decoding, no scaling, no summing.

Shapes follow the page "aclnnQuantReduceScatter": x is ``[BS, H]`` one byte
per element per rank (Constraints, the xDataSize formula); after the
all-to-all each of the W ranks contributes a ``[BS/W, H]`` slice to this
GPU's share; scales are fp32 per (token, 128 columns) or E8M0 per 32
elements (Constraints, the scalesDataSize formulas). The pages print no
workload, so value distributions are this project's: normal values scaled by
a sigma for the float8 formats, uniform integers for INT8, log-uniform
power-of-two exponents for fp32 scales, uniform E8M0 codes in a band around
127.

Random stream: ``numpy.random.default_rng([seed, r])`` for rank r, so each
rank's stream depends only on the seed and the rank; x is drawn first, then
the scales.
"""

from dataclasses import dataclass, replace
from typing import List, Tuple

import numpy as np

GROUP_SIZE = {"f32_group128": 128, "e8m0_block32": 32}


@dataclass(frozen=True)
class Workload:
    """One problem: W rank slices of ``[rows, H]`` plus their scales."""

    name: str
    world_size: int
    bs: int  # tokens per rank before the all-to-all; rows = bs // world_size
    h: int
    x_format: str  # "int8" | "e4m3fn" | "e5m2"
    scale_layout: str  # "f32_group128" | "e8m0_block32"
    out_dtype: str  # "f32" | "bf16" | "f16"
    # x values: "int_uniform" draws integers in [-x_param, x_param];
    # "normal" draws N(0,1) * x_param, clipped to the format's finite range.
    x_dist: str = "normal"
    x_param: float = 1.0
    # fp32 scales: 2**uniform(lo, hi). E8M0 scales: integer codes in [lo, hi].
    scale_lo: float = -8.0
    scale_hi: float = 0.0
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.bs // self.world_size

    @property
    def group(self) -> int:
        return GROUP_SIZE[self.scale_layout]

    @property
    def out_bytes_per_elem(self) -> int:
        return 4 if self.out_dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the share must move: W x slices, W scale slices, one output.

        Per output element: W * (1 + 1/32) + (4 or 2) bytes, since both scale
        layouts carry 1/32 byte per element (4 B per 128, or 1 B per 32).
        """
        elems = self.rows * self.h
        scale_bytes = (elems // self.group) * (4 if self.scale_layout == "f32_group128" else 1)
        return self.world_size * (elems + scale_bytes) + elems * self.out_bytes_per_elem

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the hot path.
WORKLOADS = {
    "w2_bs32_h1024_int8_f32": Workload("w2_bs32_h1024_int8_f32", 2, 32, 1024, "int8", "f32_group128", "f32",
                   x_dist="int_uniform", x_param=127, scale_lo=-10, scale_hi=-4),
    "w4_bs4096_h4096_e4m3_bf16": Workload("w4_bs4096_h4096_e4m3_bf16", 4, 4096, 4096, "e4m3fn", "f32_group128", "bf16",
                   x_dist="normal", x_param=64, scale_lo=-12, scale_hi=-2),
    "w8_bs8192_h7168_e5m2_bf16": Workload("w8_bs8192_h7168_e5m2_bf16", 8, 8192, 7168, "e5m2", "f32_group128", "bf16",
                   x_dist="normal", x_param=1024, scale_lo=-16, scale_hi=-4),
    "w8_bs16384_h8192_mx_e4m3_bf16": Workload("w8_bs16384_h8192_mx_e4m3_bf16", 8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16",
                   x_dist="normal", x_param=32, scale_lo=117, scale_hi=137),
    "w8_bs65536_h5120_mx_e5m2_f32": Workload("w8_bs65536_h5120_mx_e5m2_f32", 8, 65536, 5120, "e5m2", "e8m0_block32", "f32",
                   x_dist="normal", x_param=256, scale_lo=112, scale_hi=142),
}

# Largest finite magnitude of each float8 format (clip before encoding: the
# torch casts do not saturate).
_FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}


def _encode_fp8(values_f32: np.ndarray, x_format: str) -> np.ndarray:
    """float32 -> float8 codes (uint8) via torch's CPU cast (nearest-even)."""
    import torch

    dt = torch.float8_e4m3fn if x_format == "e4m3fn" else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(values_f32)).to(dt)
    return t.view(torch.uint8).numpy().copy()


def _draw_x(rng, wl: Workload) -> np.ndarray:
    shape = (wl.rows, wl.h)
    if wl.x_format == "int8":
        if wl.x_dist != "int_uniform":
            raise ValueError("INT8 inputs use x_dist='int_uniform'")
        k = int(wl.x_param)
        return rng.integers(-k, k + 1, size=shape, dtype=np.int8).view(np.uint8)
    if wl.x_dist != "normal":
        raise ValueError("float8 inputs use x_dist='normal'")
    lim = _FP8_MAX[wl.x_format]
    v = rng.standard_normal(size=shape) * wl.x_param
    np.clip(v, -lim, lim, out=v)
    return _encode_fp8(v.astype(np.float32), wl.x_format)


def _draw_scales(rng, wl: Workload) -> np.ndarray:
    shape = (wl.rows, wl.h // wl.group)
    if wl.scale_layout == "f32_group128":
        return np.exp2(rng.uniform(wl.scale_lo, wl.scale_hi, size=shape)).astype(np.float32)
    return rng.integers(int(wl.scale_lo), int(wl.scale_hi) + 1, size=shape, dtype=np.uint8)


def generate_rank(wl: Workload, r: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rank r's slice: (x codes uint8 [rows, H], scales [rows, H/G])."""
    rng = np.random.default_rng([wl.seed, r])
    x = _draw_x(rng, wl)
    s = _draw_scales(rng, wl)
    return x, s


def generate(wl: Workload) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """All W slices of a workload, deterministic from ``wl.seed``."""
    xs, ss = [], []
    for r in range(wl.world_size):
        x, s = generate_rank(wl, r)
        xs.append(x)
        ss.append(s)
    return xs, ss


def generate_full(wl: Workload) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Every rank's input BEFORE the all-to-all: x ``[BS, H]`` and scales
    ``[BS, H/G]`` per rank, same distributions as ``generate``; rank r draws
    from ``default_rng([seed, r, 1])`` (a stream of its own)."""
    full = wl.with_(world_size=1)  # shapes: rows == bs
    xs, ss = [], []
    for r in range(wl.world_size):
        rng = np.random.default_rng([wl.seed, r, 1])
        xs.append(_draw_x(rng, full))
        ss.append(_draw_scales(rng, full))
    return xs, ss


def generate_activations(wl: Workload, r: int, tokens: int = None) -> np.ndarray:
    """Rank r's bf16 activations ``[tokens, H]`` (default tokens = BS) as
    uint16 bit patterns, for the producer-side quantization: N(0,1) values
    times a per-token power of two drawn uniformly from 2^-8 .. 2^8, encoded
    by torch's nearest-even float32 -> bf16 cast. Stream
    ``default_rng([seed, r, 2])``."""
    import torch

    t = wl.bs if tokens is None else tokens
    rng = np.random.default_rng([wl.seed, r, 2])
    v = rng.standard_normal(size=(t, wl.h)).astype(np.float32)
    v *= np.exp2(rng.integers(-8, 9, size=(t, 1))).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
