"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
share through the C ABI, and compare with the oracle."""

import sys

import numpy as np
import torch

import quantized_collective_reduction_amd as qrs


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_device(xs, ss, dev="cuda"):
    dx = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in xs]
    ds = [torch.from_numpy(np.ascontiguousarray(s)).to(dev) for s in ss]
    return dx, ds


OUT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def empty_out(rows, h, out_dtype, dev="cuda"):
    return torch.empty((rows, h), dtype=OUT_TORCH[out_dtype], device=dev)


def out_bits(out_t):
    """Device output -> numpy bit patterns (uint32 for fp32, uint16 for bf16)."""
    if out_t.dtype == torch.float32:
        return out_t.cpu().view(torch.int32).numpy().view(np.uint32)
    return out_t.cpu().view(torch.int16).numpy().view(np.uint16)


def run_gpu(world_size, rows, h, x_format, scale_layout, out_dtype, xs, ss, stream=None):
    p = qrs.plan(world_size, rows * world_size, h, x_format, scale_layout, out_dtype)
    dx, ds = to_device(xs, ss)
    out = empty_out(rows, h, out_dtype)
    out.fill_(float("nan"))  # anything not written shows up
    qrs.run(p, dx, ds, out, stream=stream)
    torch.cuda.synchronize()
    return out_bits(out)


def oracle_bits(oracle_out, out_dtype):
    if out_dtype == "f32":
        return np.ascontiguousarray(oracle_out).view(np.uint32)
    return np.ascontiguousarray(oracle_out)


def assert_parity(got_bits, want_bits, out_dtype, what="", max_ulp=0):
    """fp32: bit-exact (any NaN equals any NaN). bf16 / fp16: at most max_ulp
    apart in the ordered-integer sense (+0 equals -0), NaN equals NaN. Both
    sides round the same binary32 accumulator to nearest-even, so the default
    is 0: exact. Returns the count of elements that are not bit-identical."""
    assert got_bits.shape == want_bits.shape, what
    if out_dtype == "f32":
        g_nan = (got_bits & 0x7FFFFFFF) > 0x7F800000
        w_nan = (want_bits & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal(g_nan, w_nan), f"{what}: NaN positions differ"
        ok = ~w_nan
        bad = np.nonzero(got_bits[ok] != want_bits[ok])[0]
        assert bad.size == 0, f"{what}: {bad.size} fp32 mismatches, first at flat {np.nonzero(ok)[0][bad[0]]}"
        return 0
    inf_bits = 0x7F80 if out_dtype == "bf16" else 0x7C00
    g_nan = (got_bits & 0x7FFF) > inf_bits
    w_nan = (want_bits & 0x7FFF) > inf_bits
    assert np.array_equal(g_nan, w_nan), f"{what}: NaN positions differ"
    ok = ~w_nan

    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - b, b)  # sign-magnitude -> ordered (+0 == -0)

    d = np.abs(ordered(got_bits[ok]) - ordered(want_bits[ok]))
    assert d.size == 0 or d.max() <= max_ulp, f"{what}: {out_dtype} distance {d.max()} ulp"
    return int(np.count_nonzero(got_bits[ok] != want_bits[ok]))
