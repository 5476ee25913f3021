"""The pins catch plausible mistakes: plant each mistake in a copy of the
oracle (on the CPU) and check that at least one pin rejects it, while the
real oracle passes the same pins.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle.decode import GROUP_SIZE, decode_table, scale_decode_table
from oracle.reduce import fp32_to_bf16_bits, fp32_to_f16_bits, reduce_scatter_share

from test_oracle_closed_forms import build_example, load_worked_examples


def _fold(xs, ss, xf, sl, out, *, order=None, start_zero=False, wide=False, pairwise=False, group=None,
          to_bf16=fp32_to_bf16_bits, to_f16=fp32_to_f16_bits, scale_col=None, unsigned=False):
    """A configurable re-statement of the definition used only to plant mistakes."""
    g = group or GROUP_SIZE[sl]
    xt = decode_table(xf)
    if unsigned:
        xt = np.abs(xt)
    st = scale_decode_table()
    ps = []
    for x, s in zip(xs, ss):
        sv = s if sl == "f32_group128" else st[s]
        if scale_col is not None:  # planted: a wrong column -> group map
            cols = np.arange(x.shape[1])
            sv = sv[:, scale_col(cols, GROUP_SIZE[sl], sv.shape[1])]
        else:
            sv = np.repeat(sv, g, axis=1)[:, : x.shape[1]]
        if sv.shape[1] < x.shape[1]:
            sv = np.tile(sv, (1, x.shape[1] // sv.shape[1] + 1))[:, : x.shape[1]]
        with np.errstate(over="ignore", invalid="ignore"):
            if wide:
                ps.append(xt[x].astype(np.float64) * sv.astype(np.float64))
            else:
                ps.append((xt[x] * sv).astype(np.float32))
    if order is not None:
        ps = [ps[i] for i in order(len(ps))]
    if pairwise:
        while len(ps) > 1:
            ps = [ps[i] + ps[i + 1] if i + 1 < len(ps) else ps[i] for i in range(0, len(ps), 2)]
        acc = ps[0]
    else:
        acc = np.zeros_like(ps[0]) if start_zero else ps[0]
        for p in (ps if start_zero else ps[1:]):
            acc = acc + p
    acc = acc.astype(np.float32)
    if out == "f32":
        return acc
    return to_f16(acc) if out == "f16" else to_bf16(acc)


def _truncate_bf16(acc):
    return (np.ascontiguousarray(acc).view(np.uint32) >> 16).astype(np.uint16)


def _f16_toward_zero(acc):
    """binary16 by truncation toward zero (a plausible wrong rounding)."""
    a = np.ascontiguousarray(acc, dtype=np.float32).astype(np.float64)
    _, e2 = np.frexp(np.abs(a))
    q = np.ldexp(1.0, np.maximum(e2 - 1, -14) - 10)
    r = np.minimum(np.trunc(np.abs(a) / q) * q, 65504.0)
    return (np.copysign(r, a).astype(np.float16)).view(np.uint16)


def _worked_examples_pass(fn):
    for ex in load_worked_examples():
        xs, ss = build_example(ex)
        out = fn(xs, ss, ex["x_format"], ex["scale_layout"], ex["out_dtype"])
        got = out.view(np.uint32) if ex["out_dtype"] == "f32" else out
        if not np.all(got == int(ex["expected_bits"], 16)):
            return False
    return True


def _cross_layout_passes(fn):
    rng = np.random.default_rng(3)
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=8 * 2, h=1024)
    # The reference side must itself be the unmutated definition.
    xs, _ = workloads.generate(wl)
    codes128 = [rng.integers(110, 145, size=(wl.rows, wl.h // 128), dtype=np.uint8) for _ in range(8)]
    mx = [np.repeat(c, 4, axis=1) for c in codes128]
    f32 = [np.ldexp(np.float32(1.0), c.astype(np.int32) - 127).astype(np.float32) for c in codes128]
    a = fn(xs, mx, "e4m3fn", "e8m0_block32", "f32")
    b = fn(xs, f32, "e4m3fn", "f32_group128", "f32")
    ref = reduce_scatter_share(xs, f32, "e4m3fn", "f32_group128", "f32")
    return np.array_equal(a.view(np.uint32), b.view(np.uint32)) and np.array_equal(b.view(np.uint32), ref.view(np.uint32))


def _decode_pin_passes(table_fn, fmt, tdt):
    want = torch.arange(256, dtype=torch.uint8).view(tdt).float().numpy()
    got = table_fn(fmt)
    ok = ~np.isnan(want)
    return np.array_equal(np.isnan(got), ~ok) and np.array_equal(got[ok], want[ok])


MUTANTS = {
    "reverse_rank_order": dict(order=lambda n: list(range(n))[::-1]),
    "pairwise_tree_sum": dict(pairwise=True),
    "fp64_accumulate_like_fma": dict(wide=True),
    "accumulator_starts_at_plus_zero": dict(start_zero=True),
    "bf16_by_truncation": dict(to_bf16=_truncate_bf16),
    "f16_toward_zero": dict(to_f16=_f16_toward_zero),
    "group_of_64_columns": dict(group=64),
    "scale_of_the_next_group": dict(scale_col=lambda c, g, n: np.minimum(c // g + 1, n - 1)),
    "scales_indexed_by_column_modulo": dict(scale_col=lambda c, g, n: c % n),
    "sign_of_x_dropped": dict(unsigned=True),
}


def test_unmutated_restatement_passes():
    fn = lambda *a: _fold(*a)  # noqa: E731
    assert _worked_examples_pass(fn)
    assert _cross_layout_passes(fn)
    assert _worked_examples_pass(reduce_scatter_share)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    kw = MUTANTS[name]
    fn = lambda *a: _fold(*a, **kw)  # noqa: E731
    caught = (not _worked_examples_pass(fn)) or (not _cross_layout_passes(fn))
    assert caught, f"no pin rejects the planted mistake {name}"


def test_planted_decode_mistakes_are_caught():
    def e5m2_bias16(fmt):
        t = decode_table(fmt).astype(np.float64)
        return np.where(np.isfinite(t), t / 2, t).astype(np.float32)

    def e4m3_no_subnormals(fmt):
        t = decode_table(fmt).copy()
        t[1:8] = 0.0
        t[0x81:0x88] = -0.0
        return t

    def int8_unsigned(fmt):
        return np.arange(256, dtype=np.float32)

    assert _decode_pin_passes(decode_table, "e5m2", torch.float8_e5m2)
    assert not _decode_pin_passes(e5m2_bias16, "e5m2", torch.float8_e5m2)
    assert not _decode_pin_passes(e4m3_no_subnormals, "e4m3fn", torch.float8_e4m3fn)
    assert not _decode_pin_passes(int8_unsigned, "int8", torch.int8)


ORDER_MUTANTS = ("reverse_rank_order", "pairwise_tree_sum")


def test_other_orders_stated_by_the_examples():
    """The bits each fold-order example states for the other orders are what
    those orders compute."""
    checked = 0
    for ex in load_worked_examples():
        for name, bits in ex.get("other_orders", {}).items():
            xs, ss = build_example(ex)
            out = _fold(xs, ss, ex["x_format"], ex["scale_layout"], ex["out_dtype"], **MUTANTS[name])
            got = out.view(np.uint32) if ex["out_dtype"] == "f32" else out
            assert np.all(got == int(bits, 16)), (ex["name"], name, hex(int(got.ravel()[0])))
            checked += 1
    assert checked >= 6


@pytest.mark.parametrize("name", ORDER_MUTANTS)
def test_each_order_mutant_is_rejected_by_two_examples(name):
    rejected = []
    for ex in load_worked_examples():
        xs, ss = build_example(ex)
        out = _fold(xs, ss, ex["x_format"], ex["scale_layout"], ex["out_dtype"], **MUTANTS[name])
        got = out.view(np.uint32) if ex["out_dtype"] == "f32" else out
        if not np.all(got == int(ex["expected_bits"], 16)):
            rejected.append(ex["name"])
    assert len(rejected) >= 2, (name, rejected)
