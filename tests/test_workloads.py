"""The synthetic input generator: determinism, shapes, value ranges, and that
it still produces the inputs the stored digests were made from."""

import json
import os

import numpy as np
import pytest

import workloads
from oracle.decode import decode_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "digests.json")


def _small(name):
    wl = workloads.WORKLOADS[name]
    return wl.with_(bs=wl.world_size * 8)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_deterministic_and_shaped(name):
    wl = _small(name)
    xs, ss = workloads.generate(wl)
    xs2, ss2 = workloads.generate(wl)
    assert len(xs) == len(ss) == wl.world_size
    for a, b in zip(xs + ss, xs2 + ss2):
        assert np.array_equal(a, b)
    for x, s in zip(xs, ss):
        assert x.dtype == np.uint8 and x.shape == (wl.rows, wl.h)
        assert s.shape == (wl.rows, wl.h // wl.group)
        assert s.dtype == (np.float32 if wl.scale_layout == "f32_group128" else np.uint8)
    # Different seeds give different data; ranks differ from each other.
    xs3, _ = workloads.generate(wl.with_(seed=1))
    assert not np.array_equal(xs[0], xs3[0])
    assert not np.array_equal(xs[0], xs[1])


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_value_ranges(name):
    wl = _small(name)
    xs, ss = workloads.generate(wl)
    table = decode_table(wl.x_format)
    for x, s in zip(xs, ss):
        v = table[x]
        assert np.all(np.isfinite(v)), "no NaN or infinity codes in the workloads"
        if wl.x_format == "int8":
            assert v.min() >= -127 and v.max() <= 127
        if wl.scale_layout == "f32_group128":
            assert np.all(s >= np.float32(2.0 ** wl.scale_lo)) and np.all(s <= np.float32(2.0 ** wl.scale_hi))
        else:
            assert s.min() >= wl.scale_lo and s.max() <= wl.scale_hi
    # The float8 draws are spread over many codes, including both signs.
    allx = np.concatenate([x.ravel() for x in xs])
    assert len(np.unique(allx)) > 64


def test_algorithmic_bytes_match_the_size_formulas():
    # x: BS*H bytes over all ranks' slices; scales: BS*H/128*4 or BS*H/32*1.
    c4 = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"]
    assert c4.algorithmic_bytes() == 16384 * 8192 + 16384 * 8192 // 32 + 2048 * 8192 * 2 == 171_966_464
    c5 = workloads.WORKLOADS["w8_bs65536_h5120_mx_e5m2_f32"]
    assert c5.algorithmic_bytes() == 65536 * 5120 + 65536 * 5120 // 32 + 8192 * 5120 * 4 == 513_802_240
    c2 = workloads.WORKLOADS["w4_bs4096_h4096_e4m3_bf16"]
    assert c2.algorithmic_bytes() == 4096 * 4096 + 4096 * 4096 // 128 * 4 + 1024 * 4096 * 2


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_inputs_match_stored_digests(name):
    import sys

    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    from make_digests import input_digest

    with open(GOLDEN) as f:
        want = json.load(f)["configs"][name]["inputs_sha256"]
    xs, ss = workloads.generate(workloads.WORKLOADS[name])
    assert input_digest(xs, ss) == want
