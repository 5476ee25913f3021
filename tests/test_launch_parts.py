"""How a share is split into launches, on the host (no kernel runs): a HIP
grid holds fewer than 2^32 work-items along a dimension, so a share of more
than 2^34 elements runs as launches of at most 2^34 elements each, and
QRS_MAX_LAUNCH_ELEMS may lower that bound. qrs_run_launch_info reports the
launch count and the first launch's grid (with no stream and no GPU it reads
no device sizes and reports no residency cap)."""

import ctypes
import os
import subprocess
import sys

import pytest

import quantized_collective_reduction_amd as qrs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _info(lib, w, bs, h, xd="e4m3fn", sl="e8m0_block32", od="bf16"):
    p = qrs.plan(w, bs, h, xd, sl, od)
    info = qrs.LaunchInfo()
    assert lib.qrs_run_launch_info(p.handle, None, ctypes.byref(info)) == qrs.Status.OK
    return info.as_dict()


@pytest.fixture(scope="module")
def lib():
    if os.environ.get("QRS_MAX_LAUNCH_ELEMS"):
        pytest.skip("QRS_MAX_LAUNCH_ELEMS is set in this process")
    return qrs.load_library()


@pytest.mark.parametrize("w,rows,h,xd,sl,od,launches", [
    (8, 2048, 8192, "e4m3fn", "e8m0_block32", "bf16", 1),
    (2, 1 << 21, 8192, "e4m3fn", "e8m0_block32", "bf16", 1),        # exactly 2^34 elements
    (2, (1 << 21) + 64, 8192, "e4m3fn", "e8m0_block32", "f16", 2),  # 2^34 + 2^19
    (2, 1 << 22, 8192, "e5m2", "e8m0_block32", "bf16", 2),          # 2^35: one launch would hold 2^32 lanes of 8
    (2, 1 << 27, 8192, "int8", "f32_group128", "f32", 64),          # 2^40, the largest plan
    (4, 7 * (1 << 20) + 3, 5120, "e5m2", "f32_group128", "bf16", 3),
])
def test_launch_count_and_grid_bound(lib, w, rows, h, xd, sl, od, launches):
    info = _info(lib, w, w * rows, h, xd, sl, od)
    assert info["launches"] == launches == -(-rows * h // (1 << 34))
    assert info["threads_per_block"] == 256
    assert info["blocks"] * info["threads_per_block"] <= 1 << 31  # HIP's bound is 2^32 - 1
    if launches > 1:
        # the first launch covers 2^34 elements: 8 per lane, or 16 for chunks
        assert info["blocks"] * 256 in ((1 << 34) // 8, (1 << 34) // 16)


def test_plans_past_2_to_40_elements_are_rejected(lib):
    with pytest.raises(qrs.QrsError):
        qrs.plan(2, 2 * ((1 << 27) + 1), 8192, "int8", "f32_group128", "f32")


CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import quantized_collective_reduction_amd as qrs
lib = qrs.load_library()
p = qrs.plan(8, 8 * 37, 1152, "e4m3fn", "e8m0_block32", "bf16")
info = qrs.LaunchInfo()
st = lib.qrs_run_launch_info(p.handle, None, ctypes.byref(info))
print(st, info.launches, info.blocks, lib.qrs_last_error().decode())
"""


def _child(value):
    env = dict(os.environ)
    env.pop("QRS_MAX_LAUNCH_ELEMS", None)
    if value is not None:
        env["QRS_MAX_LAUNCH_ELEMS"] = value
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], env=env, capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    st, launches, blocks, msg = r.stdout.strip().split(" ", 3) + [""] * (4 - len(r.stdout.strip().split(" ", 3)))
    return int(st), int(launches), int(blocks), msg


def test_launch_bound_from_the_environment():
    # 37 rows of 1152 = 42,624 elements
    assert _child(None)[:2] == (qrs.Status.OK, 1)
    assert _child("")[:2] == (qrs.Status.OK, 1)
    st, launches, blocks, _ = _child("4096")
    assert (st, launches) == (qrs.Status.OK, 11)
    assert blocks == 4096 // 8 // 256  # the first launch: 4096 elements in 8-element pieces
    assert _child("12288")[:2] == (qrs.Status.OK, 4)
    assert _child(str(1 << 34))[:2] == (qrs.Status.OK, 1)


@pytest.mark.parametrize("value", ["4095", "6000", "0", "-4096", "+4096", " 4096", "4096x", "1e6", "abc",
                                   str((1 << 34) + 4096), "99999999999999999999999"])
def test_bad_launch_bound_fails_every_launching_call(value):
    st, _, _, msg = _child(value)
    assert st == qrs.Status.INVALID_ARG
    assert "QRS_MAX_LAUNCH_ELEMS" in msg
