"""qrs_plan against a plain statement of its constraints (page
"aclnnQuantReduceScatter", Constraints: communicator size 2, 4 or 8; H a
multiple of 128 in [1024, 8192]; BS positive and split evenly over the ranks;
the MX mode only with FP8 x; HIFLOAT8 named but undefined), on random
argument tuples. Host-only: no device is touched."""

import ctypes

from hypothesis import given, settings
from hypothesis import strategies as st

import quantized_collective_reduction_amd as qrs

X = {0: "int8", 1: "e4m3fn", 2: "e5m2", 3: "hifloat8"}
OK, INVALID, UNSUPPORTED = 0, 1, 2


def expected(w, bs, h, x, sl, out):
    if w not in (2, 4, 8):
        return INVALID
    if bs <= 0 or bs % w:
        return INVALID
    if not (1024 <= h <= 8192 and h % 128 == 0):
        return INVALID
    if (bs // w) > (1 << 40) // h:
        return INVALID
    if x == 3:
        return UNSUPPORTED
    if x not in (0, 1, 2) or sl not in (0, 1):
        return INVALID
    if sl == 1 and x == 0:
        return INVALID
    if out not in (0, 1, 2):
        return INVALID
    return OK


@settings(max_examples=3000, deadline=None)
@given(w=st.sampled_from([-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 16]),
       bs=st.one_of(st.integers(-8, 64), st.integers(1, 1 << 45)),
       h=st.one_of(st.sampled_from([0, 128, 896, 1000, 1024, 1152, 5120, 8064, 8192, 8320, 16384]),
                   st.integers(-10, 20000)),
       x=st.integers(-1, 4), sl=st.integers(-1, 2), out=st.integers(-1, 3))
def test_plan_matches_constraints(w, bs, h, x, sl, out):
    lib = qrs.load_library()
    handle = ctypes.c_void_p()
    ws = ctypes.c_size_t(12345)
    status = lib.qrs_plan(w, bs, h, x, sl, out, ctypes.byref(handle), ctypes.byref(ws))
    want = expected(w, bs, h, x, sl, out)
    assert status == want, (w, bs, h, x, sl, out, lib.qrs_last_error().decode())
    if status == OK:
        assert handle.value and ws.value == 0
        rows, hh = ctypes.c_int64(), ctypes.c_int64()
        assert lib.qrs_plan_shape(handle, ctypes.byref(rows), ctypes.byref(hh)) == OK
        assert rows.value == bs // w and hh.value == h
        assert lib.qrs_plan_destroy(handle) == OK
    else:
        assert not handle.value
        assert lib.qrs_last_error().decode() != ""


# qrs_run_strided's host checks, on fake device addresses far apart (so the
# address spans never overlap). Runs only where no GPU is visible: arguments
# the host accepts then fail at the launch (QRS_ERR_HIP), rejected ones return
# QRS_ERR_INVALID_ARG without reaching it.
import pytest  # noqa: E402

GiB4 = 1 << 32


def strided_expected(rows, h, g, sb, ob, x, s, o):
    if x < h or x % 16 or s < h // g or o < h:
        return INVALID
    lim = 1 << 48
    if x > lim // rows or s > lim // rows // sb or o > lim // rows // ob:
        return INVALID
    if rows >= GiB4 or x >= GiB4 or s * sb >= GiB4 or o * ob >= GiB4:
        return INVALID
    if (o * ob) % 16:
        return INVALID
    if ((rows - 1) * s + h // g) * sb >= GiB4:
        return INVALID
    return 3  # QRS_ERR_HIP: accepted, and the launch fails without a device


@pytest.fixture(scope="module")
def no_gpu_lib():
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-address checks run only without a GPU")
    return qrs.load_library()


STRIDE = st.one_of(st.integers(-(1 << 63), (1 << 63) - 1), st.integers(-64, 20000),
                   st.integers(0, 1 << 34).map(lambda v: v // 16 * 16), st.sampled_from([0, 1, 16, 1024, 1 << 32, (1 << 32) - 16]))


@settings(max_examples=2000, deadline=None)
@given(rows=st.sampled_from([1, 2, 7, 4096, 1 << 20]), h=st.sampled_from([1024, 1152, 8192]),
       mode=st.sampled_from([(1, 0), (1, 1)]), out=st.sampled_from([0, 1, 2]), x=STRIDE, s=STRIDE, o=STRIDE)
def test_strided_checks_match_constraints(no_gpu_lib, rows, h, mode, out, x, s, o):
    lib = no_gpu_lib
    xd, sl = mode
    p = qrs.plan(2, 2 * rows, h, X[xd], "f32_group128" if sl == 0 else "e8m0_block32",
                 {0: "f32", 1: "bf16", 2: "f16"}[out])
    g, sb = (128, 4) if sl == 0 else (32, 1)
    ob = 4 if out == 0 else 2
    base, step = 1 << 52, 1 << 50
    xs = (ctypes.c_void_p * 2)(base, base + step)
    ss = (ctypes.c_void_p * 2)(base + 2 * step, base + 3 * step)
    status = lib.qrs_run_strided(p.handle, xs, x, ss, s, base + 4 * step, o, None, 0, None)
    assert status == strided_expected(rows, h, g, sb, ob, x, s, o), (rows, h, mode, out, x, s, o,
                                                                     lib.qrs_last_error().decode())
