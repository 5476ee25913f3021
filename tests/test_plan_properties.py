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
