"""The C-ABI boundary on the host: the library loads, exports every function
include/qrs.h declares, and rejects invalid problems before any GPU work.
No compute call is made here (no GPU needed)."""

import ctypes
import os
import re

import pytest

import quantized_collective_reduction_amd as qrs

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qrs.h")


@pytest.fixture(scope="module")
def lib():
    return qrs.load_library()


@pytest.fixture(scope="module")
def fake_ptr_lib(lib):
    """For tests that hand fake device addresses to calls expected to fail
    their host checks: run them only where no GPU is visible, so a missing
    check could never launch a kernel on such an address."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-address checks run only without a GPU")
    return lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qrs_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    declared = _declared_functions()
    assert declared == sorted(qrs.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in qrs.Status:
        assert lib.qrs_status_string(int(s)).decode() == f"QRS_{'OK' if s == 0 else 'ERR_' + s.name}"
    assert lib.qrs_status_string(99).decode() == "QRS_ERR_UNKNOWN"


VALID_MODES = [
    ("int8", "f32_group128"),
    ("e4m3fn", "f32_group128"),
    ("e5m2", "f32_group128"),
    ("e4m3fn", "e8m0_block32"),
    ("e5m2", "e8m0_block32"),
]


@pytest.mark.parametrize("x,s", VALID_MODES)
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("w", [2, 4, 8])
def test_valid_plans(lib, x, s, out, w):
    p = qrs.plan(w, 16 * w, 1024, x, s, out)
    assert p.rows == 16 and p.workspace_bytes == 0


@pytest.mark.parametrize("h", [1024, 1152, 4096, 5120, 7168, 8192])
def test_accepted_h(lib, h):
    assert qrs.plan(2, 2, h, "e4m3fn", "e8m0_block32", "bf16").rows == 1


@pytest.mark.parametrize(
    "args,status",
    [
        ((0, 16, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((1, 16, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((3, 18, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((5, 20, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((16, 32, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1000, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 896, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 8320, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1088, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 0, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, -2, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((4, 18, 1024, "int8", "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1024, "int8", "e8m0_block32", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1024, "hifloat8", "f32_group128", "f32"), qrs.Status.UNSUPPORTED),
        ((2, 16, 1024, 7, "f32_group128", "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1024, "int8", 5, "f32"), qrs.Status.INVALID_ARG),
        ((2, 16, 1024, "int8", "f32_group128", 9), qrs.Status.INVALID_ARG),
    ],
)
def test_rejected_plans(lib, args, status):
    with pytest.raises(qrs.QrsError) as ei:
        qrs.plan(*args)
    assert ei.value.status == status
    assert str(ei.value)


def test_null_out_params(lib):
    ws = ctypes.c_size_t()
    h = ctypes.c_void_p(1234)
    assert lib.qrs_plan(2, 16, 1024, 0, 0, 0, None, ctypes.byref(ws)) == qrs.Status.INVALID_ARG
    assert lib.qrs_plan(2, 16, 1024, 0, 0, 0, ctypes.byref(h), None) == qrs.Status.INVALID_ARG
    assert h.value is None  # cleared on error
    assert b"non-null" in lib.qrs_last_error()


def test_destroy_null_and_shape_of_null(lib):
    assert lib.qrs_plan_destroy(None) == qrs.Status.OK
    assert lib.qrs_plan_shape(None, None, None) == qrs.Status.INVALID_ARG


def test_launch_info_rejects_null_arguments(lib):
    info = qrs.LaunchInfo()
    assert lib.qrs_run_launch_info(None, None, ctypes.byref(info)) == qrs.Status.INVALID_ARG
    p = qrs.plan(8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16")
    assert lib.qrs_run_launch_info(p.handle, None, None) == qrs.Status.INVALID_ARG


# qrs_run checks its arguments on the host before it touches the GPU; these
# calls return before any HIP call.


def _run_raw(lib, p, xs, ss, out):
    w = len(xs)
    xa = (ctypes.c_void_p * w)(*xs)
    sa = (ctypes.c_void_p * w)(*ss)
    return lib.qrs_run(p.handle if p else None, xa, sa, out, None, 0, None)


def test_run_rejects_bad_pointers_on_host(fake_ptr_lib):
    lib = fake_ptr_lib
    p = qrs.plan(2, 32, 1024, "e4m3fn", "f32_group128", "f32")
    n = p.rows * p.h
    A = 1 << 40  # fake, never dereferenced: every call below fails its host checks
    good_x = [A, A + (1 << 30)]
    good_s = [A + (2 << 30), A + (3 << 30)]
    out = A + (4 << 30)
    assert _run_raw(lib, None, good_x, good_s, out) == qrs.Status.INVALID_ARG
    assert lib.qrs_run(p.handle, None, None, out, None, 0, None) == qrs.Status.INVALID_ARG
    assert _run_raw(lib, p, good_x, good_s, 0) == qrs.Status.INVALID_ARG
    assert _run_raw(lib, p, [A, 0], good_s, out) == qrs.Status.INVALID_ARG
    assert _run_raw(lib, p, [A + 8, good_x[1]], good_s, out) == qrs.Status.INVALID_ARG  # x misaligned
    assert _run_raw(lib, p, good_x, [good_s[0] + 2, good_s[1]], out) == qrs.Status.INVALID_ARG  # fp32 scale
    assert _run_raw(lib, p, good_x, good_s, out + 4) == qrs.Status.INVALID_ARG  # out misaligned
    # out overlapping an x slice or a scale slice
    assert _run_raw(lib, p, good_x, good_s, good_x[1] + n - 16) == qrs.Status.INVALID_ARG
    assert _run_raw(lib, p, good_x, good_s, good_s[0] - 16) == qrs.Status.INVALID_ARG
    assert b"overlaps" in lib.qrs_last_error()


def _create_raw(lib, p, xs, ss, out, handle):
    w = len(xs)
    xa = (ctypes.c_void_p * w)(*xs)
    sa = (ctypes.c_void_p * w)(*ss)
    return lib.qrs_launch_create(p.handle if p else None, xa, sa, out, None, handle)


def test_prepared_launch_rejects_what_run_rejects_on_host(fake_ptr_lib):
    # qrs_launch_create makes qrs_run's checks before it touches the GPU
    # (these calls return before any HIP call) and leaves the handle NULL.
    lib = fake_ptr_lib
    p = qrs.plan(2, 32, 1024, "e4m3fn", "f32_group128", "f32")
    n = p.rows * p.h
    A = 1 << 40  # fake, never dereferenced
    good_x = [A, A + (1 << 30)]
    good_s = [A + (2 << 30), A + (3 << 30)]
    out = A + (4 << 30)
    h = ctypes.c_void_p(12345)
    cases = [
        (None, good_x, good_s, out),
        (p, good_x, good_s, 0),
        (p, [A, 0], good_s, out),
        (p, [A + 8, good_x[1]], good_s, out),
        (p, good_x, [good_s[0] + 2, good_s[1]], out),
        (p, good_x, good_s, out + 4),
        (p, good_x, good_s, good_x[1] + n - 16),
    ]
    for case in cases:
        h.value = 12345
        assert _create_raw(lib, *case, ctypes.byref(h)) == qrs.Status.INVALID_ARG
        assert not h.value
    assert _create_raw(lib, p, good_x, good_s, out, None) == qrs.Status.INVALID_ARG  # no handle pointer
    assert lib.qrs_launch_enqueue(None) == qrs.Status.INVALID_ARG
    assert lib.qrs_launch_destroy(None) == qrs.Status.OK


def test_stream_copy_rejects_bad_arguments_on_host(fake_ptr_lib):
    lib = fake_ptr_lib
    A = 1 << 40
    assert lib.qrs_stream_copy(None, A, 16, None) == qrs.Status.INVALID_ARG
    assert lib.qrs_stream_copy(A, A + 4096, 0, None) == qrs.Status.INVALID_ARG
    assert lib.qrs_stream_copy(A, A + 4096, 24, None) == qrs.Status.INVALID_ARG
    assert lib.qrs_stream_copy(A + 8, A + 4096, 16, None) == qrs.Status.INVALID_ARG
    assert lib.qrs_stream_copy(A, A + 16, 32, None) == qrs.Status.INVALID_ARG


def test_binding_rejects_host_tensors_and_wrong_sizes(lib):
    import torch

    p = qrs.plan(2, 32, 1024, "e4m3fn", "f32_group128", "f32")
    x = [torch.zeros(16, 1024, dtype=torch.uint8) for _ in range(2)]
    s = [torch.zeros(16, 8, dtype=torch.float32) for _ in range(2)]
    out = torch.zeros(16, 1024, dtype=torch.float32)
    with pytest.raises(ValueError):
        qrs.run(p, x, s, out)  # CPU tensors: no CPU path
    with pytest.raises(ValueError):
        qrs.run(p, x[:1], s, out)
    with pytest.raises(ValueError):
        qrs.run(p, x, [torch.zeros(16, 4, dtype=torch.float32)] * 2, out)


def test_prepared_launch_checks_arguments_on_host(lib):
    import torch

    p = qrs.plan(2, 32, 1024, "e4m3fn", "e8m0_block32", "bf16")
    x = [torch.zeros(16, 1024, dtype=torch.uint8) for _ in range(2)]
    s = [torch.zeros(16, 32, dtype=torch.uint8) for _ in range(2)]
    out = torch.zeros(16, 1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qrs.Launch(p, x, s, out)  # CPU tensors
    with pytest.raises(ValueError):
        qrs.Launch(p, x, s, torch.zeros(16, 1024, dtype=torch.float32))  # wrong output size


def test_binding_rejects_floating_dtypes_other_than_the_modes():
    """Typed tensors must carry the element types the mode names (integer
    tensors are raw bytes). The dtype check runs before any pointer is taken,
    so host tensors reach it."""
    import torch

    p = qrs.plan(2, 32, 1024, "e4m3fn", "e8m0_block32", "bf16")
    x = [torch.zeros(16, 1024, dtype=torch.uint8) for _ in range(2)]
    s = [torch.zeros(16, 32, dtype=torch.uint8) for _ in range(2)]
    for bad_out in (torch.zeros(16, 1024, dtype=torch.float16), torch.zeros(16, 512, dtype=torch.float32)):
        with pytest.raises(ValueError, match="does not match"):
            qrs.run(p, x, s, bad_out)
        with pytest.raises(ValueError, match="does not match"):
            qrs.Launch(p, x, s, bad_out)
    out = torch.zeros(16, 1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x slice 1"):
        qrs.run(p, [x[0], torch.zeros(16, 1024, dtype=torch.float8_e5m2)], s, out)
    with pytest.raises(ValueError, match="scale slice 0"):
        qrs.run(p, x, [torch.zeros(16, 32, dtype=torch.float8_e4m3fn), s[1]], out)
    # Matching float8 and E8M0 dtypes pass the dtype check and fail only at the host-tensor check.
    with pytest.raises(ValueError, match="device tensors only"):
        qrs.run(p, [t.view(torch.float8_e4m3fn) for t in x], [t.view(torch.float8_e8m0fnu) for t in s], out)

    pg = qrs.plan(2, 32, 1024, "e5m2", "f32_group128", "f32")
    xg = [torch.zeros(32, 1024, dtype=torch.uint8) for _ in range(2)]
    sg = [torch.zeros(32, 8, dtype=torch.float32) for _ in range(2)]
    outs = [torch.zeros(16, 512, dtype=torch.bfloat16), torch.zeros(16, 1024, dtype=torch.float32)]
    with pytest.raises(ValueError, match="output of share 0"):
        qrs.run_all_shares(pg, xg, sg, outs)
    with pytest.raises(ValueError, match="scales of rank 1"):
        qrs.AllSharesLaunch(pg, xg, [sg[0], torch.zeros(32, 4, dtype=torch.float64)], [outs[1], outs[1]])

    xb = torch.zeros(16, 1024, dtype=torch.float16)
    with pytest.raises(ValueError, match="x_bf16"):
        qrs.quantize(xb, torch.zeros(16, 1024, dtype=torch.uint8), torch.zeros(16, 32, dtype=torch.uint8),
                     "e4m3fn", "e8m0_block32")
    with pytest.raises(ValueError, match="x_codes"):
        qrs.QuantizeLaunch(xb.view(torch.bfloat16), torch.zeros(16, 1024, dtype=torch.float8_e5m2),
                           torch.zeros(16, 32, dtype=torch.uint8), "e4m3fn", "e8m0_block32")
    with pytest.raises(ValueError, match="unknown XDtype"):
        qrs.plan(2, 32, 1024, "fp8", "f32_group128", "f32")


def test_strided_run_rejects_bad_strides_on_host(fake_ptr_lib):
    lib = fake_ptr_lib
    p = qrs.plan(2, 32, 1024, "e4m3fn", "e8m0_block32", "f32")
    A = 1 << 40
    xs = (ctypes.c_void_p * 2)(A, A + (1 << 30))
    ss = (ctypes.c_void_p * 2)(A + (2 << 30), A + (3 << 30))
    out = A + (4 << 30)

    def call(ldx, lds, ldo, o=out):
        return lib.qrs_run_strided(p.handle, xs, ldx, ss, lds, o, ldo, None, 0, None)

    assert call(1000, 32, 1024) == qrs.Status.INVALID_ARG  # x stride < h
    assert call(1032, 32, 1024) == qrs.Status.INVALID_ARG  # not a multiple of 16
    assert call(1024, 31, 1024) == qrs.Status.INVALID_ARG  # scale stride < h/32
    assert call(1024, 32, 1020) == qrs.Status.INVALID_ARG  # out stride < h
    assert call(1024, 32, 1026) == qrs.Status.INVALID_ARG  # 1026 * 4 bytes is not a multiple of 16
    assert call(1024, 32, 1024, o=out + 4) == qrs.Status.INVALID_ARG  # misaligned out
    # out span overlapping the last row of rank 1's x slice
    assert call(4096, 32, 1024, o=A + (1 << 30) + 15 * 4096) == qrs.Status.INVALID_ARG


def test_slice_pitch(lib):
    p = qrs.plan(8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16")
    xp, sp = qrs.slice_pitch(p)
    assert xp == 16 * 2**20 + 1280 * 1024 and sp == 2048 * 8192 // 32 + 40 * 1024
    xp, sp = qrs.slice_pitch(p, full_inputs=True)
    assert xp == 16384 * 8192 + 1280 * 1024
    p2 = qrs.plan(2, 6, 1152, "int8", "f32_group128", "f32")  # 3 rows: 3456 bytes per slice
    xp, sp = qrs.slice_pitch(p2)
    assert xp == 1280 * 1024 and sp == 4096 + 40 * 1024  # 64 KiB, then staggered to 1.25 MiB
    # Slices that are not a multiple of 4 MiB get the stagger that makes the
    # pitch 1.25 MiB modulo 4 MiB: 7 MiB slices -> 9.25 MiB, 15 MiB -> 17.25.
    p3 = qrs.plan(8, 8192, 7168, "e5m2", "f32_group128", "bf16")
    assert qrs.slice_pitch(p3)[0] == (9 << 20) + (1 << 18)
    p4 = qrs.plan(8, 24576, 5120, "e5m2", "e8m0_block32", "f32")
    assert qrs.slice_pitch(p4)[0] == (17 << 20) + (1 << 18)
    for bs, h in [(8, 1024), (16384, 1152), (65536, 5120), (12345 * 8, 1024)]:
        xp = qrs.slice_pitch(qrs.plan(8, bs, h, "e4m3fn", "e8m0_block32", "bf16"))[0]
        assert xp >= bs // 8 * h and xp % 65536 == 0 and xp % (4 << 20) == 1280 * 1024
    assert lib.qrs_slice_pitch(None, 0, None, None) == qrs.Status.INVALID_ARG
    assert lib.qrs_slice_pitch(p.handle, 2, None, None) == qrs.Status.INVALID_ARG


def test_quantize_rejects_bad_arguments_on_host(fake_ptr_lib):
    lib = fake_ptr_lib
    A = 1 << 40
    x, c, s = A, A + (1 << 30), A + (2 << 30)

    def q(tokens=16, h=1024, xd=1, sl=1, xp=x, cp=c, sp=s):
        return lib.qrs_quantize(tokens, h, xd, sl, xp, cp, sp, None)

    assert q(tokens=0) == qrs.Status.INVALID_ARG
    assert q(tokens=-3) == qrs.Status.INVALID_ARG
    assert q(h=1000) == qrs.Status.INVALID_ARG
    assert q(h=9216) == qrs.Status.INVALID_ARG
    assert q(xd=3) == qrs.Status.UNSUPPORTED  # HIFLOAT8
    assert q(xd=0, sl=1) == qrs.Status.INVALID_ARG  # INT8 with E8M0
    assert q(xd=9) == qrs.Status.INVALID_ARG
    assert q(sl=4) == qrs.Status.INVALID_ARG
    assert q(xp=0) == qrs.Status.INVALID_ARG
    assert q(xp=x + 8) == qrs.Status.INVALID_ARG  # input misaligned
    assert q(cp=c + 8) == qrs.Status.INVALID_ARG  # codes misaligned
    assert q(sl=0, xd=1, sp=s + 2) == qrs.Status.INVALID_ARG  # fp32 scales misaligned
    assert q(cp=x + 1024) == qrs.Status.INVALID_ARG  # codes overlap the input
    assert q(sp=c + 100) == qrs.Status.INVALID_ARG  # scales overlap the codes
    assert b"overlap" in lib.qrs_last_error()


def test_all_shares_rejects_bad_arguments_on_host(fake_ptr_lib):
    lib = fake_ptr_lib
    p = qrs.plan(2, 32, 1024, "e4m3fn", "f32_group128", "bf16")
    A = 1 << 40
    G = 1 << 30
    xs = (ctypes.c_void_p * 2)(A, A + G)
    ss = (ctypes.c_void_p * 2)(A + 2 * G, A + 3 * G)

    def run(o0, o1, x=xs, s=ss):
        outs = (ctypes.c_void_p * 2)(o0, o1)
        return lib.qrs_run_all_shares(p.handle, x, s, outs, None, 0, None)

    assert lib.qrs_run_all_shares(None, xs, ss, (ctypes.c_void_p * 2)(A + 4 * G, A + 5 * G), None, 0, None) \
        == qrs.Status.INVALID_ARG
    assert run(A + 4 * G, 0) == qrs.Status.INVALID_ARG  # null output
    assert run(A + 4 * G, A + 4 * G + 16) == qrs.Status.INVALID_ARG  # outputs overlap
    assert run(A + 4 * G + 4, A + 5 * G) == qrs.Status.INVALID_ARG  # misaligned output
    assert run(A + 32 * 1024 - 16, A + 5 * G) == qrs.Status.INVALID_ARG  # output overlaps rank 0's x
    bad_x = (ctypes.c_void_p * 2)(A + 8, A + G)
    assert run(A + 4 * G, A + 5 * G, x=bad_x) == qrs.Status.INVALID_ARG  # misaligned x
    bad_s = (ctypes.c_void_p * 2)(A + 2 * G + 2, A + 3 * G)
    assert run(A + 4 * G, A + 5 * G, s=bad_s) == qrs.Status.INVALID_ARG  # misaligned fp32 scales


def test_header_compiles_as_c99_and_cxx(tmp_path):
    """include/qrs.h is a plain C header: it compiles as C99 and as C++,
    and a C caller can reference every declared entry point."""
    import shutil
    import subprocess

    decls = _declared_functions()
    src = tmp_path / "use.c"
    src.write_text('#include "qrs.h"\n' + "typedef void (*fn)(void);\n"
                   + "fn refs[] = {" + ", ".join(f"(fn){d}" for d in decls) + "};\n"
                   "int main(void) { qrs_status s = QRS_OK; qrs_out_dtype o = QRS_OUT_F16; (void)o; return (int)s; }\n")
    inc = os.path.dirname(HEADER)
    gcc = shutil.which("gcc") or shutil.which("cc")
    gxx = shutil.which("g++") or shutil.which("c++")
    if gcc is None or gxx is None:
        pytest.skip("no host C/C++ compiler")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only", "-I", inc, str(src)], check=True)
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++", "-I", inc, str(src)],
                   check=True)


def test_strided_run_rejects_address_overflow(fake_ptr_lib):
    lib = fake_ptr_lib
    p = qrs.plan(2, 2 * 65536, 1024, "e4m3fn", "e8m0_block32", "f32")
    A = 1 << 40
    xs = (ctypes.c_void_p * 2)(A, A + (1 << 30))
    ss = (ctypes.c_void_p * 2)(A + (2 << 30), A + (3 << 30))
    huge = (1 << 62) // 16 * 16  # (rows - 1) * stride would overflow 64 bits
    assert lib.qrs_run_strided(p.handle, xs, huge, ss, 32, A + (4 << 30), 1024, None, 0, None) == \
        qrs.Status.INVALID_ARG
    assert lib.qrs_run_strided(p.handle, xs, 1024, ss, 1 << 60, A + (4 << 30), 1024, None, 0, None) == \
        qrs.Status.INVALID_ARG
    assert lib.qrs_run_strided(p.handle, xs, 1024, ss, 32, A + (4 << 30), 1 << 61, None, 0, None) == \
        qrs.Status.INVALID_ARG


def test_strided_run_rejects_row_strides_of_4gib(fake_ptr_lib):
    # Row offsets are 32 x 32-bit products in the kernel: each row stride must
    # stay below 4 GiB (checked on the host, before any launch).
    lib = fake_ptr_lib
    p = qrs.plan(2, 4, 1024, "e4m3fn", "f32_group128", "f32")  # 2 rows
    A = 1 << 44
    xs = (ctypes.c_void_p * 2)(A, A + (8 << 30))
    ss = (ctypes.c_void_p * 2)(A + (16 << 30), A + (24 << 30))
    out = A + (32 << 30)

    def call(ldx, lds, ldo):
        return lib.qrs_run_strided(p.handle, xs, ldx, ss, lds, out, ldo, None, 0, None)

    assert call(1 << 32, 8, 1024) == qrs.Status.INVALID_ARG  # x: 4 GiB
    assert call(1024, 1 << 30, 1024) == qrs.Status.INVALID_ARG  # fp32 scales: 2^30 * 4 bytes
    assert call(1024, 8, 1 << 30) == qrs.Status.INVALID_ARG  # fp32 out: 2^30 * 4 bytes
    assert "4 GiB" in lib.qrs_last_error().decode()


def test_strided_run_rejects_scale_span_of_4gib(fake_ptr_lib):
    lib = fake_ptr_lib
    p = qrs.plan(2, 2 * 5000, 1024, "e4m3fn", "f32_group128", "f32")  # 5000 rows
    A = 1 << 44
    xs = (ctypes.c_void_p * 2)(A, A + (64 << 30))
    ss = (ctypes.c_void_p * 2)(A + (128 << 30), A + (192 << 30))
    out = A + (256 << 30)
    # 5000 rows of fp32 scales 2^18 elements (1 MiB) apart: 4.9 GiB span.
    assert lib.qrs_run_strided(p.handle, xs, 1024, ss, 1 << 18, out, 1024, None, 0, None) == qrs.Status.INVALID_ARG
    assert "4 GiB" in lib.qrs_last_error().decode()


def test_last_error_is_per_thread(lib):
    # Two threads fail at the same time with different arguments; each then
    # reads its own message, not the other thread's.
    import threading

    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, w, h):
        handle = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        for _ in range(200):
            st = lib.qrs_plan(w, 8 * w, h, 1, 1, 1, ctypes.byref(handle), ctypes.byref(ws))
            barrier.wait()  # both calls have failed before either reads
            msg = lib.qrs_last_error().decode()
            barrier.wait()
            if st != qrs.Status.INVALID_ARG or msg != seen.setdefault(name, msg):
                seen[name] = f"changed: {msg}"
                return

    a = threading.Thread(target=worker, args=("w", 3, 1024))
    b = threading.Thread(target=worker, args=("h", 2, 1000))
    a.start()
    b.start()
    a.join(60)
    b.join(60)
    assert seen["w"].startswith("world_size 3"), seen
    assert seen["h"].startswith("h 1000"), seen


def test_last_error_cleared_by_a_successful_call(lib):
    handle = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    assert lib.qrs_plan(3, 24, 1024, 1, 1, 1, ctypes.byref(handle), ctypes.byref(ws)) == qrs.Status.INVALID_ARG
    assert lib.qrs_last_error().decode() != ""
    assert lib.qrs_plan(2, 16, 1024, 1, 1, 1, ctypes.byref(handle), ctypes.byref(ws)) == qrs.Status.OK
    assert lib.qrs_last_error().decode() == ""
    lib.qrs_plan_destroy(handle)


def test_missing_library_fails_loudly(tmp_path):
    """Without the built libqrs.so the binding raises at its first call: there
    is no CPU fallback for any entry point. Checked on a copy of the package
    without the library, in a fresh interpreter."""
    import shutil
    import subprocess
    import sys

    pkg = os.path.dirname(os.path.abspath(qrs.__file__))
    dst = tmp_path / "quantized_collective_reduction_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    assert not list(dst.glob("*.so"))
    code = (
        "import quantized_collective_reduction_amd as q\n"
        "for call in (lambda: q.plan(8, 64, 1024, 'e4m3fn', 'e8m0_block32', 'bf16'),\n"
        "             lambda: q.load_library()):\n"
        "    try:\n"
        "        call()\n"
        "    except ImportError as e:\n"
        "        assert 'no CPU fallback' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('no error without the library')\n"
        "print('ok')\n"
    )
    res = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=120,
                         env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr[-2000:]


def test_failed_plan_construction_leaves_nothing_to_clean_up(lib):
    """A Plan whose arguments are rejected before the C call (an unknown
    dtype name) is finalized without error: no exception escapes __del__."""
    import gc
    import sys

    caught = []
    old = sys.unraisablehook
    sys.unraisablehook = caught.append
    try:
        with pytest.raises(ValueError):
            qrs.plan(8, 64, 1024, "e4m3", "e8m0_block32", "bf16")
        with pytest.raises(qrs.QrsError):
            qrs.plan(3, 64, 1024, "e4m3fn", "e8m0_block32", "bf16")
        gc.collect()
    finally:
        sys.unraisablehook = old
    assert not caught, [str(c.exc_value) for c in caught]
