"""Python binding for libqrs: one GPU's share of a quantized reduce-scatter
on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/qrs.h). torch supplies device memory and
streams. If the built library is missing, loading fails with an error; there
is no CPU fallback.

    p = plan(world_size=8, bs=16384, h=8192, x_dtype="e4m3fn",
             scale_layout="e8m0_block32", out_dtype="bf16")
    run(p, x_slices, scale_slices, out)        # on torch's current stream

``x_slices`` / ``scale_slices`` are sequences of W device tensors (or raw
device pointers as ints); ``out`` is a ``[rows, H]`` device tensor.
"""

import ctypes
import os
from enum import IntEnum

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqrs.so")

__all__ = [
    "Status",
    "XDtype",
    "ScaleLayout",
    "OutDtype",
    "QrsError",
    "Plan",
    "load_library",
    "plan",
    "run",
    "run_all_shares",
    "run_strided",
    "slice_pitch",
    "alloc_slices",
    "quantize",
    "Launch",
    "StridedLaunch",
    "AllSharesLaunch",
    "QuantizeLaunch",
    "stream_copy",
    "run_launch_info",
    "LaunchInfo",
    "EXPORTED_SYMBOLS",
]


class Status(IntEnum):
    OK = 0
    INVALID_ARG = 1
    UNSUPPORTED = 2
    HIP = 3
    OUT_OF_MEMORY = 4


class XDtype(IntEnum):
    INT8 = 0
    FP8_E4M3FN = 1
    FP8_E5M2 = 2
    HIFLOAT8 = 3


class ScaleLayout(IntEnum):
    F32_GROUP128 = 0
    E8M0_BLOCK32 = 1


class OutDtype(IntEnum):
    F32 = 0
    BF16 = 1
    F16 = 2


_X_NAMES = {"int8": XDtype.INT8, "e4m3fn": XDtype.FP8_E4M3FN, "e5m2": XDtype.FP8_E5M2, "hifloat8": XDtype.HIFLOAT8}
_SCALE_NAMES = {"f32_group128": ScaleLayout.F32_GROUP128, "e8m0_block32": ScaleLayout.E8M0_BLOCK32}
_OUT_NAMES = {"f32": OutDtype.F32, "bf16": OutDtype.BF16, "f16": OutDtype.F16}

# Every function include/qrs.h declares.
EXPORTED_SYMBOLS = (
    "qrs_plan",
    "qrs_run",
    "qrs_run_all_shares",
    "qrs_run_strided",
    "qrs_quantize",
    "qrs_plan_destroy",
    "qrs_plan_shape",
    "qrs_slice_pitch",
    "qrs_status_string",
    "qrs_last_error",
    "qrs_stream_copy",
    "qrs_run_launch_info",
    "qrs_launch_create",
    "qrs_launch_enqueue",
    "qrs_launch_destroy",
)


class LaunchInfo(ctypes.Structure):
    """qrs_launch_info: the launch qrs_run makes for a plan (see run_launch_info)."""

    _fields_ = [
        ("blocks", ctypes.c_uint64),
        ("threads_per_block", ctypes.c_uint32),
        ("dynamic_lds_bytes", ctypes.c_uint32),
        ("blocks_per_cu_cap", ctypes.c_uint32),
        ("device_cus", ctypes.c_uint32),
        ("device_lds_per_cu", ctypes.c_uint32),
        ("device_lds_per_block", ctypes.c_uint32),
        ("launches", ctypes.c_uint32),
    ]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class QrsError(RuntimeError):
    def __init__(self, status, message):
        self.status = Status(status)
        super().__init__(f"{self.status.name}: {message}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqrs.so and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m quantized_collective_reduction_amd._build` "
            "(there is no CPU fallback)"
        )
    lib = ctypes.CDLL(path)
    c_int, c_i64, c_sz, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.qrs_plan.argtypes = [c_int, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(vp), ctypes.POINTER(c_sz)]
    lib.qrs_plan.restype = c_int
    lib.qrs_run.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, c_sz, vp]
    lib.qrs_run.restype = c_int
    lib.qrs_launch_create.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, ctypes.POINTER(vp)]
    lib.qrs_launch_create.restype = c_int
    lib.qrs_launch_enqueue.argtypes = [vp]
    lib.qrs_launch_enqueue.restype = c_int
    lib.qrs_launch_destroy.argtypes = [vp]
    lib.qrs_launch_destroy.restype = c_int
    lib.qrs_run_all_shares.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), vp, c_sz, vp]
    lib.qrs_run_all_shares.restype = c_int
    lib.qrs_run_strided.argtypes = [vp, ctypes.POINTER(vp), c_i64, ctypes.POINTER(vp), c_i64, vp, c_i64, vp, c_sz, vp]
    lib.qrs_run_strided.restype = c_int
    lib.qrs_quantize.argtypes = [c_i64, c_i64, c_int, c_int, vp, vp, vp, vp]
    lib.qrs_quantize.restype = c_int
    lib.qrs_plan_destroy.argtypes = [vp]
    lib.qrs_plan_destroy.restype = c_int
    lib.qrs_plan_shape.argtypes = [vp, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]
    lib.qrs_plan_shape.restype = c_int
    lib.qrs_slice_pitch.argtypes = [vp, c_int, ctypes.POINTER(c_sz), ctypes.POINTER(c_sz)]
    lib.qrs_slice_pitch.restype = c_int
    lib.qrs_status_string.argtypes = [c_int]
    lib.qrs_status_string.restype = ctypes.c_char_p
    lib.qrs_last_error.argtypes = []
    lib.qrs_last_error.restype = ctypes.c_char_p
    lib.qrs_stream_copy.argtypes = [vp, vp, c_sz, vp]
    lib.qrs_stream_copy.restype = c_int
    lib.qrs_run_launch_info.argtypes = [vp, vp, ctypes.POINTER(LaunchInfo)]
    lib.qrs_run_launch_info.restype = c_int
    _lib = lib
    return lib


def _check(status):
    if status != Status.OK:
        msg = _lib.qrs_last_error().decode(errors="replace")
        raise QrsError(status, msg)


def _enum(value, names, enum_cls):
    if isinstance(value, str):
        key = value.lower()
        if key not in names:
            raise ValueError(f"unknown {enum_cls.__name__} {value!r}; expected one of {sorted(names)}")
        return names[key]
    return enum_cls(value) if value in enum_cls._value2member_map_ else int(value)


class Plan:
    """An immutable plan for one share shape and mode (phase 1 of the op)."""

    def __init__(self, world_size, bs, h, x_dtype, scale_layout, out_dtype):
        self._handle = None  # set first: __del__ runs even when a check below raises
        lib = load_library()
        self.world_size = int(world_size)
        self.bs = int(bs)
        self.h = int(h)
        self.x_dtype = _enum(x_dtype, _X_NAMES, XDtype)
        self.scale_layout = _enum(scale_layout, _SCALE_NAMES, ScaleLayout)
        self.out_dtype = _enum(out_dtype, _OUT_NAMES, OutDtype)
        handle = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.qrs_plan(self.world_size, self.bs, self.h, int(self.x_dtype), int(self.scale_layout),
                            int(self.out_dtype), ctypes.byref(handle), ctypes.byref(ws)))
        self._handle = handle
        self.workspace_bytes = ws.value
        rows, hh = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.qrs_plan_shape(handle, ctypes.byref(rows), ctypes.byref(hh)))
        self.rows = rows.value

    @property
    def handle(self):
        return self._handle

    @property
    def group(self):
        return 128 if self.scale_layout == ScaleLayout.F32_GROUP128 else 32

    def __del__(self):
        if getattr(self, "_handle", None) is not None and _lib is not None:
            _lib.qrs_plan_destroy(self._handle)
            self._handle = None


def plan(world_size, bs, h, x_dtype, scale_layout, out_dtype) -> Plan:
    return Plan(world_size, bs, h, x_dtype, scale_layout, out_dtype)


def slice_pitch(p: Plan, full_inputs=False):
    """Recommended byte distance between consecutive rank slices of x and of
    the scales when each kind shares one allocation (qrs_slice_pitch)."""
    lib = load_library()
    xp, sp = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.qrs_slice_pitch(p.handle, 1 if full_inputs else 0, ctypes.byref(xp), ctypes.byref(sp)))
    return xp.value, sp.value


def alloc_slices(p: Plan, device="cuda", full_inputs=False):
    """One x buffer and one scale buffer holding the W rank slices at the
    recommended pitch. Returns (x_views, scale_views): lists of W contiguous
    device views, ``[rows, H]`` uint8 and ``[rows, H/G]`` fp32 or uint8
    (``rows`` = BS with ``full_inputs``)."""
    import torch

    w = p.world_size
    rows = p.bs if full_inputs else p.rows
    xp, sp = slice_pitch(p, full_inputs)
    g = p.group
    x_buf = torch.empty(xp * w, dtype=torch.uint8, device=device)
    s_buf = torch.empty(sp * w, dtype=torch.uint8, device=device)
    xs = [x_buf[r * xp:r * xp + rows * p.h].view(rows, p.h) for r in range(w)]
    n_s = rows * p.h // g
    if p.scale_layout == ScaleLayout.F32_GROUP128:
        ss = [s_buf[r * sp:r * sp + 4 * n_s].view(torch.float32).view(rows, p.h // g) for r in range(w)]
    else:
        ss = [s_buf[r * sp:r * sp + n_s].view(rows, p.h // g) for r in range(w)]
    return xs, ss


def _element_dtypes():
    """torch element types of the codes, scales and outputs each mode names."""
    import torch

    return (
        {XDtype.INT8: torch.int8, XDtype.FP8_E4M3FN: torch.float8_e4m3fn, XDtype.FP8_E5M2: torch.float8_e5m2},
        {ScaleLayout.F32_GROUP128: torch.float32, ScaleLayout.E8M0_BLOCK32: torch.float8_e8m0fnu},
        {OutDtype.F32: torch.float32, OutDtype.BF16: torch.bfloat16, OutDtype.F16: torch.float16},
    )


def _check_dtype(t, want, what):
    """A tensor with a floating-point element type must have the one the mode
    names (a float16 tensor handed a bf16 result would hold wrong values);
    integer tensors are taken as raw bytes. Raw pointers are not checked, nor
    modes the library rejects anyway (want is None)."""
    if isinstance(t, int) or want is None or t.dtype == want:
        return
    if t.dtype.is_floating_point or t.dtype.is_complex:
        raise ValueError(f"{what}: dtype {t.dtype} does not match the mode's {want}")


def _check_plan_dtypes(p, xs, ss, outs, x_what, s_what, o_what):
    x_dt, s_dt, o_dt = _element_dtypes()
    for r, t in enumerate(xs):
        _check_dtype(t, x_dt.get(p.x_dtype), f"{x_what} {r}")
    for r, t in enumerate(ss):
        _check_dtype(t, s_dt.get(p.scale_layout), f"{s_what} {r}")
    for r, t in enumerate(outs):
        _check_dtype(t, o_dt.get(p.out_dtype), o_what if len(outs) == 1 else f"{o_what} {r}")


def _ptr(t):
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensors only (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream_handle(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_tensor(t, nbytes, what):
    if isinstance(t, int):
        return
    if t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{what}: expected {nbytes} bytes, got {t.numel() * t.element_size()}")


def run(p: Plan, x_slices, scale_slices, out, stream=None):
    """Phase 2: enqueue the share on ``stream`` (torch's current stream by default)."""
    lib = load_library()
    w = p.world_size
    if len(x_slices) != w or len(scale_slices) != w:
        raise ValueError(f"need {w} x slices and {w} scale slices")
    n = p.rows * p.h
    scale_bytes = n // 128 * 4 if p.scale_layout == ScaleLayout.F32_GROUP128 else n // 32
    for r in range(w):
        _check_tensor(x_slices[r], n, f"x slice {r}")
        _check_tensor(scale_slices[r], scale_bytes, f"scale slice {r}")
    _check_tensor(out, n * (4 if p.out_dtype == OutDtype.F32 else 2), "out")
    _check_plan_dtypes(p, x_slices, scale_slices, [out], "x slice", "scale slice", "out")
    xs = (ctypes.c_void_p * w)(*[_ptr(t) for t in x_slices])
    ss = (ctypes.c_void_p * w)(*[_ptr(t) for t in scale_slices])
    _check(lib.qrs_run(p.handle, xs, ss, _ptr(out), None, 0, _stream_handle(stream)))


def _row_stride(tensors, rows, cols, what):
    """Common row stride (in elements) of 2-D device views [rows, cols] whose
    elements within a row are adjacent."""
    strides = set()
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("device tensors only (there is no CPU path)")
        if t.dim() != 2 or tuple(t.shape) != (rows, cols):
            raise ValueError(f"{what}: expected shape [{rows}, {cols}], got {list(t.shape)}")
        if t.stride(1) != 1 and cols > 1:
            raise ValueError(f"{what}: elements within a row must be adjacent")
        strides.add(t.stride(0) if rows > 1 else cols)
    if len(strides) != 1:
        raise ValueError(f"{what}: every slice must have the same row stride")
    return strides.pop()


def _strided_strides(p: Plan, x_slices, scale_slices, out):
    """Row strides of ``run_strided``'s views, in the units qrs_run_strided
    takes (bytes for x, scale elements, output elements). Each view's element
    must be the size of the mode's element, since the library counts its
    strides and row lengths in those."""
    ld_x = _row_stride(x_slices, p.rows, p.h, "x slices")
    ld_s = _row_stride(scale_slices, p.rows, p.h // p.group, "scale slices")
    ld_o = _row_stride([out], p.rows, p.h, "out")
    sizes = ((x_slices, 1, "x slices"),
             (scale_slices, 4 if p.scale_layout == ScaleLayout.F32_GROUP128 else 1, "scale slices"),
             ([out], 4 if p.out_dtype == OutDtype.F32 else 2, "out"))
    for tensors, size, what in sizes:
        for t in tensors:
            if t.element_size() != size:
                raise ValueError(f"{what}: {size}-byte elements expected for this plan, got {t.dtype}")
    return ld_x, ld_s, ld_o


def run_strided(p: Plan, x_slices, scale_slices, out, stream=None):
    """``run`` for 2-D views whose rows are not adjacent (row ranges of wider
    buffers, padded rows): x slices ``[rows, H]`` uint8, scale slices
    ``[rows, H/G]``, out ``[rows, H]``; each kind shares one row stride."""
    lib = load_library()
    w = p.world_size
    if len(x_slices) != w or len(scale_slices) != w:
        raise ValueError(f"need {w} x slices and {w} scale slices")
    ld_x, ld_s, ld_o = _strided_strides(p, x_slices, scale_slices, out)
    _check_plan_dtypes(p, x_slices, scale_slices, [out], "x slice", "scale slice", "out")
    xs = (ctypes.c_void_p * w)(*[t.data_ptr() for t in x_slices])
    ss = (ctypes.c_void_p * w)(*[t.data_ptr() for t in scale_slices])
    _check(lib.qrs_run_strided(p.handle, xs, ld_x, ss, ld_s, out.data_ptr(), ld_o, None, 0, _stream_handle(stream)))


def run_all_shares(p: Plan, x_full, scale_full, out_shares, stream=None):
    """Every rank's share from the ranks' inputs before the all-to-all.

    ``x_full[r]``: rank r's ``[BS, H]`` codes; ``scale_full[r]``: its scales
    for all BS rows; ``out_shares[j]``: share j's ``[BS/W, H]`` output.
    """
    lib = load_library()
    w = p.world_size
    if len(x_full) != w or len(scale_full) != w or len(out_shares) != w:
        raise ValueError(f"need {w} inputs, {w} scale tensors and {w} outputs")
    n = p.rows * p.h
    scale_bytes = n // 128 * 4 if p.scale_layout == ScaleLayout.F32_GROUP128 else n // 32
    for r in range(w):
        _check_tensor(x_full[r], n * w, f"x of rank {r}")
        _check_tensor(scale_full[r], scale_bytes * w, f"scales of rank {r}")
        _check_tensor(out_shares[r], n * (4 if p.out_dtype == OutDtype.F32 else 2), f"output of share {r}")
    _check_plan_dtypes(p, x_full, scale_full, out_shares, "x of rank", "scales of rank", "output of share")
    xs = (ctypes.c_void_p * w)(*[_ptr(t) for t in x_full])
    ss = (ctypes.c_void_p * w)(*[_ptr(t) for t in scale_full])
    os_ = (ctypes.c_void_p * w)(*[_ptr(t) for t in out_shares])
    _check(lib.qrs_run_all_shares(p.handle, xs, ss, os_, None, 0, _stream_handle(stream)))


def _check_quantize_dtypes(x_bf16, x_codes, scales, xd, sl):
    import torch

    x_dt, s_dt, _ = _element_dtypes()
    _check_dtype(x_bf16, torch.bfloat16, "x_bf16")
    _check_dtype(x_codes, x_dt.get(xd), "x_codes")
    _check_dtype(scales, s_dt.get(sl), "scales")


def quantize(x_bf16, x_codes, scales, x_dtype, scale_layout, stream=None):
    """Producer-side quantization of a bf16 ``[tokens, H]`` device tensor into
    ``x_codes`` (uint8 ``[tokens, H]``) and ``scales`` (fp32 ``[tokens, H/128]``
    or uint8 E8M0 ``[tokens, H/32]``)."""
    lib = load_library()
    if isinstance(x_bf16, int):
        raise ValueError("pass tensors (the shape is taken from x_bf16)")
    tokens, h = x_bf16.shape
    xd = _enum(x_dtype, _X_NAMES, XDtype)
    sl = _enum(scale_layout, _SCALE_NAMES, ScaleLayout)
    n = tokens * h
    _check_tensor(x_bf16, 2 * n, "x_bf16")
    _check_tensor(x_codes, n, "x_codes")
    _check_tensor(scales, n // 128 * 4 if sl == ScaleLayout.F32_GROUP128 else n // 32, "scales")
    _check_quantize_dtypes(x_bf16, x_codes, scales, xd, sl)
    _check(lib.qrs_quantize(tokens, h, int(xd), int(sl), _ptr(x_bf16), _ptr(x_codes), _ptr(scales),
                            _stream_handle(stream)))


class Launch:
    """``run`` prepared once (qrs_launch_create: the checks, the kernel, grid
    and residency cap), for repeated launches of one plan on fixed buffers
    and one stream: each call is one qrs_launch_enqueue with one argument."""

    def __init__(self, p: Plan, x_slices, scale_slices, out, stream=None):
        lib = load_library()
        w = p.world_size
        if len(x_slices) != w or len(scale_slices) != w:
            raise ValueError(f"need {w} x slices and {w} scale slices")
        n = p.rows * p.h
        scale_bytes = n // 128 * 4 if p.scale_layout == ScaleLayout.F32_GROUP128 else n // 32
        for r in range(w):
            _check_tensor(x_slices[r], n, f"x slice {r}")
            _check_tensor(scale_slices[r], scale_bytes, f"scale slice {r}")
        _check_tensor(out, n * (4 if p.out_dtype == OutDtype.F32 else 2), "out")
        _check_plan_dtypes(p, x_slices, scale_slices, [out], "x slice", "scale slice", "out")
        self._plan = p  # keeps the plan alive
        self._keep = (list(x_slices), list(scale_slices), out)  # keeps the buffers alive
        xs = (ctypes.c_void_p * w)(*[_ptr(t) for t in x_slices])
        ss = (ctypes.c_void_p * w)(*[_ptr(t) for t in scale_slices])
        h = ctypes.c_void_p()
        _check(lib.qrs_launch_create(p.handle, xs, ss, ctypes.c_void_p(_ptr(out)),
                                     ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(h)))
        self._h = h
        self._destroy = lib.qrs_launch_destroy
        self._fn = lib.qrs_launch_enqueue

    def on_stream(self, stream):
        """The same launch (plan and buffers) enqueued on another stream."""
        return Launch(self._plan, *self._keep, stream=stream)

    def __call__(self):
        status = self._fn(self._h)
        if status:
            _check(status)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None


class StridedLaunch:
    """``run_strided`` with its arguments marshalled once."""

    def __init__(self, p: Plan, x_slices, scale_slices, out, stream=None):
        lib = load_library()
        w = p.world_size
        if len(x_slices) != w or len(scale_slices) != w:
            raise ValueError(f"need {w} x slices and {w} scale slices")
        self._ld_x, self._ld_s, self._ld_o = _strided_strides(p, x_slices, scale_slices, out)
        _check_plan_dtypes(p, x_slices, scale_slices, [out], "x slice", "scale slice", "out")
        self._plan = p
        self._keep = (list(x_slices), list(scale_slices), out)
        self._xs = (ctypes.c_void_p * w)(*[t.data_ptr() for t in x_slices])
        self._ss = (ctypes.c_void_p * w)(*[t.data_ptr() for t in scale_slices])
        self._out = ctypes.c_void_p(out.data_ptr())
        self._stream = ctypes.c_void_p(_stream_handle(stream))
        self._fn = lib.qrs_run_strided
        self._handle = p.handle

    def on_stream(self, stream):
        """The same launch (plan and views) enqueued on another stream."""
        return StridedLaunch(self._plan, *self._keep, stream=stream)

    def __call__(self):
        status = self._fn(self._handle, self._xs, self._ld_x, self._ss, self._ld_s, self._out, self._ld_o, None, 0,
                          self._stream)
        if status:
            _check(status)


class AllSharesLaunch:
    """``run_all_shares`` with its arguments marshalled once."""

    def __init__(self, p: Plan, x_full, scale_full, out_shares, stream=None):
        lib = load_library()
        w = p.world_size
        if len(x_full) != w or len(scale_full) != w or len(out_shares) != w:
            raise ValueError(f"need {w} inputs, {w} scale tensors and {w} outputs")
        n = p.rows * p.h
        scale_bytes = n // 128 * 4 if p.scale_layout == ScaleLayout.F32_GROUP128 else n // 32
        for r in range(w):
            _check_tensor(x_full[r], n * w, f"x of rank {r}")
            _check_tensor(scale_full[r], scale_bytes * w, f"scales of rank {r}")
            _check_tensor(out_shares[r], n * (4 if p.out_dtype == OutDtype.F32 else 2), f"output of share {r}")
        _check_plan_dtypes(p, x_full, scale_full, out_shares, "x of rank", "scales of rank", "output of share")
        self._plan = p
        self._keep = (list(x_full), list(scale_full), list(out_shares))
        self._xs = (ctypes.c_void_p * w)(*[_ptr(t) for t in x_full])
        self._ss = (ctypes.c_void_p * w)(*[_ptr(t) for t in scale_full])
        self._os = (ctypes.c_void_p * w)(*[_ptr(t) for t in out_shares])
        self._stream = ctypes.c_void_p(_stream_handle(stream))
        self._fn = lib.qrs_run_all_shares
        self._handle = p.handle

    def on_stream(self, stream):
        """The same launch (plan and buffers) enqueued on another stream."""
        return AllSharesLaunch(self._plan, *self._keep, stream=stream)

    def __call__(self):
        status = self._fn(self._handle, self._xs, self._ss, self._os, None, 0, self._stream)
        if status:
            _check(status)


class QuantizeLaunch:
    """``quantize`` with its arguments marshalled once."""

    def __init__(self, x_bf16, x_codes, scales, x_dtype, scale_layout, stream=None):
        lib = load_library()
        tokens, h = x_bf16.shape
        self._xd = int(_enum(x_dtype, _X_NAMES, XDtype))
        self._sl = int(_enum(scale_layout, _SCALE_NAMES, ScaleLayout))
        n = tokens * h
        _check_tensor(x_bf16, 2 * n, "x_bf16")
        _check_tensor(x_codes, n, "x_codes")
        _check_tensor(scales, n // 128 * 4 if self._sl == ScaleLayout.F32_GROUP128 else n // 32, "scales")
        _check_quantize_dtypes(x_bf16, x_codes, scales, self._xd, self._sl)
        self._keep = (x_bf16, x_codes, scales)
        self._args = (tokens, h, self._xd, self._sl, _ptr(x_bf16), _ptr(x_codes), _ptr(scales),
                      ctypes.c_void_p(_stream_handle(stream)))
        self._fn = lib.qrs_quantize

    def on_stream(self, stream):
        """The same launch (mode and buffers) enqueued on another stream."""
        return QuantizeLaunch(*self._keep, self._xd, self._sl, stream=stream)

    def __call__(self):
        status = self._fn(*self._args)
        if status:
            _check(status)


def run_launch_info(p: Plan, stream=None) -> dict:
    """The grid, residency cap and device sizes of the launch ``run`` makes
    for ``p`` on ``stream``'s device (qrs_run_launch_info); launches nothing."""
    lib = load_library()
    info = LaunchInfo()
    _check(lib.qrs_run_launch_info(p.handle, _stream_handle(stream), ctypes.byref(info)))
    return info.as_dict()


def stream_copy(src, dst, nbytes=None, stream=None):
    """Calibration copy of ``nbytes`` (default: all of src) from src to dst."""
    lib = load_library()
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _check(lib.qrs_stream_copy(_ptr(src), _ptr(dst), int(nbytes), _stream_handle(stream)))
