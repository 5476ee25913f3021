"""The residency cap of large contiguous shares comes from the launch
device's own sizes: qrs_run_launch_info reports the CU count and LDS sizes
the library read, and they must be the ones the HIP runtime reports for the
device; the cap must follow from them."""

import ctypes

import pytest
import torch

import quantized_collective_reduction_amd as qrs

pytestmark = pytest.mark.gpu

# hipDeviceAttribute_t values (hip_runtime_api.h, ROCm 7)
ATTR_MULTIPROCESSOR_COUNT = 63
ATTR_MAX_SHARED_MEMORY_PER_MULTIPROCESSOR = 10002
ATTR_MAX_SHARED_MEMORY_PER_BLOCK = 74
BLOCKS_PER_CU = 4  # the library's cap for large contiguous shares of 16-element chunks
PIECE_BLOCKS_PER_CU_W8 = 6  # ... and of 8-element pieces (MX scales, 16-bit output) at W = 8
PIECE32_BLOCKS_PER_CU = {8: 4, 4: 6}  # ... and of fp32-output pieces (W = 8 and 4)


def _hip_attr(attr, dev=0):
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    assert path is not None, "the HIP runtime is not loaded"
    hip = ctypes.CDLL(path)
    v = ctypes.c_int(0)
    assert hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0
    return v.value


def _static_lds(info):
    # dynamic = lds_per_cu / cap - static
    return info["device_lds_per_cu"] // info["blocks_per_cu_cap"] - info["dynamic_lds_bytes"]



def test_device_sizes_are_the_runtimes(gpu):
    torch.zeros(1, device="cuda")  # the runtime is initialised
    p = qrs.plan(8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16")
    info = qrs.run_launch_info(p)
    assert info["device_cus"] == _hip_attr(ATTR_MULTIPROCESSOR_COUNT)
    assert info["device_cus"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert info["device_lds_per_cu"] == _hip_attr(ATTR_MAX_SHARED_MEMORY_PER_MULTIPROCESSOR)
    assert info["device_lds_per_block"] == _hip_attr(ATTR_MAX_SHARED_MEMORY_PER_BLOCK)


def _expected_layout(w, sl, od):
    """Elements per lane and blocks per CU of the contiguous share: MX scales
    with a 16-bit output take 8-element pieces, capped at 6 blocks per CU at
    W = 8 and uncapped below; with an fp32 output pieces at W = 8 and 4,
    capped at 4 and 6; every other mode 16-element chunks capped at 4."""
    if sl == "e8m0_block32" and od == "f32" and w in PIECE32_BLOCKS_PER_CU:
        return 8, PIECE32_BLOCKS_PER_CU[w]
    if sl == "e8m0_block32" and od != "f32":
        return 8, (PIECE_BLOCKS_PER_CU_W8 if w == 8 else 0)
    return 16, BLOCKS_PER_CU


@pytest.mark.parametrize("w,bs,h,xd,sl,od", [
    (8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16"),   # 8192 piece blocks
    (8, 16384, 8192, "e5m2", "e8m0_block32", "f16"),      # 8192 piece blocks
    (4, 8192, 8192, "e4m3fn", "e8m0_block32", "bf16"),    # 8192 piece blocks, uncapped at W = 4
    (8, 65536, 5120, "e5m2", "e8m0_block32", "f32"),      # 20480 piece blocks
    (4, 32768, 8192, "e5m2", "e8m0_block32", "f32"),      # 32768 piece blocks, capped at 6
    (2, 16384, 8192, "e4m3fn", "e8m0_block32", "f32"),    # 16384 blocks: chunks at W = 2, fp32 staging in LDS
    (2, 8192, 8192, "int8", "f32_group128", "f32"),       # 8192 blocks
    (8, 16384, 8192, "e4m3fn", "f32_group128", "bf16"),   # 4096 blocks
])
def test_cap_follows_from_the_device(gpu, w, bs, h, xd, sl, od):
    p = qrs.plan(w, bs, h, xd, sl, od)
    info = qrs.run_launch_info(p)
    cus = info["device_cus"]
    per_lane, n_cap = _expected_layout(w, sl, od)
    assert info["threads_per_block"] == 256
    assert info["blocks"] == -(-p.rows * h // per_lane // 256)
    if n_cap and info["blocks"] >= 3 * cus * n_cap:
        assert info["blocks_per_cu_cap"] == n_cap
        per_block = info["device_lds_per_cu"] // n_cap
        assert per_block <= info["device_lds_per_block"]
        static = _static_lds(info)
        if od == "f32" and per_lane == 16:
            assert static == 16 * 1024  # the fp32 chunks' staging buffer
        else:
            assert static < 1024
        assert info["dynamic_lds_bytes"] == per_block - static
    else:
        assert info["blocks_per_cu_cap"] == 0 and info["dynamic_lds_bytes"] == 0


@pytest.mark.parametrize("w,bs,h,xd,sl,od", [
    (8, 8192, 7168, "e5m2", "f32_group128", "bf16"),   # 1792 blocks: one generation, uncapped
    (2, 32, 1024, "int8", "f32_group128", "f32"),      # 4 blocks
])
def test_small_grids_are_not_capped(gpu, w, bs, h, xd, sl, od):
    p = qrs.plan(w, bs, h, xd, sl, od)
    info = qrs.run_launch_info(p)
    assert info["blocks"] < 3 * info["device_cus"] * BLOCKS_PER_CU
    assert info["blocks_per_cu_cap"] == 0 and info["dynamic_lds_bytes"] == 0


def test_launch_info_on_a_side_stream(gpu):
    s = torch.cuda.Stream()
    p = qrs.plan(8, 16384, 8192, "e4m3fn", "e8m0_block32", "bf16")
    assert qrs.run_launch_info(p, stream=s) == qrs.run_launch_info(p)
