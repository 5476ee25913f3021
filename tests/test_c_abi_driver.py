"""The C ABI driven from C++ with no Python in between (tests/c_abi/run_share).

* CPU: a plan the library must reject comes back as a status and message from
  a plain C++ caller (qrs_plan touches no device).
* GPU: the caller runs seeded shares on its own HIP stream with its own
  buffers; the output bytes match the oracle to the same bar as the Python
  binding's parity tests.
"""

import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_parity, log, oracle_bits

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "c_abi", "run_share")

X_CODE = {"int8": 0, "e4m3fn": 1, "e5m2": 2}
SCALE_CODE = {"f32_group128": 0, "e8m0_block32": 1}
OUT_CODE = {"f32": 0, "bf16": 1, "f16": 2}


@pytest.fixture(scope="module")
def driver():
    if not os.path.exists(DRIVER):
        from quantized_collective_reduction_amd import _build

        _build.build_c_abi_driver()
    return DRIVER


def write_problem(path, w, bs, h, x_format, scale_layout, out_dtype, xs, ss):
    with open(path, "wb") as f:
        f.write(struct.pack("<iqqiii", w, bs, h, X_CODE[x_format], SCALE_CODE[scale_layout], OUT_CODE[out_dtype]))
        for x in xs:
            f.write(np.ascontiguousarray(x).tobytes())
        for s in ss:
            f.write(np.ascontiguousarray(s).tobytes())


def test_driver_reports_a_rejected_plan(driver, tmp_path):
    # W = 3 is not a supported world size: qrs_plan fails before any device call.
    src = tmp_path / "bad.bin"
    write_problem(src, 3, 6, 1024, "int8", "f32_group128", "f32", [], [])
    res = subprocess.run([driver, str(src), str(tmp_path / "out.bin")], capture_output=True, text=True, timeout=60)
    assert res.returncode == 3, res.stderr
    assert "qrs_plan: QRS_ERR_INVALID_ARG" in res.stderr and "world_size 3" in res.stderr


def test_driver_reports_h_not_a_group_multiple(driver, tmp_path):
    src = tmp_path / "bad.bin"
    write_problem(src, 2, 4, 1000, "e4m3fn", "e8m0_block32", "bf16", [], [])
    res = subprocess.run([driver, str(src), str(tmp_path / "out.bin")], capture_output=True, text=True, timeout=60)
    assert res.returncode == 3, res.stderr
    assert "qrs_plan: QRS_ERR_INVALID_ARG" in res.stderr


CASES = [
    ("w2_bs32_h1024_int8_f32", None),
    ("w4_bs4096_h4096_e4m3_bf16", 4 * 24),
    ("w8_bs8192_h7168_e5m2_bf16", 8 * 5),
    ("w8_bs16384_h8192_mx_e4m3_bf16", 8 * 6),
    ("w8_bs65536_h5120_mx_e5m2_f32", 8 * 3),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,bs", CASES, ids=[c[0] for c in CASES])
def test_driver_matches_oracle(gpu, driver, tmp_path, name, bs):
    wl = workloads.WORKLOADS[name]
    if bs is not None:
        wl = wl.with_(bs=bs)
    xs, ss = workloads.generate(wl)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    write_problem(src, wl.world_size, wl.bs, wl.h, wl.x_format, wl.scale_layout, wl.out_dtype, xs, ss)
    log(f"c_abi driver: {name} W={wl.world_size} rows={wl.rows} H={wl.h}")
    res = subprocess.run([driver, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    dt = np.uint32 if wl.out_dtype == "f32" else np.uint16
    got = np.fromfile(dst, dtype=dt).reshape(wl.rows, wl.h)
    want = oracle_bits(oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype), wl.out_dtype)
    assert_parity(got, want, wl.out_dtype, name)
