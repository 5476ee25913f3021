"""Build libqrs.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m quantized_collective_reduction_amd._build

Flags that matter for results: ``-ffp-contract=off`` (plus a pragma in the
kernel source) keeps every product and sum a separate rounding; packed fp32
instructions are disabled (``-packed-fp32-ops``) so the compiler emits plain
v_mul_f32 / v_add_f32. No fast-math.
"""

import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_ROOT, "include")
LIB_NAME = "libqrs.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [
    os.path.join(CSRC, "qrs.cpp"),
    os.path.join(CSRC, "qrs_kernels.hip"),
    os.path.join(CSRC, "qrs_quantize.hip"),
]

BASE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Kernels whose leading arguments are scalars or pointers get the first
    # 14 dwords of them preloaded into SGPRs at wave launch (the contiguous
    # piece share, the copy, the quantize kernel); kernels whose first
    # argument is a struct are unaffected.
    "-Xarch_device", "-mllvm=-amdgpu-kernarg-preload-count=14",
    "-Wall",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out_path: str = LIB_PATH, defines=(), verbose: bool = False) -> str:
    """Compile the sources into ``out_path`` (atomically replaced)."""
    out_dir = os.path.dirname(os.path.abspath(out_path))
    fd, tmp = tempfile.mkstemp(prefix=".libqrs.", suffix=".so.tmp", dir=out_dir)
    os.close(fd)
    cmd = [hipcc(), *BASE_FLAGS, "-I", INCLUDE, "-I", CSRC, *[f"-D{d}" for d in defines], *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


C_ABI_DRIVER_SRC = os.path.join(REPO_ROOT, "tests", "c_abi", "run_share.cpp")
C_ABI_DRIVER = os.path.join(REPO_ROOT, "tests", "c_abi", "run_share")


def build_c_abi_driver(verbose: bool = False) -> str:
    """Compile the C++ caller used by the tests to exercise the C ABI without
    Python. Links libqrs.so from the package directory (rpath relative to the
    executable)."""
    rel = os.path.relpath(PKG_DIR, os.path.dirname(C_ABI_DRIVER))
    cmd = [hipcc(), "-O2", "-std=c++17", "-I", INCLUDE, C_ABI_DRIVER_SRC, "-L", PKG_DIR, "-lqrs",
           f"-Wl,-rpath,$ORIGIN/{rel}", "-o", C_ABI_DRIVER]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    return C_ABI_DRIVER


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_abi_driver(verbose="-v" in sys.argv))
