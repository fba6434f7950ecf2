"""Build the gfx950 shared library libkvq.so in-tree with hipcc.

    python quantized_fp8_int4_amd/build.py

Flags: IEEE single precision on the device (no fast-math, FP32 denormals kept,
no mul-add contraction: the kernels place every fused multiply-add
explicitly), and no packed FP32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libkvq.so")
SOURCES = ["kvq_kernels.hip", "kvq_calib.hip", "kvq_attention.hip", "kvq_api.cpp", "kvq_layout.cpp",
           "kvq_planner.cpp", "kvq_launch_geometry.cpp"]
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, at most 4 compilers) and link
    libkvq.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as pool:
        objs = list(pool.map(lambda src: _compile(src, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


HW_CHECK_SRC = os.path.join(ROOT, "tests", "hw_checks", "rcp_newton.hip")
HW_CHECK_LIB = os.path.join(ROOT, "tests", "hw_checks", "_build", "libkvq_hwcheck.so")


def build_hw_checks(verbose: bool = False) -> str:
    """The device test library that checks the exact scale arithmetic."""
    os.makedirs(os.path.dirname(HW_CHECK_LIB), exist_ok=True)
    tmp = HW_CHECK_LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", CSRC, HW_CHECK_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {HW_CHECK_SRC}:\n{r.stderr}")
    os.replace(tmp, HW_CHECK_LIB)
    return HW_CHECK_LIB


C_DEVICE_SRC = os.path.join(ROOT, "tests", "c_api", "device_roundtrip.c")
C_DEVICE_EXE = os.path.join(ROOT, "tests", "c_api", "_build", "device_roundtrip")


def build_c_tests(verbose: bool = False) -> str:
    """The plain C99 GPU test program (HIP runtime C API + the library's C ABI),
    compiled by gcc; it finds libkvq.so relative to itself."""
    os.makedirs(os.path.dirname(C_DEVICE_EXE), exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_DEVICE_EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_DEVICE_SRC,
           "-L", BUILD_DIR, "-lkvq", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../../quantized_fp8_int4_amd/_build", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_DEVICE_SRC}:\n{r.stderr}")
    os.replace(tmp, C_DEVICE_EXE)
    return C_DEVICE_EXE


CEILING_SRC = os.path.join(ROOT, "ceiling", "copy_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "ceiling", "_build", "libkvq_ceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """The benchmark's bandwidth-ceiling kernels (a separate library, never
    loaded by libkvq.so or the binding)."""
    os.makedirs(os.path.dirname(CEILING_LIB), exist_ok=True)
    tmp = CEILING_LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", CEILING_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CEILING_SRC}:\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_hw_checks(verbose="-v" in sys.argv))
    print(build_c_tests(verbose="-v" in sys.argv))
    print(build_ceiling(verbose="-v" in sys.argv))
