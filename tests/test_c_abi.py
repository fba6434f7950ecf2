"""The boundary from plain C: tests/c_api/host_calls.c includes
include/kvq.h, is compiled by gcc as strict C99, links the built libkvq.so
and calls the host-only entry points (no device is touched, so it runs on
the CPU)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "quantized_fp8_int4_amd", "_build")


def test_c99_caller_of_the_host_entry_points(tmp_path):
    assert os.path.exists(os.path.join(LIB_DIR, "libkvq.so")), "build the library first"
    exe = str(tmp_path / "host_calls")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_api", "host_calls.c"),
           "-L", LIB_DIR, "-lkvq", f"-Wl,-rpath,{LIB_DIR}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi ok" in r.stdout
