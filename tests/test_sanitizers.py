"""The library's host code and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/sanitize/host_drive.cpp drives the host half of the library (byte
accounting, the C-ABI argument checks, the capacity planner and the block
manager) and the oracle's store, gather, calibration and attention through
random geometries and operation sequences.  The kernel launches are replaced
by tests/sanitize/launch_stub.cpp, which checks every launch description it
receives against the cache buffer and enqueues nothing, so the build needs no
HIP.  Everything is compiled by gcc/g++ with -fsanitize=address,undefined and
-fno-sanitize-recover=all: any report, or any failed property, fails the test.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_fp8_int4_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("kvq_layout.cpp", "kvq_planner.cpp", "kvq_launch_geometry.cpp",
                                                "kvq_api.cpp")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def sanitized_drive(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    orc_obj = str(d / "kvq_oracle.o")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
          "-Wall", "-Wno-unknown-pragmas", "-c", os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-o", orc_obj])
    exe = str(d / "host_drive")
    _run(["g++", "-std=c++17", *SAN, "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *HOST_SOURCES,
          os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "host_drive.cpp"), orc_obj, "-fopenmp", "-lm", "-o", exe])
    return exe


def test_host_code_and_oracle_under_asan_ubsan(sanitized_drive):
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:detect_stack_use_after_return=1:strict_string_checks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sanitized_drive], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "runtime error" not in report and "Sanitizer" not in report, report[-6000:]
    assert "sanitized host drive ok" in r.stdout


def test_the_sanitized_build_catches_a_planted_overrun(tmp_path):
    """The same flags do report: a one-past-the-end write in a tiny program
    built alike aborts with an AddressSanitizer report (so a clean drive is
    not a build that checks nothing)."""
    src = tmp_path / "overrun.cpp"
    src.write_text("#include <vector>\nint main(int argc, char**) { std::vector<int> v(4); int* p = v.data();"
                   " p[3 + argc] = 1; return 0; }\n")
    exe = str(tmp_path / "overrun")
    _run(["g++", "-std=c++17", *SAN, str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0"))
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr
