"""The GPU path from plain C: tests/c_api/device_roundtrip.c (built by
__graft_entry__.build() with gcc: HIP runtime C API + the library's C ABI, no
Python and no torch in the process) stores per-token-head FP8 and INT4 rows
whose round trip is exact by construction and gathers them back through a
permuted block table, bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_api", "_build", "device_roundtrip")


def test_c99_program_stores_and_gathers_on_the_gpu():
    assert os.path.exists(EXE), "run __graft_entry__.build() first"
    print("[c-abi] device_roundtrip", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi device ok" in r.stdout
