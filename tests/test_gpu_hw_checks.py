"""Device checks of the FP32 scale arithmetic the store kernel uses in place
of IEEE division (tests/hw_checks/rcp_newton.hip): the hardware reciprocal
plus one Newton step equals the IEEE reciprocal on every normal FP32 input,
and the corrected constant division equals IEEE a/448 and a/7 on every BF16
absmax >= 2^-100."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_checks", "_build", "libkvq_hwcheck.so")


@pytest.fixture(scope="module")
def hw():
    import torch  # noqa: F401  (HIP runtime shared with the library)
    lib = ctypes.CDLL(LIB)
    lib.kvq_hw_rcp_mismatches.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint64)]
    lib.kvq_hw_cdiv_mismatches.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_uint64)]
    return lib


def test_rcp_newton_exact_on_every_normal_float(hw):
    print("[hw] rcp_exact over [2^-126, 2^126)", flush=True)
    out = ctypes.c_uint64(123)
    assert hw.kvq_hw_rcp_mismatches(1 << 23, 253 << 23, ctypes.byref(out)) == 0
    assert out.value == 0


@pytest.mark.parametrize("q", [448, 7])
def test_constant_division_exact_on_every_bf16_absmax(hw, q):
    print(f"[hw] div_by_const<{q}>", flush=True)
    out = ctypes.c_uint64(123)
    assert hw.kvq_hw_cdiv_mismatches(q, ctypes.byref(out)) == 0
    assert out.value == 0
