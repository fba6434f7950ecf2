"""Static scales for the tests' static layers, derived on each side by that
side's own code.

The static layouts take their scales from a calibration pass ("Per-tensor vs
per-head FP8 KV cache scales", "Calibration changes which scale layout
exists": an amax estimated during warmup, mapped to the largest E4M3 value).
The HIP side calibrates with kvq_calibrate_amax + kvq_static_scales; the
oracle side with the oracle's calibrate_amax and numpy float32 division.  The
two must agree bit for bit (tests/test_gpu_calibration.py checks the same);
a test stores with each side's own scales.
"""
import numpy as np
import torch

PER_TENSOR, PER_HEAD = 1, 2


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_static_scales(orc, keys: torch.Tensor, values: torch.Tensor, mode: int) -> np.ndarray:
    """RN32(amax / 448) per (K/V, head) (per-head) or of the maximum over heads
    (per-tensor), from the oracle's amax; a zero maximum gives the smallest
    positive float32, which keeps the scale valid for a store."""
    hkv, hd = int(keys.shape[1]), int(keys.shape[2])
    a = orc.calibrate_amax(_bits(keys), _bits(values), hkv, hd)
    if mode == PER_TENSOR:
        a = np.array([a[:hkv].max(), a[hkv:].max()], np.float32)
    s = (a / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(np.finfo(np.float32).smallest_subnormal)
    return s


def hip_static_scales(kvq, keys: torch.Tensor, values: torch.Tensor, mode: int) -> list:
    """The same scales from the library: kvq_calibrate_amax on the device,
    then kvq_static_scales."""
    hkv = int(keys.shape[1])
    amax = torch.zeros(2 * hkv, dtype=torch.float32, device=keys.device)
    kvq.kvq_calibrate_amax(keys, values, amax)
    return kvq.kvq_static_scales(amax, hkv, mode)
