"""Pins of the oracle's scalar codecs against things other than itself:
torch's float8_e4m3fn / bfloat16 conversions, numpy's IEEE float32 division,
brute-force nearest-code search, and the E4M3 closed form.

E4M3 itself: "Per-tensor vs per-head FP8 KV cache scales", "Range sharing
explains the accuracy trade" (values are mapped through a scale into E4M3;
values outside the range clip).  INT4: "Per-token-head KV cache scale
overhead", "INT4 makes the metadata fraction larger".
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

CHUNK = 1 << 26


def _torch_e4m3_saturating(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(v).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(orc.e4m3_encode(f), _torch_e4m3_saturating(f))


def test_e4m3_encode_all_positive_fp32_and_strided_negative(orc):
    """Every finite positive float32 pattern, and every 7th negative one."""
    for start in range(0, 0x7F800000, CHUNK):
        stop = min(start + CHUNK, 0x7F800000)
        f = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        got = orc.e4m3_encode(f)
        want = _torch_e4m3_saturating(f)
        if not np.array_equal(got, want):
            i = int(np.nonzero(got != want)[0][0])
            pytest.fail(f"fp32 {f[i]!r} (bits {start + i:#x}): oracle {got[i]:#x} torch {want[i]:#x}")
    for start in range(0x80000000, 0xFF800000, CHUNK * 7):
        stop = min(start + CHUNK * 7, 0xFF800000)
        f = np.arange(start, stop, 7, dtype=np.uint64).astype(np.uint32).view(np.float32)
        assert np.array_equal(orc.e4m3_encode(f), _torch_e4m3_saturating(f))


def _e4m3_value(code: int) -> Fraction:
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    mag = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_closed_form_and_torch(orc):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    got = orc.e4m3_decode(codes)
    for c, g in zip(codes, got):
        assert Fraction(float(g)) == _e4m3_value(int(c)), hex(c)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert got[codes == 0x7E][0] == 448.0


def _brute_force_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest of the 127 non-negative finite codes to min(|v|, 448); ties go
    to the even code.  Sign copied from v."""
    vals = np.array([float(_e4m3_value(c)) for c in range(127)], np.float64)
    m = np.minimum(np.abs(v.astype(np.float64)), 448.0)[:, None]
    d = np.abs(m - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    ties = d == best
    # among the tied codes pick the even one (there are at most two, adjacent)
    idx = np.where(ties.sum(1) > 1,
                   np.argmax(ties & (np.arange(127)[None, :] % 2 == 0), axis=1),
                   np.argmax(ties, axis=1))
    return (idx.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8))


def test_e4m3_encode_brute_force_midpoints(orc):
    vals = np.array([float(_e4m3_value(c)) for c in range(127)], np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = rng.uniform(-500, 500, 20000).astype(np.float32)
    tiny = (rng.uniform(-1, 1, 5000) * 2.0 ** -5).astype(np.float32)
    v = np.concatenate([mids, up, dn, -mids, -up, -dn, rnd, tiny, vals.astype(np.float32),
                        np.array([0.0, -0.0, 448.0, 464.0, 1e30, -1e30], np.float32)])
    assert np.array_equal(orc.e4m3_encode(v), _brute_force_e4m3(v))


def test_int4_encode_vs_torch_round(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-10, 10, 100000),
                        np.arange(-20, 20.5, 0.5),
                        [0.0, -0.0, 7.49, 7.5, -8.5, -8.49, 1e9, -1e9]]).astype(np.float32)
    want = torch.round(torch.from_numpy(v)).clamp(-8, 7).to(torch.int8).numpy()
    assert np.array_equal(orc.int4_encode(v), want)


def test_quotient_vs_numpy_ieee_division(orc):
    rng = np.random.default_rng(3)
    x = (rng.integers(0, 1 << 16, 2_000_000, dtype=np.uint32) << 16).view(np.float32)
    s = rng.integers(0x00000001, 0x7F7FFFFF, 2_000_000, dtype=np.uint32).view(np.float32)
    ok = np.isfinite(x)
    x, s = x[ok], s[ok]
    with np.errstate(all="ignore"):
        want = x / s
    got = orc.quotient(x, s)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_quotient_on_dynamic_scales_vs_numpy(orc):
    """x / RN(a/448) and x / RN(a/7) for every positive finite bf16 a and
    x drawn from the bf16 values not above a (the domain the store reaches)."""
    a = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(5)
    for qmax in (448.0, 7.0):
        s = orc.dynamic_scale(a, qmax)
        with np.errstate(all="ignore"):
            assert np.array_equal(s.view(np.uint32), (a / np.float32(qmax)).view(np.uint32))
        # 64 random bf16 magnitudes <= a per a, both signs
        frac = rng.integers(0, 1 << 16, (a.size, 64), dtype=np.uint32)
        abits = (a.view(np.uint32) >> 16)[:, None]
        xb = (frac % (abits + 1)) | (rng.integers(0, 2, frac.shape, dtype=np.uint32) << 15)
        x = (xb.astype(np.uint32) << 16).view(np.float32)
        ss = np.broadcast_to(s[:, None], x.shape)
        got = orc.quotient(x.ravel(), ss.ravel())
        with np.errstate(all="ignore"):
            want = (x / ss).ravel()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_rounding_vs_torch(orc):
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 1 << 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    halfway = ((rng.integers(0, 1 << 16, 100000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    halfway = halfway[np.isfinite(halfway) & (np.abs(halfway) < 3.3e38)]
    f = np.concatenate([f, halfway, np.array([0.0, -0.0, 1e-45, -1e-45], np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.float_to_bf16(f), want)


def test_dequant_product_then_bf16(orc):
    """BF16_RNE(RN32(decode(code) * s)) against torch float32 multiply and bf16 cast."""
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 256, 500000, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    s = rng.integers(1, 0x7F000000, codes.size, dtype=np.uint32).view(np.float32)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    prod = dec * torch.from_numpy(s)
    ok = torch.isfinite(prod).numpy() & (prod.abs() < 3.3e38).numpy()
    want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.dequant_fp8(codes, s)
    assert np.array_equal(got[ok], want[ok])


def test_max_element_hits_top_code_for_every_absmax(orc):
    """For every positive finite bf16 absmax a: a / RN(a/448) encodes to 448
    (code 0x7E) and a / RN(a/7) rounds to 7 -- so every non-zero token-head
    uses the top of its range, and INT4 -8 never occurs in dynamic mode."""
    a = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    s8 = orc.dynamic_scale(a, 448.0)
    assert (orc.e4m3_encode(orc.quotient(a, s8)) == 0x7E).all()
    assert (orc.e4m3_encode(orc.quotient(-a, s8)) == 0xFE).all()
    s4 = orc.dynamic_scale(a, 7.0)
    q4 = orc.quotient(a, s4)
    assert (orc.int4_encode(q4) == 7).all() and (orc.int4_encode(-q4) == -7).all()
    assert q4.max() < 7.5 and (s8 > 0).all() and (s4 > 0).all()
