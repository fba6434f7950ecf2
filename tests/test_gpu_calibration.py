"""GPU parity of on-the-fly calibration (kvq_calibrate_amax) against the
oracle, and the calibrated static layouts end to end."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    return kvq


def _bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("hkv", [1, 3, 8])
def test_calibrate_amax_matches_oracle(kvq, orc, hd, hkv):
    print(f"[calib] hd={hd} hkv={hkv}", flush=True)
    amax = torch.full((2 * hkv,), 123.0, dtype=torch.float32, device=DEV)
    ref = None
    for i, n in enumerate((1000, 37, 4097)):
        k, v = W.gqa_kv(n, hkv, hd, seed=70 + i)
        if i == 1:                                    # a batch with a huge outlier and a -0 row
            k[3, 0, 5] = -3.0e38
            v[0] = -0.0
        kvq.kvq_calibrate_amax(k.to(DEV), v.to(DEV), amax, accumulate=i > 0)
        ref = orc.calibrate_amax(_bits(k), _bits(v), hkv, hd, amax=ref)
        torch.cuda.synchronize()
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), ref.view(np.uint32)), f"batch {i}"
    e = torch.empty((0, hkv, hd), dtype=torch.bfloat16, device=DEV)
    kvq.kvq_calibrate_amax(e, e, amax, accumulate=False)
    torch.cuda.synchronize()
    assert (amax.cpu() == 0).all()


def test_calibrate_amax_many_rows(kvq, orc):
    """Enough rows (40001 tokens x 8 KV heads) that every workgroup loops
    over several row groups, with a ragged last group."""
    print("[calib] many rows", flush=True)
    k, v = W.gqa_kv(40001, 8, 128, seed=75)
    amax = torch.empty((16,), dtype=torch.float32, device=DEV)
    kvq.kvq_calibrate_amax(k.to(DEV), v.to(DEV), amax, accumulate=False)
    ref = orc.calibrate_amax(_bits(k), _bits(v), 8, 128)
    torch.cuda.synchronize()
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("mode", [W.FP8_PER_TENSOR, W.FP8_PER_HEAD], ids=["per_tensor", "per_head"])
def test_calibrated_static_layout_end_to_end(kvq, orc, mode):
    """Warmup batches -> device amax -> static scales -> store and gather of a
    new batch, all bit-exact against the oracle with the oracle's own amax."""
    print(f"[calib e2e] mode={W.MODE_NAMES[mode]}", flush=True)
    hkv, hd, bs, n = 8, 128, 16, 4096
    amax = torch.empty((2 * hkv,), dtype=torch.float32, device=DEV)
    ref = None
    for i in range(3):
        k, v = W.gqa_kv(2048, hkv, hd, seed=80 + i, device=DEV)
        kvq.kvq_calibrate_amax(k, v, amax, accumulate=i > 0)
        ref = orc.calibrate_amax(_bits(k), _bits(v), hkv, hd, amax=ref)
    scales = kvq.kvq_static_scales(amax, hkv, mode)
    if mode == W.FP8_PER_HEAD:
        want = (ref / np.float32(448.0)).astype(np.float32)
    else:
        want = np.array([ref[:hkv].max(), ref[hkv:].max()], np.float32) / np.float32(448.0)
    assert np.array_equal(np.array(scales, np.float32), want)
    cfg = kvq.CacheConfig(bs, hkv, hd, [mode], [n // bs])
    cache = kvq.Cache(cfg, device=DEV)
    g = orc.Geometry(bs, hkv, hd, [mode], [n // bs])
    host = orc.new_cache(g)
    k, v = W.gqa_kv(n, hkv, hd, seed=90, device=DEV)
    slots = torch.randperm(n, generator=torch.Generator().manual_seed(4)).to(torch.int64)
    cache.store(0, k, v, slots.to(DEV), scales)
    orc.store(g, host, 0, _bits(k), _bits(v), slots.numpy(), want)
    torch.cuda.synchronize()
    assert np.array_equal(cache.buffer.cpu().numpy(), host)
    cache.close()
