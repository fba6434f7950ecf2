"""kvq_decode_attention_noalloc (split partials in the library's fixed
per-GPU array) against kvq_decode_attention (partials in a caller
workspace), through the C ABI: the same kernels and plan, so every output
element must be equal, bit for bit.  Two calls in a row, the second with a
smaller input, so the second reads the array that the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return kvq


def _bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy()


def _call_noalloc(kvq, cache, layer, q, bt, sl, sm, out):
    st = kvq._lib.kvq_decode_attention_noalloc(
        cache.handle, layer, ctypes.c_void_p(q.data_ptr()), int(q.shape[1]), ctypes.c_void_p(bt.data_ptr()),
        int(bt.shape[1]), ctypes.c_void_p(sl.data_ptr()), int(sl.numel()), ctypes.c_float(sm),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.OK, kvq._lib.kvq_status_string(st)


def _call_workspace(kvq, cache, layer, q, bt, sl, sm, out):
    need = kvq.kvq_decode_attention_workspace(cache.handle, q.shape[1], bt.shape[1], sl.numel())
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    st = kvq._lib.kvq_decode_attention(
        cache.handle, layer, ctypes.c_void_p(q.data_ptr()), int(q.shape[1]), ctypes.c_void_p(bt.data_ptr()),
        int(bt.shape[1]), ctypes.c_void_p(sl.data_ptr()), int(sl.numel()), ctypes.c_float(sm),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ctypes.c_uint64(ws.numel()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.OK, kvq._lib.kvq_status_string(st)
    return need


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 128), (W.INT4_PER_TOKEN_HEAD, 64), (W.BF16, 256)],
                         ids=["fp8_per_token_head-128", "int4_per_token_head-64", "bf16-256"])
def test_noalloc_attention_equals_workspace_attention(kvq, mode, hd):
    print(f"[noalloc] mode={W.MODE_NAMES[mode]} hd={hd}", flush=True)
    bs, hkv, H = 16, 8, 32
    n = 6000
    nblocks = n // bs + 1
    cache = kvq.Cache(kvq.CacheConfig(bs, hkv, hd, [mode], [nblocks]), device=DEV)
    try:
        k, v = W.gqa_kv(n, hkv, hd, seed=31, device=DEV)
        perm = torch.randperm(nblocks, generator=torch.Generator().manual_seed(5)).to(torch.int32)
        slots = (perm[torch.arange(n) // bs].to(torch.int64) * bs + torch.arange(n) % bs).to(DEV)
        cache.store(0, k, v, slots)
        bt_all = perm.view(1, -1)
        # first call: three sequences over the same blocks, the longest split
        # many times; second call: one shorter sequence
        for lens in ([n, 2500, 77], [1800]):
            ns = len(lens)
            bt = bt_all.repeat(ns, 1).to(DEV)
            sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
            g = torch.Generator(device=DEV).manual_seed(sum(lens))
            q = torch.randn((ns, H, hd), generator=g, device=DEV).to(torch.bfloat16)
            sm = 1.0 / float(np.sqrt(hd))
            ref = torch.full_like(q, float("nan"))
            got = torch.full_like(q, float("nan"))
            need = _call_workspace(kvq, cache, 0, q, bt, sl, sm, ref)
            assert 0 < need <= kvq.ATTENTION_SCRATCH_BYTES     # the shape is split: the array is used
            _call_noalloc(kvq, cache, 0, q, bt, sl, sm, got)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(got), _bits(ref)), f"lengths {lens}"
            assert torch.isfinite(got.float()).all()
    finally:
        cache.close()


def test_noalloc_attention_one_split_and_empty(kvq):
    """A batch taking one split needs no partials; zero sequences is a no-op."""
    print("[noalloc] one split", flush=True)
    bs, hkv, hd, H = 16, 8, 128, 32
    cache = kvq.Cache(kvq.CacheConfig(bs, hkv, hd, [W.FP8_PER_TOKEN_HEAD], [64]), device=DEV)
    try:
        k, v = W.normal_kv(1024, hkv, hd, seed=3, device=DEV)
        cache.store(0, k, v, torch.arange(1024, dtype=torch.int64, device=DEV))
        bt = torch.arange(64, dtype=torch.int32, device=DEV).view(8, 8)
        sl = torch.tensor([128, 100, 0, 1, 64, 17, 128, 5], dtype=torch.int32, device=DEV)
        q = torch.randn((8, H, hd), generator=torch.Generator(device=DEV).manual_seed(4), device=DEV).to(torch.bfloat16)
        assert kvq.kvq_decode_attention_workspace(cache.handle, H, 8, 8) == 0
        ref = torch.empty_like(q)
        got = torch.empty_like(q)
        _call_workspace(kvq, cache, 0, q, bt, sl, 0.09, ref)
        _call_noalloc(kvq, cache, 0, q, bt, sl, 0.09, got)
        kvq.kvq_decode_attention_noalloc(cache.handle, 0, q[:0], bt[:0], sl[:0], 0.09, got[:0])
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(ref))
    finally:
        cache.close()
