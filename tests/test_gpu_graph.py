"""The library's launches under HIP graph capture.  A store, a dequantizing
gather and a split decode attention with its merge (through a caller
workspace and through the allocation-free entry point) are captured once in
a torch CUDA graph and replayed.  Each replay follows eager work on the same
stream (its outputs cleared by fill kernels, unrelated arithmetic) and a
synchronization, and must reproduce the eager calls' outputs bit for bit:
the calls allocate nothing, clear nothing with a memset, and launch on the
stream they are given, so the captured launches are the eager ones."""
import ctypes

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


def _noalloc(kvq, cache, q, bt, sl, sm, out):
    st = kvq._lib.kvq_decode_attention_noalloc(
        cache.handle, 0, ctypes.c_void_p(q.data_ptr()), int(q.shape[1]), ctypes.c_void_p(bt.data_ptr()),
        int(bt.shape[1]), ctypes.c_void_p(sl.data_ptr()), int(sl.numel()), ctypes.c_float(sm),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.OK, kvq._lib.kvq_status_string(st)


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 128), (W.INT4_PER_TOKEN_HEAD, 64),
                                     (W.FP8_PER_TENSOR, 128)],
                         ids=["fp8_per_token_head-hd128", "int4_per_token_head-hd64", "fp8_per_tensor-hd128"])
def test_graph_replays_equal_eager(kvq, mode, hd):
    hkv, bs, H = 8, 16, 32
    lens = [2000, 37, 600]             # the long sequence takes 16 split ranges and the wide merge
    S = len(lens)
    need = [-(-n // bs) for n in lens]
    maxb = max(need) + 1
    nblocks = sum(need) + 4
    st = W.DecodeState(S, bs, nblocks, maxb, seed=71)
    slots = []
    for b, n in enumerate(lens):
        slots += st.append(b, n)
    n = len(slots)
    slots = torch.tensor(slots, dtype=torch.int64, device=DEV)
    k, v = W.gqa_kv(n, hkv, hd, seed=72, device=DEV)
    scales = [0.05, 0.04] if mode == W.FP8_PER_TENSOR else None
    cache = kvq.Cache(kvq.CacheConfig(bs, hkv, hd, [mode], [nblocks]), device=DEV)
    bt = st.block_table.to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = torch.randn((S, H, hd), generator=torch.Generator(device=DEV).manual_seed(73), device=DEV).to(torch.bfloat16)
    sm = 1.0 / hd ** 0.5
    ws = torch.empty(max(kvq.kvq_decode_attention_workspace(cache.handle, H, maxb, S), 16), dtype=torch.uint8,
                     device=DEV)

    def buffers():
        return [torch.empty((n, hkv, hd), dtype=torch.bfloat16, device=DEV),
                torch.empty((n, hkv, hd), dtype=torch.bfloat16, device=DEV),
                torch.empty_like(q), torch.empty_like(q)]

    def step(o):
        cache.store(0, k, v, slots, scales)
        cache.gather_dequant(0, bt, sl, total_tokens=n, out=(o[0], o[1]))
        cache.decode_attention(0, q, bt, sl, sm, out=o[2], workspace=ws)
        _noalloc(kvq, cache, q, bt, sl, sm, o[3])

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    assert torch.equal(eager[2], eager[3])        # the two attention entry points agree

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(buffers())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    got = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(got)
    torch.cuda.synchronize()
    try:
        for rep in range(3):
            for t in got:
                t.zero_()
            junk = (k.float() * (rep + 2)).sum()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, a, b in zip(("keys", "values", "attention", "attention_noalloc"), got, eager):
                assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
            assert torch.isfinite(junk)
    finally:
        del graph
        cache.close()
