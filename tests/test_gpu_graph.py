"""The library's launches under HIP graph capture and on concurrent streams.

Graphs: a store, a dequantizing
gather and a split decode attention with its merge (through a caller
workspace and through the allocation-free entry point) are captured once in
a torch CUDA graph and replayed.  Each replay follows eager work on the same
stream (its outputs cleared by fill kernels, unrelated arithmetic) and a
synchronization, and must reproduce the eager calls' outputs bit for bit:
the calls allocate nothing, clear nothing with a memset, and launch on the
stream they are given, so the captured launches are the eager ones.

Streams: two caches stored and gathered at once from two streams give what
each gives alone."""
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


def test_two_streams_two_caches(kvq):
    """Distinct caches used at once from two streams: each stream stores a
    layer and gathers it back while the other does the same; the results
    equal one stream's calls made alone, bit for bit."""
    hkv, hd, bs = 8, 128, 16
    lens = [1500, 900, 41]
    need = [-(-n // bs) for n in lens]
    maxb, nblocks = max(need) + 1, sum(need) + 2
    st = W.DecodeState(len(lens), bs, nblocks, maxb, seed=81)
    slots = []
    for b, n in enumerate(lens):
        slots += st.append(b, n)
    n = len(slots)
    slots = torch.tensor(slots, dtype=torch.int64, device=DEV)
    bt = st.block_table.to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    modes = (W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD)
    inputs = [W.gqa_kv(n, hkv, hd, seed=82 + i, device=DEV) for i in range(2)]

    def run(cache, kv, out):
        cache.store(0, kv[0], kv[1], slots)
        cache.gather_dequant(0, bt, sl, total_tokens=n, out=out)

    def outs():
        return (torch.empty((n, hkv, hd), dtype=torch.bfloat16, device=DEV),
                torch.empty((n, hkv, hd), dtype=torch.bfloat16, device=DEV))

    caches = [kvq.Cache(kvq.CacheConfig(bs, hkv, hd, [m], [nblocks]), device=DEV) for m in modes]
    try:
        alone = []
        for c, kv in zip(caches, inputs):
            o = outs()
            run(c, kv, o)
            torch.cuda.synchronize()
            alone.append(o)
        together = [outs(), outs()]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for rep in range(3):
            for c, kv, o, s in zip(caches, inputs, together, streams):
                with torch.cuda.stream(s):
                    o[0].zero_()
                    o[1].zero_()
                    run(c, kv, o)
            torch.cuda.synchronize()
            for i in range(2):
                assert torch.equal(together[i][0], alone[i][0]) and torch.equal(together[i][1], alone[i][1]), \
                    f"rep {rep}: cache {i} differs when run beside the other"
    finally:
        for c in caches:
            c.close()
