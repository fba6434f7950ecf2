"""End to end on the GPU: a model with sliding BF16 layers (ring buffers)
and full quantized layers, sized by kvq_plan_capacity, filled through the
block manager's slots by kvq_store, then read by kvq_gather_dequant and
kvq_decode_attention.  The oracle holds its own image, written by its own
store with the same slots; the sliding layers' attention is also checked
against a plain float64 attention over the last W tokens of the inputs."""
import math

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BS, HKV, HD, GROUP = 16, 2, 64, 4
WINS = [32, 0, 32, 0]
MODES = [W.BF16, W.FP8_PER_TOKEN_HEAD, W.BF16, W.INT4_PER_TOKEN_HEAD]


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return kvq


def _bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_sliding_and_full_layers_through_the_manager(kvq, orc):
    print("[layer-skip] plan, manager, store, gather, attention", flush=True)
    model = kvq.ModelConfig(BS, HKV, HD, MODES, WINS)
    context = 112
    plan, blocks = kvq.kvq_plan_capacity(model, context, 1 << 20)
    assert plan["max_sequences"] >= 3
    cfg = model.cache_config(blocks)
    cache = kvq.Cache(cfg, device=DEV)
    g = orc.Geometry(BS, HKV, HD, MODES, blocks)
    img = orc.new_cache(g)
    maxb = -(-context // BS)
    m = kvq.SeqManager(model, blocks, maxb)
    hist = {l: {} for l in range(4)}           # layer -> seq -> list of (k, v) bf16 rows per token
    gen = torch.Generator().manual_seed(7)
    plan_steps = [(0, 70), (1, 20), (2, 100)] + [(s, 1) for _ in range(5) for s in range(3)] + [(1, 30)]
    for seq, n in plan_steps:
        slots = m.append(seq, n)
        for l in range(4):
            k = (torch.randn((n, HKV, HD), generator=gen) * (1 + l)).to(torch.bfloat16)
            v = torch.randn((n, HKV, HD), generator=gen).to(torch.bfloat16)
            sl = torch.tensor(slots[m.layer_group(l)], dtype=torch.int64)
            cache.store(l, k.to(DEV), v.to(DEV), sl.to(DEV))
            orc.store(g, img, l, _bits(k), _bits(v), sl.numpy())
            hist[l].setdefault(seq, []).extend(zip(_bits(k), _bits(v)))
    torch.cuda.synchronize()
    assert np.array_equal(cache.buffer.cpu().numpy(), img), "cache bytes differ from the oracle's store"

    seqs = [0, 1, 2]
    q = torch.randn((3, HKV * GROUP, HD), generator=gen).to(torch.bfloat16)
    sm = 1.0 / math.sqrt(HD)
    for l in range(4):
        grp = m.layer_group(l)
        bt, lens = m.tables(grp, seqs, maxb)
        bt, lens = np.array(bt, np.int32), np.array(lens, np.int32)
        w = WINS[l]
        for i, s in enumerate(seqs):
            assert lens[i] == (min(len(hist[l][s]), w) if w else len(hist[l][s]))
        # gather, bit exact against the oracle's gather of its own image
        tot = int(lens.sum())
        out = (torch.empty((tot, HKV, HD), dtype=torch.bfloat16, device=DEV),
               torch.empty((tot, HKV, HD), dtype=torch.bfloat16, device=DEV))
        cache.gather_dequant(l, torch.tensor(bt).to(DEV), torch.tensor(lens).to(DEV), out=out)
        ko, vo = orc.gather(g, img, l, bt, lens)
        assert np.array_equal(_bits(out[0]), ko) and np.array_equal(_bits(out[1]), vo)
        # attention within the kernel's error bound
        got = cache.decode_attention(l, q.to(DEV), torch.tensor(bt).to(DEV), torch.tensor(lens).to(DEV), sm)
        torch.cuda.synchronize()
        ref, absv = orc.decode_attention(g, img, l, _bits(q), bt, lens, sm, with_absv=True)
        tol = orc.attention_error_bound(g, img, l, _bits(q), bt, lens, sm, ref, absv)
        err = np.abs(_f64(_bits(got)) - ref)
        assert (err <= tol).all(), f"layer {l}: attention outside the bound by {float((err - tol).max()):.3g}"
        if MODES[l] == W.BF16:
            # a sliding BF16 layer attends over exactly the last W tokens appended
            for i, s in enumerate(seqs):
                rows = hist[l][s][-w:]
                kk = np.stack([_f64(r[0]) for r in rows])            # [n, HKV, HD]
                vv = np.stack([_f64(r[1]) for r in rows])
                for qh in range(HKV * GROUP):
                    sc = kk[:, qh // GROUP, :] @ _f64(_bits(q))[i, qh] * sm
                    p = np.exp(sc - sc.max())
                    want = (p / p.sum()) @ vv[:, qh // GROUP, :]
                    assert np.allclose(ref[i, qh], want, rtol=1e-12, atol=1e-12)
    m.close()
    cache.close()
