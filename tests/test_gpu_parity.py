"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for
bit (cache bytes, FP32 scales and dequantized BF16), on the same seeded
inputs.  Small cases span several workgroups plus a ragged tail; full-size
cases use the workloads' real shapes."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import _calib as C

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return kvq


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _flush(msg):
    print(msg, flush=True)


class Pair:
    """One geometry held by both sides: a device cache and an oracle image."""

    def __init__(self, kvq, orc, bs, hkv, hd, modes, nblocks):
        self.kvq, self.orc = kvq, orc
        self.cfg = kvq.CacheConfig(bs, hkv, hd, modes, nblocks)
        self.cache = kvq.Cache(self.cfg, device=DEV)
        self.g = orc.Geometry(bs, hkv, hd, modes, nblocks)
        self.host = orc.new_cache(self.g)
        assert self.host.size == self.cache.bytes["total"]

    def store(self, layer, k, v, slots, scales=None, orc_scales=None):
        """Store on both sides; orc_scales (default: scales) are the oracle's
        own static scales where each side derives them itself."""
        self.cache.store(layer, k.to(DEV), v.to(DEV), slots.to(DEV), scales)
        if orc_scales is None:
            orc_scales = scales
        sc = None if orc_scales is None else np.asarray(orc_scales, np.float32)
        self.orc.store(self.g, self.host, layer, _bits(k), _bits(v), slots.cpu().numpy(), sc)

    def store_ordered(self, layer, k, v, slots, order, scales=None, orc_scales=None, followed=True):
        """The device side takes the tokens in `order` (kvq_store_ordered);
        the oracle stores, in token order, the tokens the order names (an
        entry outside [0, n) names none) where the layer follows the order,
        else every token: the same cache bytes."""
        n = int(slots.numel())
        self.cache.store(layer, k.to(DEV), v.to(DEV), slots.to(DEV), scales,
                         order=torch.as_tensor(order, dtype=torch.int32).to(DEV))
        o = np.asarray(order, np.int64)
        named = np.zeros(n, bool)
        named[o[(o >= 0) & (o < n)]] = True
        if not followed:
            named[:] = True
        kept = np.where(named, slots.cpu().numpy(), -1).astype(np.int64)
        if orc_scales is None:
            orc_scales = scales
        sc = None if orc_scales is None else np.asarray(orc_scales, np.float32)
        self.orc.store(self.g, self.host, layer, _bits(k), _bits(v), kept, sc)

    def assert_buffers_equal(self):
        torch.cuda.synchronize()
        dev = self.cache.buffer.cpu().numpy()
        if not np.array_equal(dev, self.host):
            bad = np.nonzero(dev != self.host)[0]
            pytest.fail(f"{bad.size} cache bytes differ; first at {bad[0]}: gpu {dev[bad[0]]:#x} "
                        f"oracle {self.host[bad[0]]:#x}")

    def gather_and_compare(self, layer, block_table, seq_lens):
        total = int(np.clip(np.asarray(seq_lens), 0, None).sum())
        shape = (total, self.cfg.num_kv_heads, self.cfg.head_dim)
        out = (torch.zeros(shape, dtype=torch.bfloat16, device=DEV),
               torch.zeros(shape, dtype=torch.bfloat16, device=DEV))
        bt = torch.as_tensor(np.asarray(block_table), dtype=torch.int32).to(DEV)
        sl = torch.as_tensor(np.asarray(seq_lens), dtype=torch.int32).to(DEV)
        self.cache.gather_dequant(layer, bt, sl, total_tokens=total, out=out)
        ko, vo = self.orc.gather(self.g, self.host, layer, np.asarray(block_table), np.asarray(seq_lens))
        for name, d, o in (("keys", out[0], ko), ("values", out[1], vo)):
            db = _bits(d)
            if not np.array_equal(db, o):
                bad = np.argwhere(db != o)
                pytest.fail(f"gather {name}: {len(bad)} elements differ; first at {tuple(bad[0])}: "
                            f"gpu {db[tuple(bad[0])]:#06x} oracle {o[tuple(bad[0])]:#06x}")


def _adversarial_kv(n, hkv, hd, seed):
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(2):
        x = torch.randn((n, hkv, hd), generator=g)
        kinds = torch.randint(0, 8, (n, hkv), generator=g)
        scale = torch.ones((n, hkv))
        scale[kinds == 1] = 0.0
        scale[kinds == 2] = 2.0 ** -130          # BF16 subnormal rows
        scale[kinds == 3] = 2.0 ** 100
        scale[kinds == 4] = 2.0 ** -70            # normal but tiny absmax
        x = x * scale[..., None]
        e = torch.randint(-40, 40, (n, hkv, hd), generator=g).float()
        x = torch.where((kinds == 5)[..., None], x * torch.exp2(e), x)
        x = torch.where((kinds == 6)[..., None] & (torch.rand((n, hkv, hd), generator=g) < 0.5),
                        -0.0 * x.abs(), x)
        out.append(x.to(torch.bfloat16))
    return out


MODES = [W.BF16, W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD]


@pytest.mark.parametrize("hkv", [31, 32, 33, 40])
@pytest.mark.parametrize("hd", [64, 128])
def test_static_per_head_many_kv_heads(kvq, orc, hd, hkv):
    """Static per-head scales with 31-40 KV heads: up to 32 heads each wave
    fetches the whole 2 x hkv table once and reads its heads' pairs across
    lanes; beyond, every lane loads its own pair.  Every head has its own
    scale pair, so a wrong pair changes the codes."""
    _flush(f"[parity] per-head many heads hd={hd} hkv={hkv}")
    bs, nblocks, n = 16, 12, 170
    pair = Pair(kvq, orc, bs, hkv, hd, [W.FP8_PER_HEAD], [nblocks])
    rng = np.random.default_rng(7000 + hd + hkv)
    k, v = _adversarial_kv(n, hkv, hd, seed=int(rng.integers(1 << 30)))
    slots = rng.permutation(nblocks * bs)[:n].astype(np.int64)
    slots[3] = -1
    scales = list((rng.uniform(0.001, 0.05, 2 * hkv) * np.exp2(rng.integers(-4, 5, 2 * hkv))).astype(np.float32))
    pair.store(0, k, v, torch.from_numpy(slots), scales)
    pair.assert_buffers_equal()
    lens = [60, 0, 77, 33]
    bt = np.full((4, nblocks), -1, dtype=np.int32)
    order = rng.permutation(nblocks)
    c = 0
    for b, ln in enumerate(lens):
        for j in range((ln + bs - 1) // bs):
            bt[b, j] = order[c]
            c += 1
    pair.gather_and_compare(0, bt, lens)


@pytest.mark.parametrize("mode", MODES, ids=[W.MODE_NAMES[m] for m in MODES])
@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("hkv", [1, 3, 8])
def test_store_gather_parity_small(kvq, orc, mode, hd, hkv):
    _flush(f"[parity] mode={W.MODE_NAMES[mode]} hd={hd} hkv={hkv}")
    bs = 16 if hkv % 2 else 8
    nblocks, n = 48, 301
    modes = [W.FP8_PER_TOKEN_HEAD, mode, W.INT4_PER_TOKEN_HEAD]
    pair = Pair(kvq, orc, bs, hkv, hd, modes, [3, nblocks, 2])
    rng = np.random.default_rng(hd * 100 + hkv * 7 + mode)
    k, v = _adversarial_kv(n, hkv, hd, seed=int(rng.integers(1 << 30)))
    slots = rng.permutation(nblocks * bs)[:n].astype(np.int64)
    slots[5] = -1
    slots[17] = nblocks * bs + 3
    slots[n - 1] = -7
    scales = None
    if mode == W.FP8_PER_TENSOR:
        scales = [0.013, 0.021]
    elif mode == W.FP8_PER_HEAD:
        scales = list(rng.uniform(0.001, 0.05, 2 * hkv).astype(np.float32))
    pair.store(1, k, v, torch.from_numpy(slots), scales)
    pair.assert_buffers_equal()
    perm = rng.permutation(nblocks).astype(np.int32)
    maxb = 20
    bt = np.full((3, maxb), -1, np.int32)
    bt[0, :16] = perm[:16]
    bt[1, :20] = perm[16:36]
    bt[2, :12] = perm[36:]
    bt[1, 7] = nblocks + 100                     # out-of-range entry: rows left unwritten
    seq_lens = [16 * bs - 5, 20 * bs, 0]
    pair.gather_and_compare(1, bt, seq_lens)
    pair.gather_and_compare(1, bt, [3, -4, 12 * bs])
    pair.cache.close()


@pytest.mark.parametrize("mode", MODES, ids=[W.MODE_NAMES[m] for m in MODES])
@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("hkv", [1, 8])
def test_store_ordered_parity(kvq, orc, mode, hd, hkv):
    """kvq_store_ordered: the tokens taken in slot order, in a random order,
    and in an order with entries outside [0, n) and a repeated token; every
    cache byte against the oracle.  Layers that follow the order (FP8 and
    BF16 at head_dim >= 128) store exactly the tokens it names; the others
    take every token in its own order."""
    _flush(f"[ordered] mode={W.MODE_NAMES[mode]} hd={hd} hkv={hkv}")
    bs, nblocks, n = 16, 40, 437
    rng = np.random.default_rng(77 + hd * 10 + hkv + 1000 * mode)
    slots = rng.permutation(nblocks * bs)[:n].astype(np.int64)
    slots[3] = -1
    slots[n - 2] = nblocks * bs + 5
    scales = None
    if mode == W.FP8_PER_TENSOR:
        scales = [0.017, 0.011]
    elif mode == W.FP8_PER_HEAD:
        scales = list(rng.uniform(0.001, 0.05, 2 * hkv).astype(np.float32))
    broken = rng.permutation(n).astype(np.int64)
    broken[10] = -3                          # names no token
    broken[11] = n + 9                       # names no token
    broken[12] = broken[13]                  # one token twice, another never
    orders = {"slot": np.argsort(slots, kind="stable"), "random": rng.permutation(n), "broken": broken}
    for name, order in orders.items():
        pair = Pair(kvq, orc, bs, hkv, hd, [mode], [nblocks])
        try:
            k, v = _adversarial_kv(n, hkv, hd, seed=int(rng.integers(1 << 30)))
            pair.store_ordered(0, k, v, torch.from_numpy(slots), order.astype(np.int32), scales,
                               followed=bool(kvq._lib.kvq_store_follows_order(mode, hd)))
            pair.assert_buffers_equal()
        finally:
            pair.cache.close()


def _random_geometry(seed):
    rng = np.random.default_rng(9000 + seed)
    bs = int(rng.choice([1, 2, 4, 32, 64, 128, 1024]))
    hkv = int(rng.choice([1, 2, 3, 5, 8, 16]))
    hd = int(rng.choice([64, 128, 256]))
    mode = int(rng.choice(MODES))
    if bs * hkv % 2 and mode in (W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD):
        hkv += 1                      # such a block's scale trailer is not 16-byte sized
    slots_total = max(64, int(rng.integers(64, 2048)) // bs * bs)
    nblocks = max(1, slots_total // bs)
    return rng, bs, hkv, hd, mode, nblocks


@pytest.mark.parametrize("seed", range(24))
def test_store_gather_random_geometries(kvq, orc, seed):
    """Seeded random geometries beyond the fixed cases: block sizes 1 to 1024,
    1 to 16 KV heads, every mode and head_dim, slots permuted with skipped and
    out-of-range entries, block tables with entries outside the layer, ragged
    lengths; every cache byte and gathered value against the oracle."""
    rng, bs, hkv, hd, mode, nblocks = _random_geometry(seed)
    nslots = nblocks * bs
    n = int(rng.integers(1, min(nslots, 300) + 1))
    _flush(f"[random {seed}] mode={W.MODE_NAMES[mode]} bs={bs} hkv={hkv} hd={hd} blocks={nblocks} tokens={n}")
    pair = Pair(kvq, orc, bs, hkv, hd, [mode], [nblocks])
    try:
        k, v = _adversarial_kv(n, hkv, hd, seed=int(rng.integers(1 << 30)))
        slots = rng.permutation(nslots)[:n].astype(np.int64)
        drop = rng.random(n) < 0.05
        slots[drop] = -1
        far = rng.random(n) < 0.03
        slots[far] = nslots + rng.integers(0, 50, int(far.sum()))
        scales = None
        if mode == W.FP8_PER_TENSOR:
            scales = [float(rng.uniform(0.005, 0.05)), float(rng.uniform(0.005, 0.05))]
        elif mode == W.FP8_PER_HEAD:
            scales = list(rng.uniform(0.001, 0.05, 2 * hkv).astype(np.float32))
        pair.store(0, k, v, torch.from_numpy(slots), scales)
        pair.assert_buffers_equal()
        nseq = int(rng.integers(1, 5))
        maxb = int(rng.integers(1, min(nblocks, 12) + 1))
        bt = rng.integers(0, nblocks, (nseq, maxb)).astype(np.int32)
        bad = rng.random((nseq, maxb)) < 0.1
        bt[bad] = rng.choice([-1, nblocks, nblocks + 7])
        lens = [int(rng.integers(0, maxb * bs + 1)) for _ in range(nseq)]
        pair.gather_and_compare(0, bt, lens)
    finally:
        pair.cache.close()


def _exhaustive_rows(start, stride, seed):
    """Rows of 64 BF16 values: element 0 is a positive absmax a (every
    stride-th finite BF16 magnitude from start), the others enumerate every
    BF16 magnitude <= a with random signs."""
    a = torch.arange(start, 0x7F80, stride, dtype=torch.int32)
    counts = a + 1
    rows_per = (counts + 62) // 63
    row_a = torch.repeat_interleave(a, rows_per)
    first = torch.repeat_interleave(torch.cumsum(rows_per, 0) - rows_per, rows_per)
    k = torch.arange(row_a.numel()) - first
    xb = k[:, None] * 63 + torch.arange(63, dtype=torch.int32)[None, :]
    lim = torch.repeat_interleave(counts, rows_per)[:, None]
    xb = torch.where(xb < lim, xb, torch.zeros_like(xb))
    g = torch.Generator().manual_seed(seed)
    sign = torch.randint(0, 2, xb.shape, generator=g, dtype=torch.int32) << 15
    rows = torch.cat([row_a[:, None], xb | sign], dim=1)
    asign = torch.randint(0, 2, (rows.shape[0],), generator=g, dtype=torch.int32) << 15
    rows[:, 0] |= asign
    return rows.to(torch.int16).view(torch.bfloat16)


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD],
                         ids=["fp8_per_token_head", "int4_per_token_head"])
def test_exhaustive_absmax_quotients(kvq, orc, mode):
    """Every positive finite BF16 absmax a (odd bit patterns in K, even in V)
    paired with every BF16 magnitude <= a, random signs: codes, scales and
    dequantized values bit-exact.  Covers every scale the dynamic modes can
    produce (subnormal, tiny, huge) and every quotient below each."""
    _flush(f"[exhaustive] mode={W.MODE_NAMES[mode]}")
    k = _exhaustive_rows(1, 2, seed=1)
    v = _exhaustive_rows(2, 2, seed=2)
    n = max(k.shape[0], v.shape[0])
    n += (-n) % 2
    pad = lambda x: torch.cat([x, torch.zeros((n - x.shape[0], 64), dtype=x.dtype)])   # all-zero rows
    k, v = pad(k), pad(v)
    # two KV heads per token so a block holds an even number of token-heads
    n2 = n // 2
    k, v = k.reshape(n2, 2, 64), v.reshape(n2, 2, 64)
    nb = (n2 + 15) // 16
    pair = Pair(kvq, orc, 16, 2, 64, [mode], [nb])
    pair.store(0, k, v, torch.arange(n2, dtype=torch.int64))
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, np.arange(nb, dtype=np.int32)[None, :], [n2])
    pair.cache.close()


def _all_finite_bf16_rows(hkv):
    b = torch.arange(0, 1 << 16, dtype=torch.int32)
    f = b.to(torch.int16).view(torch.bfloat16)
    f = f[torch.isfinite(f.float())]
    per = hkv * 64
    n = (f.numel() + per - 1) // per
    pad = n * per - f.numel()
    f = torch.cat([f, f[:pad]])
    return f.reshape(n, hkv, 64)


STATIC_SCALES = [1.0, 3.0, 1.0 / 3.0, 2.0 ** -70, 2.0 ** 70, 1e-40, 3e38, 0.0123]


def test_static_scales_every_bf16_value(kvq, orc):
    """Per-tensor layers with scales 1, 3, 1/3, 2^-70, 2^70, an FP32 subnormal,
    3e38 and 0.0123 applied to every finite BF16 value: saturation, prescaled
    division and the E4M3 conversion over the whole input range."""
    _flush("[static] per-tensor all-bf16")
    x = _all_finite_bf16_rows(2)
    n = x.shape[0]
    L = len(STATIC_SCALES)
    pair = Pair(kvq, orc, 16, 2, 64, [W.FP8_PER_TENSOR] * L, [(n + 15) // 16] * L)
    for layer, s in enumerate(STATIC_SCALES):
        sv = float(np.float32(s))
        pair.store(layer, x, x.flip(0).contiguous(), torch.arange(n, dtype=torch.int64), [sv, sv])
    pair.assert_buffers_equal()
    nb = (n + 15) // 16
    for layer in range(L):
        pair.gather_and_compare(layer, np.arange(nb, dtype=np.int32)[None, :], [n])
    pair.cache.close()


def test_static_per_head_extreme_scales(kvq, orc):
    _flush("[static] per-head extremes")
    hkv = 8
    x = _all_finite_bf16_rows(hkv)
    n = x.shape[0]
    sc = [float(np.float32(s)) for s in STATIC_SCALES]
    pair = Pair(kvq, orc, 16, hkv, 64, [W.FP8_PER_HEAD], [(n + 15) // 16])
    pair.store(0, x, x, torch.arange(n, dtype=torch.int64), sc + sc[::-1])
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, np.arange((n + 15) // 16, dtype=np.int32)[None, :], [n])
    # static scales are fixed after first use
    pair.cache.store(0, x.to(DEV), x.to(DEV), torch.arange(n, dtype=torch.int64, device=DEV))
    with pytest.raises(kvq.KVQError):
        pair.cache.store(0, x.to(DEV), x.to(DEV), torch.arange(n, dtype=torch.int64, device=DEV),
                         [1.0] * (2 * hkv))
    pair.cache.close()


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.FP8_PER_TENSOR, W.FP8_PER_HEAD],
                         ids=["fp8_per_token_head", "fp8_per_tensor", "fp8_per_head"])
def test_gqa32_layer_full_size(kvq, orc, mode):
    """32-layer GQA shape, one layer call at full size: 8 sequences x 4096
    tokens, 8 KV heads, head_dim 128, permuted block table; every cache byte and
    every gathered value compared."""
    cfgw = W.WORKLOADS["gqa32"]
    layer = 5
    _flush(f"[gqa32] mode={W.MODE_NAMES[mode]} layer={layer}")
    n = cfgw["num_seqs"] * cfgw["seq_len"]
    nblocks = n // 16
    k, v = W.gqa_kv(n, 8, 128, seed=1000 + layer, device=DEV)
    bt = W.permuted_block_table(cfgw["num_seqs"], cfgw["seq_len"] // 16, nblocks, seed=1000)
    slots = W.slots_from_block_table(bt, [cfgw["seq_len"]] * cfgw["num_seqs"], 16)
    scales = orc_scales = None
    if mode == W.FP8_PER_TENSOR:
        scales = [1.0, 1.0]
    elif mode == W.FP8_PER_HEAD:
        # calibrated on a separate draw, by each side's own calibration
        kc, vc = W.gqa_kv(4096, 8, 128, seed=2000 + layer, device=DEV)
        scales = C.hip_static_scales(kvq, kc, vc, mode)
        orc_scales = C.oracle_static_scales(orc, kc, vc, mode)
        assert np.array_equal(np.asarray(scales, np.float32).view(np.uint32), orc_scales.view(np.uint32))
    pair = Pair(kvq, orc, 16, 8, 128, [mode], [nblocks])
    pair.store(0, k.cpu(), v.cpu(), slots, scales, orc_scales)
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, bt.numpy(), [cfgw["seq_len"]] * cfgw["num_seqs"])
    pair.cache.close()


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.INT4_PER_TOKEN_HEAD],
                         ids=["fp8_per_token_head", "fp8_per_tensor", "fp8_per_head", "int4_per_token_head"])
def test_gqa32_layer_full_size_slot_order(kvq, orc, mode):
    """The GQA-32 layer call as the benchmark times it: 8 sequences x 4096
    tokens under the permuted block table, stored in slot order
    (kvq_store_ordered with argsort of the slots); every cache byte compared."""
    cfgw = W.WORKLOADS["gqa32"]
    layer = 9
    _flush(f"[gqa32 slot order] mode={W.MODE_NAMES[mode]} layer={layer}")
    n = cfgw["num_seqs"] * cfgw["seq_len"]
    nblocks = n // 16
    k, v = W.gqa_kv(n, 8, 128, seed=1000 + layer, device=DEV)
    bt = W.permuted_block_table(cfgw["num_seqs"], cfgw["seq_len"] // 16, nblocks, seed=1000)
    slots = W.slots_from_block_table(bt, [cfgw["seq_len"]] * cfgw["num_seqs"], 16)
    order = np.argsort(slots.numpy(), kind="stable").astype(np.int32)
    scales = orc_scales = None
    if mode == W.FP8_PER_TENSOR:
        scales = [1.0, 1.0]
    elif mode == W.FP8_PER_HEAD:
        kc, vc = W.gqa_kv(4096, 8, 128, seed=2000 + layer, device=DEV)
        scales = C.hip_static_scales(kvq, kc, vc, mode)
        orc_scales = C.oracle_static_scales(orc, kc, vc, mode)
    pair = Pair(kvq, orc, 16, 8, 128, [mode], [nblocks])
    try:
        pair.store_ordered(0, k.cpu(), v.cpu(), slots, order, scales, orc_scales)
        pair.assert_buffers_equal()
    finally:
        pair.cache.close()


@pytest.mark.parametrize("tp,mode", [(8, W.FP8_PER_TOKEN_HEAD), (8, W.INT4_PER_TOKEN_HEAD), (2, W.FP8_PER_TOKEN_HEAD)],
                         ids=["tp8-fp8_per_token_head", "tp8-int4_per_token_head", "tp2-fp8_per_token_head"])
def test_gqa32_shard_layer_full_size(kvq, orc, tp, mode):
    """One tensor-parallel shard's share of a GQA-32 layer call, as the
    benchmark's --tp runs it: 8 / tp KV heads, 8 sequences x 4096 tokens,
    head_dim 128, permuted block table.  At one KV head a block fills half a
    gather workgroup, which then takes half the chunks per thread.  Every cache
    byte and every gathered value compared."""
    cfgw = W.WORKLOADS["gqa32"]
    layer, hkv = 3, 8 // tp
    _flush(f"[gqa32 shard] tp={tp} hkv={hkv} mode={W.MODE_NAMES[mode]} layer={layer}")
    n = cfgw["num_seqs"] * cfgw["seq_len"]
    nblocks = n // 16
    k, v = W.gqa_kv(n, hkv, 128, seed=1000 + layer, device=DEV)
    bt = W.permuted_block_table(cfgw["num_seqs"], cfgw["seq_len"] // 16, nblocks, seed=1000)
    slots = W.slots_from_block_table(bt, [cfgw["seq_len"]] * cfgw["num_seqs"], 16)
    pair = Pair(kvq, orc, 16, hkv, 128, [mode], [nblocks])
    pair.store(0, k.cpu(), v.cpu(), slots)
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, bt.numpy(), [cfgw["seq_len"]] * cfgw["num_seqs"])
    pair.cache.close()


def test_gptoss_sliding_and_full_layers(kvq, orc):
    """gpt-oss shape: a sliding layer kept BF16 in a 128-slot ring buffer and a
    full layer in per-token-head FP8, head_dim 64, 32768 tokens."""
    _flush("[gptoss]")
    T, Wn = 32768, 128
    modes = [W.BF16, W.FP8_PER_TOKEN_HEAD]
    pair = Pair(kvq, orc, 16, 8, 64, modes, [Wn // 16, T // 16])
    for layer in range(2):
        k, v = W.normal_kv(T, 8, 64, seed=4000 + layer, device=DEV)
        slots = W.ring_slots(T, Wn) if layer == 0 else torch.arange(T, dtype=torch.int64)
        pair.store(layer, k.cpu(), v.cpu(), slots)
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, W.ring_block_table(Wn, 16).numpy(), [Wn])
    pair.gather_and_compare(1, np.arange(T // 16, dtype=np.int32)[None, :], [T])
    pair.cache.close()


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 128), (W.INT4_PER_TOKEN_HEAD, 128),
                                     (W.FP8_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 64)],
                         ids=["fp8-128", "int4-128", "fp8-64", "int4-64"])
def test_decode_append_reduced(kvq, orc, mode, hd):
    """Decode pattern at reduced context: 64 sequences x 512-token prefill in a
    random free list of blocks, then 20 steps appending one token per sequence
    (crossing into new blocks), with a full-context gather after some steps."""
    _flush(f"[decode-reduced] mode={W.MODE_NAMES[mode]} hd={hd}")
    S, ctx, steps = 64, 512, 20
    maxb = (ctx + steps + 15) // 16
    nblocks = S * maxb + 7
    st = W.DecodeState(S, 16, nblocks, maxb, seed=5000)
    pair = Pair(kvq, orc, 16, 8, hd, [mode], [nblocks])
    slots = []
    for b in range(S):
        slots += st.append(b, ctx)
    k, v = W.normal_kv(S * ctx, 8, hd, seed=5001, device=DEV)
    pair.store(0, k.cpu(), v.cpu(), torch.tensor(slots, dtype=torch.int64))
    for step in range(steps):
        sl = [st.append(b, 1)[0] for b in range(S)]
        k, v = W.normal_kv(S, 8, hd, seed=5100 + step, device=DEV)
        pair.store(0, k.cpu(), v.cpu(), torch.tensor(sl, dtype=torch.int64))
        if step in (0, 15, steps - 1):
            pair.gather_and_compare(0, st.block_table.numpy(), st.seq_lens)
    pair.assert_buffers_equal()
    pair.cache.close()


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 128), (W.INT4_PER_TOKEN_HEAD, 128),
                                     (W.FP8_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 64)],
                         ids=["fp8_per_token_head-128", "int4_per_token_head-128", "fp8_per_token_head-64",
                              "int4_per_token_head-64"])
def test_decode_layer_full_size(kvq, orc, mode, hd):
    """Decode shape at full size, one layer, in the benchmark's launch
    configuration: 256 sequences prefilled with 8192 tokens each in store
    calls of 32768 tokens, blocks popped from a random free list, then two
    steps appending one token per sequence (the first opens a new block for
    every sequence); every cache byte compared, and the full-context gather of
    all 256 sequences (one launch) compared with the oracle's, 64 sequences at
    a time."""
    _flush(f"[decode-full] mode={W.MODE_NAMES[mode]} hd={hd}")
    S, ctx, bs, hkv, chunk = 256, 8192, 16, 8, 32768
    maxb = ctx // bs + 1
    nblocks = S * maxb
    st = W.DecodeState(S, bs, nblocks, maxb, seed=5000)
    slots = []
    for b in range(S):
        slots += st.append(b, ctx)
    slots = torch.tensor(slots, dtype=torch.int64)
    pair = Pair(kvq, orc, bs, hkv, hd, [mode], [nblocks])
    for c0 in range(0, S * ctx, chunk):
        k, v = W.normal_kv(chunk, hkv, hd, seed=5000 + c0 // chunk, device=DEV)
        pair.store(0, k, v, slots[c0: c0 + chunk])
    for step in range(2):
        sl = torch.tensor([st.append(b, 1)[0] for b in range(S)], dtype=torch.int64)
        k, v = W.normal_kv(S, hkv, hd, seed=6000 + step, device=DEV)
        pair.store(0, k, v, sl)
    pair.assert_buffers_equal()
    lens = np.array(st.seq_lens, np.int32)
    bt = st.block_table.numpy()
    total = int(lens.sum())
    ok = torch.empty((total, hkv, hd), dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ok)
    pair.cache.gather_dequant(0, torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV),
                              total_tokens=total, out=(ok, ov))
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(lens)])
    for b0 in range(0, S, 64):
        rk, rv = orc.gather(pair.g, pair.host, 0, bt[b0: b0 + 64], lens[b0: b0 + 64])
        r0, r1 = int(starts[b0]), int(starts[b0 + 64])
        for name, d, o in (("keys", ok, rk), ("values", ov, rv)):
            db = _bits(d[r0:r1])
            if not np.array_equal(db, o):
                bad = np.argwhere(db != o)
                pytest.fail(f"{name} of sequences {b0}..{b0 + 63}: {len(bad)} elements differ, first at "
                            f"row {r0 + bad[0][0]}")
        del rk, rv
    del ok, ov
    pair.cache.close()


def test_long80_layer_full_size(kvq, orc):
    """80-layer long-context shape, one layer: a single 131072-token sequence,
    heads alternating N(0,1) and Student-t(3), per-token-head FP8, full
    store and full gather compared."""
    _flush("[long80] one layer")
    T = 131072
    k, v = W.heavy_tail_kv(T, 8, 128, seed=3000, device=DEV)
    pair = Pair(kvq, orc, 16, 8, 128, [W.FP8_PER_TOKEN_HEAD], [T // 16])
    pair.store(0, k.cpu(), v.cpu(), torch.arange(T, dtype=torch.int64))
    pair.assert_buffers_equal()
    pair.gather_and_compare(0, np.arange(T // 16, dtype=np.int32)[None, :], [T])
    pair.cache.close()


@pytest.mark.parametrize("num_seqs", [300, 1100])
@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD, W.FP8_PER_HEAD, W.BF16],
                         ids=["fp8_per_token_head", "int4_per_token_head", "fp8_per_head", "bf16"])
def test_gather_many_sequences(kvq, orc, num_seqs, mode):
    """One gather over more than 256 sequences, so the sequence offsets of
    most workgroups are summed past the first 256 lengths: ragged lengths 0 to
    40, some negative, block tables with entries outside the layer; every
    gathered value against the oracle."""
    _flush(f"[many-seqs] num_seqs={num_seqs} mode={W.MODE_NAMES[mode]}")
    bs, hkv, hd, nblocks = 16, 2, 128, 96
    rng = np.random.default_rng(num_seqs * 10 + mode)
    pair = Pair(kvq, orc, bs, hkv, hd, [mode], [nblocks])
    try:
        n = nblocks * bs
        k, v = W.gqa_kv(n, hkv, hd, seed=int(rng.integers(1 << 30)))
        scales = orc_scales = None
        if mode == W.FP8_PER_HEAD:
            scales = C.hip_static_scales(kvq, k.to(DEV), v.to(DEV), mode)
            orc_scales = C.oracle_static_scales(orc, k, v, mode)
        pair.store(0, k, v, torch.from_numpy(rng.permutation(n).astype(np.int64)), scales, orc_scales)
        pair.assert_buffers_equal()
        maxb = 3
        bt = rng.integers(0, nblocks, (num_seqs, maxb)).astype(np.int32)
        bad = rng.random((num_seqs, maxb)) < 0.05
        bt[bad] = rng.choice([-1, nblocks, nblocks + 1000])
        lens = rng.integers(0, 41, num_seqs).astype(np.int32)
        neg = rng.random(num_seqs) < 0.05
        lens[neg] = -rng.integers(1, 30, int(neg.sum()))
        lens[0], lens[255], lens[256], lens[-1] = 40, 0, -5, 33
        pair.gather_and_compare(0, bt, lens)
    finally:
        pair.cache.close()


def test_gather_short_output_is_never_overrun(kvq, orc):
    """An output shorter than the sequences' total receives exactly its
    leading rows, and the bytes just past it (a guard region of the same
    allocation) stay untouched; an output of zero rows receives nothing."""
    _flush("[short output]")
    bs, hkv, hd, nblocks = 16, 2, 64, 8
    pair = Pair(kvq, orc, bs, hkv, hd, [W.FP8_PER_TOKEN_HEAD], [nblocks])
    try:
        n = nblocks * bs
        k, v = W.normal_kv(n, hkv, hd, seed=77)
        pair.store(0, k, v, torch.arange(n, dtype=torch.int64))
        bt = np.arange(nblocks, dtype=np.int32).reshape(2, 4)
        lens = np.array([60, 50], np.int32)
        rk, rv = orc.gather(pair.g, pair.host, 0, bt, lens)
        guard = 0x7FC1                                  # a BF16 NaN pattern the gather never writes
        for short in (0, 1, 37, 59, 60, 83, 109):
            big_k = torch.full((110 + 16, hkv, hd), guard, dtype=torch.int16, device=DEV)
            big_v = big_k.clone()
            ok = big_k.view(torch.bfloat16)[:short]
            ov = big_v.view(torch.bfloat16)[:short]
            kvq.kvq_gather_dequant(pair.cache.handle, 0, torch.from_numpy(bt).to(DEV),
                                   torch.from_numpy(lens).to(DEV), ok, ov)
            torch.cuda.synchronize()
            for big, ref in ((big_k, rk), (big_v, rv)):
                hb = big.cpu().numpy().view(np.uint16)
                assert np.array_equal(hb[:short], ref[:short]), f"rows below {short}"
                assert (hb[short:] == guard).all(), f"guard past {short} rows written"
        # the binding refuses a zero-row or short output unless the total is stated
        e = torch.empty((0, hkv, hd), dtype=torch.bfloat16, device=DEV)
        with pytest.raises(ValueError):
            pair.cache.gather_dequant(0, torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV), out=(e, e))
        with pytest.raises(ValueError):
            s = torch.empty((50, hkv, hd), dtype=torch.bfloat16, device=DEV)
            pair.cache.gather_dequant(0, torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV),
                                      total_tokens=110, out=(s, s))
    finally:
        pair.cache.close()


def test_binding_rejects_wrong_shapes(kvq):
    """The C ABI cannot see a device buffer's size, so the binding checks every
    shape it knows against the cache geometry and raises before any launch."""
    _flush("[binding shapes]")
    cache = kvq.Cache(kvq.CacheConfig(16, 2, 64, [W.FP8_PER_TOKEN_HEAD], [4]), device=DEV)
    try:
        bf = dict(dtype=torch.bfloat16, device=DEV)
        slots = torch.arange(10, dtype=torch.int64, device=DEV)
        good = torch.zeros((10, 2, 64), **bf)
        for k, v, sl in ((torch.zeros((10, 4, 64), **bf), good, slots),        # wrong KV heads
                         (torch.zeros((10, 2, 128), **bf), good, slots),       # wrong head_dim
                         (good, torch.zeros((9, 2, 64), **bf), slots),         # values short
                         (good, good, slots[:8]),                              # slot count
                         (good.view(10, 128), good, slots)):                   # flattened rows
            with pytest.raises(ValueError):
                cache.store(0, k, v, sl)
        bt = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
        sl = torch.tensor([10], dtype=torch.int32, device=DEV)
        with pytest.raises(ValueError):
            cache.gather_dequant(0, bt, sl, out=(torch.zeros((10, 2, 32), **bf), torch.zeros((10, 2, 32), **bf)))
        with pytest.raises(ValueError):
            cache.gather_dequant(0, bt, sl, out=(good, torch.zeros((8, 2, 64), **bf)))
        for q in (torch.zeros((1, 3, 64), **bf), torch.zeros((1, 4, 128), **bf)):
            with pytest.raises(ValueError):
                cache.decode_attention(0, q, bt, sl, 0.125)
        torch.cuda.synchronize()
    finally:
        cache.close()


def test_edge_cases(kvq, orc):
    """Zero tokens, zero sequences, a layer with no blocks, tokens beyond the
    block table, and repeated stores of the same tokens."""
    _flush("[edge]")
    pair = Pair(kvq, orc, 16, 2, 64, [W.FP8_PER_TOKEN_HEAD, W.BF16], [4, 0])
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    pair.cache.store(0, e, e, torch.empty(0, dtype=torch.int64, device=DEV))
    k, v = W.normal_kv(64, 2, 64, seed=9, device=DEV)
    pair.cache.store(1, k, v, torch.arange(64, dtype=torch.int64, device=DEV))   # no blocks: nothing stored
    pair.store(0, k.cpu(), v.cpu(), torch.arange(64, dtype=torch.int64))
    pair.store(0, k.cpu(), v.cpu(), torch.arange(64, dtype=torch.int64))           # idempotent
    pair.assert_buffers_equal()
    out = pair.cache.gather_dequant(0, torch.zeros((0, 4), dtype=torch.int32, device=DEV),
                                    torch.zeros(0, dtype=torch.int32, device=DEV), total_tokens=0)
    assert out[0].numel() == 0
    # seq_len beyond max_blocks * block_size: tokens past the table are not written
    pair.gather_and_compare(0, np.array([[2, 3]], np.int32), [40])
    pair.gather_and_compare(0, np.array([[0, 1, 2, 3], [3, 2, 1, 0]], np.int32), [64, 33])
    pair.cache.close()
