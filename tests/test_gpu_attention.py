"""GPU parity of the fused decode attention: the HIP kernel, called through
the C ABI, against the oracle's float64 attention over the same cache image.
The image is written by the oracle's own store on the CPU and uploaded byte
for byte, so no input of the oracle comes from the HIP path.

Tolerance, per output element: oracle.attention_error_bound, derived from
the kernel's arithmetic (BF16 softmax weights times the V scales in the value
product, FP32 accumulation, a BF16 output, FP32 score error and underflow).
Short sequences make a dropped or stray token exceed the bound; long ones
exercise the split and combine kernels."""
import math

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


def _f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _flush(msg):
    print(msg, flush=True)


class Scenario:
    """One layer of one mode: an oracle-written cache image, the same bytes
    on the device, a block table, lengths and queries."""

    def __init__(self, kvq, orc, mode, hd, hkv, bs, lens, group, seed=0, extra_blocks=3, kv=None):
        self.kvq, self.orc = kvq, orc
        self.mode, self.hd, self.hkv, self.bs, self.group = mode, hd, hkv, bs, group
        self.lens = [int(x) for x in lens]
        need = [-(-n // bs) for n in self.lens]
        self.maxb = max(need + [1]) + 1
        self.nblocks = sum(need) + extra_blocks
        self.g = orc.Geometry(bs, hkv, hd, [mode], [self.nblocks])
        self.img = orc.new_cache(self.g)
        st = W.DecodeState(len(self.lens), bs, self.nblocks, self.maxb, seed)
        slots = []
        for b, n in enumerate(self.lens):
            slots += st.append(b, n)
        self.bt = st.block_table.numpy().copy()
        n = len(slots)
        k, v = kv if kv is not None else W.gqa_kv(n, hkv, hd, seed=seed + 1)
        self.scales = None
        if mode in (W.FP8_PER_TENSOR, W.FP8_PER_HEAD):
            self.scales = C.oracle_static_scales(orc, k, v, mode)
        if n:
            orc.store(self.g, self.img, 0, _bits(k), _bits(v), np.array(slots, np.int64), self.scales)
        elif self.scales is not None:
            orc.store(self.g, self.img, 0, np.zeros((0, hkv, hd), np.uint16), np.zeros((0, hkv, hd), np.uint16),
                      np.zeros(0, np.int64), self.scales)
        self.cfg = kvq.CacheConfig(bs, hkv, hd, [mode], [self.nblocks])
        self.cache = kvq.Cache(self.cfg, device=DEV, buffer=torch.from_numpy(self.img).to(DEV))
        if self.scales is not None:          # registers the static table (same bytes)
            e = torch.zeros((0, hkv, hd), dtype=torch.bfloat16, device=DEV)
            self.cache.store(0, e, e, torch.zeros(0, dtype=torch.int64, device=DEV), self.scales.tolist())
        gq = torch.Generator().manual_seed(seed + 7)
        self.q = torch.randn((len(self.lens), hkv * group, hd), generator=gq).to(torch.bfloat16)
        self.sm_scale = 1.0 / math.sqrt(hd)

    def run_gpu(self, bt=None, lens=None, q_scales=None):
        bt = self.bt if bt is None else bt
        lens = self.lens if lens is None else lens
        qs = None if q_scales is None else torch.as_tensor(q_scales, dtype=torch.float32).to(DEV)
        out = self.cache.decode_attention(0, self.q.to(DEV), torch.as_tensor(bt, dtype=torch.int32).to(DEV),
                                          torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV),
                                          self.sm_scale, q_scales=qs)
        torch.cuda.synchronize()
        return _f64(_bits(out))

    def reference(self, rows=None, bt=None, lens=None, q_scales=None):
        """Oracle output, weighted |V| sums and the tolerance, for sequences rows."""
        bt = self.bt if bt is None else bt
        lens = np.asarray(self.lens if lens is None else lens)
        rows = np.arange(len(lens)) if rows is None else np.asarray(rows)
        qb = _bits(self.q)[rows]
        ref, absv = self.orc.decode_attention(self.g, self.img, 0, qb, bt[rows], lens[rows], self.sm_scale,
                                              with_absv=True, q_scales=q_scales)
        v_big = 1.0 if self.scales is None else float(self.scales[len(self.scales) // 2:].max())
        tol = self.orc.attention_error_bound(self.g, self.img, 0, qb, bt[rows], lens[rows], self.sm_scale, ref, absv,
                                             v_big, q_scales=q_scales)
        return ref, tol

    def check(self, out, ref, tol, what):
        err = np.abs(out - ref)
        if not (err <= tol).all():
            i = np.unravel_index(np.argmax(err - tol), err.shape)
            pytest.fail(f"{what}: {(err > tol).sum()} of {err.size} outside the bound; worst at {i}: "
                        f"gpu {out[i]:.6g} oracle {ref[i]:.6g} bound {tol[i]:.3g}")

    def close(self):
        self.cache.close()


def _run(kvq, orc, what, **kw):
    _flush(f"[attention] {what}")
    sc = Scenario(kvq, orc, **kw)
    try:
        out = sc.run_gpu()
        ref, tol = sc.reference()
        sc.check(out, ref, tol, what)
        return sc, out, ref
    finally:
        sc.close()


MODES = [W.BF16, W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD]
RAGGED = [0, 1, 15, 16, 17, 100, 260]          # empty, single, partial and whole tiles


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("mode", MODES)
def test_attention_modes_and_head_dims(kvq, orc, mode, hd):
    """Several splits per sequence (maximum context 288 tokens)."""
    _run(kvq, orc, f"mode {W.MODE_NAMES[mode]} hd {hd} ragged", mode=mode, hd=hd, hkv=2, bs=16, lens=RAGGED,
         group=4, seed=hd + mode)


@pytest.mark.parametrize("mode", MODES)
def test_attention_single_split(kvq, orc, mode):
    """Contexts of at most 8 tiles: one split, output written by the first kernel."""
    _run(kvq, orc, f"mode {W.MODE_NAMES[mode]} single split", mode=mode, hd=128, hkv=2, bs=16,
         lens=[0, 1, 7, 16, 33, 100], group=4, seed=20 + mode)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 8, 9, 16, 20, 33])
def test_attention_query_groups(kvq, orc, group, hd):
    """Query heads per KV head below, at and above one 16-wide MFMA column block."""
    _run(kvq, orc, f"group {group} hd {hd}", mode=W.FP8_PER_TOKEN_HEAD, hd=hd, hkv=2, bs=16, lens=[5, 70, 200],
         group=group, seed=30 + group)


@pytest.mark.parametrize("hkv", [1, 3, 6, 12, 16])
def test_attention_kv_heads(kvq, orc, hkv):
    """KV-head counts that give 1, 2, 4 and 8 waves per workgroup and several head chunks."""
    _run(kvq, orc, f"hkv {hkv}", mode=W.FP8_PER_TOKEN_HEAD, hd=64, hkv=hkv, bs=16, lens=[3, 50, 129],
         group=2, seed=40 + hkv)


@pytest.mark.parametrize("hkv", [1, 8])
def test_attention_bf16_hd256_staged_tiles(kvq, orc, hkv):
    """BF16 at head_dim 256: 16 KiB tiles staged through LDS one per wave, with
    one (a tensor-parallel shard) and eight waves per workgroup; lengths that
    end inside, at and past whole tiles, several splits."""
    _run(kvq, orc, f"bf16 hd 256 hkv {hkv}", mode=W.BF16, hd=256, hkv=hkv, bs=16, lens=[3, 16, 50, 300, 515],
         group=4, seed=60 + hkv)


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 128])
@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD, W.BF16])
def test_attention_block_sizes(kvq, orc, mode, bs):
    """Blocks smaller than a 16-token tile (per-token block lookups) and larger ones."""
    _run(kvq, orc, f"mode {W.MODE_NAMES[mode]} bs {bs}", mode=mode, hd=64, hkv=2, bs=bs, lens=[1, 9, 40, 77],
         group=4, seed=50 + bs + mode)


def test_attention_heavy_tails(kvq, orc):
    """Student-t heads with large scores (a peaked softmax)."""
    n = 16 + 90 + 300
    k, v = W.heavy_tail_kv(n, 2, 128, seed=61)
    _run(kvq, orc, "heavy tails", mode=W.FP8_PER_TOKEN_HEAD, hd=128, hkv=2, bs=16, lens=[16, 90, 300],
         group=4, seed=60, kv=(k, v))


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD])
@pytest.mark.parametrize("hd", [64, 128])
def test_attention_extreme_value_scales(kvq, orc, mode, hd):
    """V rows whose absmax is near the BF16 maximum (scales above 2^124, whose
    16-fold overflows FP32), FP32-subnormal and BF16-subnormal ones, among
    ordinary rows; short sequences keep the weighted sums of the huge rows
    finite in FP32."""
    lens = [1, 5, 16]
    n = sum(lens)
    g = torch.Generator().manual_seed(140 + hd + mode)
    k = torch.randn((n, 2, hd), generator=g)
    v = torch.randn((n, 2, hd), generator=g)
    kinds = torch.randint(0, 4, (n, 2), generator=g)
    target = torch.tensor([1.0, 3.0e38, 1.0e-38, 2.0 ** -130])[kinds]
    v = v / v.abs().amax(dim=-1, keepdim=True) * target[..., None]
    _run(kvq, orc, f"extreme V scales mode {W.MODE_NAMES[mode]} hd {hd}", mode=mode, hd=hd, hkv=2, bs=16,
         lens=lens, group=4, seed=140 + hd, kv=(k.to(torch.bfloat16), v.to(torch.bfloat16)))


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.BF16, W.FP8_PER_HEAD])
def test_attention_skips_blocks_outside_the_layer(kvq, orc, mode):
    """Table entries that are negative or past the layer's blocks drop their
    tokens; a sequence left with none gives zeros."""
    _flush(f"[attention] foreign blocks mode {W.MODE_NAMES[mode]}")
    sc = Scenario(kvq, orc, mode=mode, hd=64, hkv=2, bs=16, lens=[70, 300, 40], group=4, seed=70)
    try:
        bt = sc.bt.copy()
        bt[0, 1] = -1
        bt[1, 3] = sc.nblocks
        bt[1, 10] = 2 ** 31 - 1
        bt[2, :] = -5
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, "foreign blocks")
        assert not out[2].any() and not ref[2].any()
    finally:
        sc.close()


def test_attention_lengths_clamped_to_the_table(kvq, orc):
    """Negative lengths count as 0; lengths past max_blocks * block_size are cut there."""
    _flush("[attention] clamped lengths")
    sc = Scenario(kvq, orc, mode=W.FP8_PER_TOKEN_HEAD, hd=64, hkv=2, bs=16, lens=[20, 40], group=2, seed=80)
    try:
        lens = [-3, 10 ** 6]
        out = sc.run_gpu(lens=lens)
        ref, tol = sc.reference(lens=lens)
        sc.check(out, ref, tol, "clamped lengths")
        assert not out[0].any()
    finally:
        sc.close()


@pytest.mark.parametrize("mode", [W.BF16, W.FP8_PER_TENSOR, W.FP8_PER_HEAD])
def test_attention_single_token_is_the_dequantized_value(kvq, orc, mode):
    """With one cached token and a static (or no) V scale the weight is exactly
    1, so the output is exactly the token's dequantized BF16 value."""
    _flush(f"[attention] single token mode {W.MODE_NAMES[mode]}")
    sc = Scenario(kvq, orc, mode=mode, hd=128, hkv=2, bs=16, lens=[1, 1, 1], group=3, seed=90)
    try:
        out = sc.run_gpu()
        _, vo = orc.gather(sc.g, sc.img, 0, sc.bt, sc.lens)
        want = np.repeat(_f64(vo), 3, axis=1)                     # [3 tokens, 6 query heads, hd]
        assert np.array_equal(out, want)
    finally:
        sc.close()


def test_attention_workspace_reuse_and_sizes(kvq, orc):
    """The workspace query matches what the call accepts: a smaller buffer is
    refused, an exact one gives the same bytes as a fresh allocation."""
    _flush("[attention] workspace")
    sc = Scenario(kvq, orc, mode=W.INT4_PER_TOKEN_HEAD, hd=128, hkv=2, bs=16, lens=[300, 500], group=4, seed=95)
    try:
        need = kvq.kvq_decode_attention_workspace(sc.cache.handle, 8, sc.maxb, 2)
        assert need > 0
        q = sc.q.to(DEV)
        bt = torch.as_tensor(sc.bt, dtype=torch.int32).to(DEV)
        sl = torch.as_tensor(sc.lens, dtype=torch.int32).to(DEV)
        out1 = torch.zeros_like(q)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)      # stale contents do not matter
        kvq.kvq_decode_attention(sc.cache.handle, 0, q, bt, sl, sc.sm_scale, out1, ws)
        with pytest.raises(kvq.KVQError) as e:
            kvq.kvq_decode_attention(sc.cache.handle, 0, q, bt, sl, sc.sm_scale, out1, ws[: need - 16])
        assert e.value.status == kvq.ERR_BUFFER_TOO_SMALL
        out2 = sc.cache.decode_attention(0, q, bt, sl, sc.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(out1, out2)
    finally:
        sc.close()


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 128), (W.INT4_PER_TOKEN_HEAD, 128),
                                     (W.INT4_PER_TOKEN_HEAD, 64), (W.FP8_PER_TOKEN_HEAD, 64)],
                         ids=["fp8_per_token_head-128", "int4_per_token_head-128", "int4_per_token_head-64",
                              "fp8_per_token_head-64"])
def test_attention_decode_workload_sampled(kvq, orc, mode, hd):
    """Full decode shape: 256 sequences of 8192-8207 cached tokens, 8 KV heads,
    32 query heads, per-token-head FP8 and INT4 at head_dim 128 and 64 (at 64
    the quad path), in the launch configuration the benchmark times; eight
    sampled sequences against the oracle."""
    _flush(f"[attention] decode 256 x 8192 {W.MODE_NAMES[mode]} hd {hd} (sampled)")
    g = torch.Generator().manual_seed(11)
    lens = (8192 + torch.randint(0, 16, (256,), generator=g)).tolist()
    n = sum(lens)
    k, v = (t.cpu() for t in W.normal_kv(n, 8, hd, seed=12, device=DEV))
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=8, bs=16, lens=lens, group=4, seed=13,
                  extra_blocks=0, kv=(k, v))
    del k, v
    try:
        assert sc.maxb == 514
        out = sc.run_gpu()
        rows = [0, 1, 77, 128, 200, 254, 255, 31]
        ref, tol = sc.reference(rows=rows)
        sc.check(out[rows], ref, tol, "decode sampled")
    finally:
        sc.close()


# the tile-quad kernel's layers (workgroups of one or two KV heads)
TQUAD_CASES = [(W.FP8_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 128),
               (W.FP8_PER_TOKEN_HEAD, 128)]
TQUAD_IDS = ["fp8_per_token_head-hd64", "int4_per_token_head-hd64", "int4_per_token_head-hd128",
             "fp8_per_token_head-hd128"]


@pytest.mark.parametrize("hkv", [1, 2], ids=["tp8-hkv1", "tp4-hkv2"])
@pytest.mark.parametrize("mode,hd", TQUAD_CASES, ids=TQUAD_IDS)
def test_attention_tensor_parallel_shard_sampled(kvq, orc, mode, hd, hkv):
    """The decode shape at one tensor-parallel shard's share of the heads (1
    or 2 of the 8 KV heads, their 4 or 8 query heads; 256 sequences of
    8192-8207 cached tokens), the tile-quad kernel in the launch configuration
    the benchmark's --tp 8 and --tp 4 lines time; eight sampled sequences
    against the oracle."""
    _flush(f"[attention] shard decode 256 x 8192 {W.MODE_NAMES[mode]} hd {hd} hkv {hkv} (sampled)")
    g = torch.Generator().manual_seed(31)
    lens = (8192 + torch.randint(0, 16, (256,), generator=g)).tolist()
    k, v = (t.cpu() for t in W.normal_kv(sum(lens), hkv, hd, seed=32 + hkv, device=DEV))
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=hkv, bs=16, lens=lens, group=4, seed=33 + hkv,
                  extra_blocks=0, kv=(k, v))
    del k, v
    try:
        out = sc.run_gpu()
        rows = [0, 3, 64, 127, 128, 190, 254, 255]
        ref, tol = sc.reference(rows=rows)
        sc.check(out[rows], ref, tol, "shard decode sampled")
    finally:
        sc.close()


# the head-quad kernel serves the per-token-head layers; the static layouts
# take the packed rounds of the one-head kernel on the same shapes
QUAD_MODES = [W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD]


@pytest.mark.parametrize("hkv,group,bs", [(4, 4, 16), (8, 4, 16), (8, 1, 32), (12, 3, 16), (16, 2, 128), (8, 2, 16)],
                         ids=["hkv4-g4", "hkv8-g4", "hkv8-g1-bs32", "hkv12-g3", "hkv16-g2-bs128", "hkv8-g2"])
@pytest.mark.parametrize("mode", QUAD_MODES, ids=[W.MODE_NAMES[m] for m in QUAD_MODES])
def test_attention_head_quads(kvq, orc, mode, hkv, group, bs):
    """Head_dim 64 with at most 4 query heads per KV head and 4 or 8 KV heads
    per workgroup.  Per-token-head layers take the head-quad kernel: each
    wave serves a quad of 4 KV heads (16 columns of 4 heads x 4 queries), the
    quad's 4 waves take every fourth tile and merge through LDS; static
    layers take the packed rounds on the same shapes.  Lengths leave some
    waves of a quad without a tile (1 to 3 tiles), end inside and at tile
    and block boundaries, and run to several splits."""
    lens = [0, 1, 15, 16, 17, 33, 48, 49, 100, 260, 600]
    _run(kvq, orc, f"quads mode {W.MODE_NAMES[mode]} hkv {hkv} group {group} bs {bs}", mode=mode, hd=64, hkv=hkv,
         bs=bs, lens=lens, group=group, seed=200 + hkv * 10 + group + mode)


@pytest.mark.parametrize("hkv,group,bs", [(4, 4, 16), (8, 4, 16), (8, 1, 32), (12, 3, 16), (16, 2, 128)],
                         ids=["hkv4-g4", "hkv8-g4", "hkv8-g1-bs32", "hkv12-g3", "hkv16-g2-bs128"])
def test_attention_head_quads_int4_hd128(kvq, orc, hkv, group, bs):
    """INT4 at head_dim 128 takes the quad kernel too (8 KiB quad tiles):
    the same lengths and shapes as at head_dim 64."""
    lens = [0, 1, 15, 16, 17, 33, 48, 49, 100, 260, 600]
    _run(kvq, orc, f"quads int4 hd128 hkv {hkv} group {group} bs {bs}", mode=W.INT4_PER_TOKEN_HEAD, hd=128,
         hkv=hkv, bs=bs, lens=lens, group=group, seed=260 + hkv * 10 + group)


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 64),
                                     (W.INT4_PER_TOKEN_HEAD, 128)],
                         ids=["fp8_per_token_head-hd64", "int4_per_token_head-hd64", "int4_per_token_head-hd128"])
def test_attention_head_quads_single_split_and_foreign_blocks(kvq, orc, mode, hd):
    """The quad path with one split (the first kernel writes the output),
    table entries outside the layer, and clamped lengths."""
    _flush(f"[attention] quads single split, foreign blocks {W.MODE_NAMES[mode]} hd {hd}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=8, bs=16, lens=[70, 120, 40, 3], group=4, seed=230 + mode + hd)
    try:
        out = sc.run_gpu()
        ref, tol = sc.reference()
        sc.check(out, ref, tol, "quads single split")
        bt = sc.bt.copy()
        bt[0, 1] = -1
        bt[1, 3] = sc.nblocks
        bt[2, :] = -5
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, "quads foreign blocks")
        assert not out[2].any() and not ref[2].any()
        lens = [-3, 10 ** 6, 40, 0]
        out = sc.run_gpu(lens=lens)
        ref, tol = sc.reference(lens=lens)
        sc.check(out, ref, tol, "quads clamped lengths")
        assert not out[0].any() and not out[3].any()
    finally:
        sc.close()


def test_attention_head_quads_layer_without_blocks(kvq, orc):
    """A layer with no blocks gives zeros on the quad path too."""
    _flush("[attention] quads, layer without blocks")
    cfg = kvq.CacheConfig(16, 8, 64, [W.INT4_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD], [4, 0])
    cache = kvq.Cache(cfg, device=DEV)
    try:
        for maxb in (2, 64):
            q = torch.randn((3, 32, 64), generator=torch.Generator().manual_seed(maxb)).to(torch.bfloat16).to(DEV)
            bt = torch.zeros((3, maxb), dtype=torch.int32, device=DEV)
            sl = torch.tensor([5, 0, 20], dtype=torch.int32, device=DEV)
            out = torch.full_like(q, 1.0)
            cache.decode_attention(1, q, bt, sl, 0.125, out=out)
            torch.cuda.synchronize()
            assert not out.any()
    finally:
        cache.close()


def test_attention_layer_without_blocks_gives_zeros(kvq, orc):
    """A layer configured with no blocks has no token to attend to."""
    _flush("[attention] layer without blocks")
    cfg = kvq.CacheConfig(16, 2, 64, [W.FP8_PER_TOKEN_HEAD, W.FP8_PER_TOKEN_HEAD], [4, 0])
    cache = kvq.Cache(cfg, device=DEV)
    try:
        for maxb in (2, 64):                                  # one split, several splits
            q = torch.randn((3, 4, 64), generator=torch.Generator().manual_seed(maxb)).to(torch.bfloat16).to(DEV)
            bt = torch.zeros((3, maxb), dtype=torch.int32, device=DEV)
            sl = torch.tensor([5, 0, 20], dtype=torch.int32, device=DEV)
            out = torch.full_like(q, 1.0)
            cache.decode_attention(1, q, bt, sl, 0.125, out=out)
            torch.cuda.synchronize()
            assert not out.any()
    finally:
        cache.close()


def _query_scales(q, shrink):
    """Static per-query-head scales amax/448 of the queries, divided by shrink
    (shrink > 1 makes the largest elements saturate at 448)."""
    amax = q.float().abs().amax(dim=(0, 2)).numpy().astype(np.float32)
    return (amax / np.float32(448.0) / np.float32(shrink)).astype(np.float32)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("mode", [W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD])
@pytest.mark.parametrize("shrink", [1.0, 4.0])
def test_fp8_query_attention(kvq, orc, mode, hd, shrink):
    """FP8 queries under static per-query-head scales, on the FP8 products."""
    what = f"fp8 query mode {W.MODE_NAMES[mode]} hd {hd} shrink {shrink}"
    _flush(f"[attention] {what}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=2, bs=16, lens=RAGGED, group=4, seed=100 + hd + mode)
    try:
        qs = _query_scales(sc.q, shrink)
        out = sc.run_gpu(q_scales=qs)
        ref, tol = sc.reference(q_scales=qs)
        sc.check(out, ref, tol, what)
        # the queries really are quantized: against BF16 queries the result moves
        plain, _ = sc.reference()
        assert np.abs(ref - plain).max() > 0
    finally:
        sc.close()


@pytest.mark.parametrize("hkv,group,bs", [(1, 4, 16), (2, 4, 16), (3, 3, 32), (6, 2, 16), (1, 1, 128), (2, 2, 64)],
                         ids=["hkv1-g4", "hkv2-g4", "hkv3-g3-bs32", "hkv6-g2", "hkv1-g1-bs128", "hkv2-g2-bs64"])
@pytest.mark.parametrize("mode,hd", TQUAD_CASES, ids=TQUAD_IDS)
def test_attention_tile_quads(kvq, orc, mode, hd, hkv, group, bs):
    """Workgroups of one or two KV heads (a tensor-parallel shard, few-head
    models): 4 consecutive tiles of one head share a wave's 16 columns (4
    waves per head, 8 for INT4), or 2 tiles of a pair of heads (the pair's 8
    waves); the waves take every fourth or eighth round and merge their
    partial states per query.  Lengths end inside a round, at tile and block
    boundaries, leave waves without a round, and run to several splits."""
    lens = [0, 1, 15, 16, 17, 33, 48, 49, 64, 65, 100, 130, 260, 600]
    _run(kvq, orc, f"tile quads mode {W.MODE_NAMES[mode]} hd {hd} hkv {hkv} group {group} bs {bs}", mode=mode,
         hd=hd, hkv=hkv, bs=bs, lens=lens, group=group, seed=400 + hkv * 10 + group + mode + hd)


@pytest.mark.parametrize("mode,hd", TQUAD_CASES, ids=TQUAD_IDS)
def test_attention_tile_quads_single_split_foreign_blocks_and_long(kvq, orc, mode, hd):
    """Tile quads with one split (the first kernel writes the output), table
    entries outside the layer inside a round, clamped lengths, and one long
    sequence over dozens of split ranges (the wide combine)."""
    _flush(f"[attention] tile quads single split, foreign blocks {W.MODE_NAMES[mode]} hd {hd}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=1, bs=16, lens=[70, 120, 40, 3], group=4, seed=450 + mode + hd)
    try:
        out = sc.run_gpu()
        ref, tol = sc.reference()
        sc.check(out, ref, tol, "tile quads single split")
        bt = sc.bt.copy()
        bt[0, 1] = -1
        bt[1, 3] = sc.nblocks
        bt[1, 5] = -2
        bt[2, :] = -5
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, "tile quads foreign blocks")
        assert not out[2].any() and not ref[2].any()
        lens = [-3, 10 ** 6, 40, 0]
        out = sc.run_gpu(lens=lens)
        ref, tol = sc.reference(lens=lens)
        sc.check(out, ref, tol, "tile quads clamped lengths")
        assert not out[0].any() and not out[3].any()
    finally:
        sc.close()
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=2, bs=16, lens=[6001], group=4, seed=460 + mode + hd)
    try:
        bt = sc.bt.copy()
        bt[0, 40:48] = -1
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, "tile quads one long sequence")
    finally:
        sc.close()


@pytest.mark.parametrize("shrink", [1.0, 4.0])
@pytest.mark.parametrize("hkv,group", [(1, 4), (2, 3)], ids=["hkv1-g4", "hkv2-g3"])
def test_fp8_query_tile_quads(kvq, orc, hkv, group, shrink):
    """FP8 queries on the tile quads (per-token-head FP8, head_dim 64): one KV
    head, and two as a head pair."""
    what = f"fp8 query tile quads hkv {hkv} group {group} shrink {shrink}"
    _flush(f"[attention] {what}")
    lens = [0, 1, 17, 49, 65, 130, 600]
    sc = Scenario(kvq, orc, mode=W.FP8_PER_TOKEN_HEAD, hd=64, hkv=hkv, bs=16, lens=lens, group=group,
                  seed=470 + hkv * 10 + group)
    try:
        qs = _query_scales(sc.q, shrink)
        out = sc.run_gpu(q_scales=qs)
        ref, tol = sc.reference(q_scales=qs)
        sc.check(out, ref, tol, what)
    finally:
        sc.close()


@pytest.mark.parametrize("hkv,group,bs", [(4, 4, 16), (8, 3, 32), (12, 2, 16), (8, 1, 16)],
                         ids=["hkv4-g4", "hkv8-g3-bs32", "hkv12-g2", "hkv8-g1"])
@pytest.mark.parametrize("mode", [W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD])
@pytest.mark.parametrize("shrink", [1.0, 4.0])
def test_fp8_query_head_quads(kvq, orc, mode, hkv, group, bs, shrink):
    """FP8 queries at head_dim 64 with groups of at most 4 and 4 or 8 KV heads
    per workgroup: per-token-head layers take the head-quad kernel
    (block-diagonal FP8 query codes through the FP8 products), static ones
    the packed rounds; ragged lengths over several splits."""
    what = f"fp8 query quads mode {W.MODE_NAMES[mode]} hkv {hkv} group {group} bs {bs} shrink {shrink}"
    _flush(f"[attention] {what}")
    lens = [0, 1, 15, 16, 17, 33, 48, 49, 100, 260, 600]
    sc = Scenario(kvq, orc, mode=mode, hd=64, hkv=hkv, bs=bs, lens=lens, group=group,
                  seed=300 + hkv * 10 + group + mode)
    try:
        qs = _query_scales(sc.q, shrink)
        out = sc.run_gpu(q_scales=qs)
        ref, tol = sc.reference(q_scales=qs)
        sc.check(out, ref, tol, what)
    finally:
        sc.close()


@pytest.mark.parametrize("hd", [128, 64])
def test_fp8_query_decode_workload_sampled(kvq, orc, hd):
    """FP8 queries on the full decode shape (256 x 8192-8207 tokens, 32/8 heads,
    head_dim 128 and 64 (head quads), per-token-head FP8), eight sequences
    against the oracle."""
    _flush(f"[attention] fp8 query decode 256 x 8192 hd {hd} (sampled)")
    g = torch.Generator().manual_seed(21)
    lens = (8192 + torch.randint(0, 16, (256,), generator=g)).tolist()
    k, v = (t.cpu() for t in W.normal_kv(sum(lens), 8, hd, seed=22, device=DEV))
    sc = Scenario(kvq, orc, mode=W.FP8_PER_TOKEN_HEAD, hd=hd, hkv=8, bs=16, lens=lens, group=4, seed=23,
                  extra_blocks=0, kv=(k, v))
    del k, v
    try:
        qs = _query_scales(sc.q, 1.0)
        out = sc.run_gpu(q_scales=qs)
        rows = [0, 5, 99, 128, 201, 255, 17, 64]
        ref, tol = sc.reference(rows=rows, q_scales=qs)
        sc.check(out[rows], ref, tol, "fp8 query decode sampled")
    finally:
        sc.close()


@pytest.mark.parametrize("mode,hd,group", [(W.BF16, 64, 8), (W.FP8_PER_TOKEN_HEAD, 128, 8),
                                           (W.INT4_PER_TOKEN_HEAD, 64, 4), (W.INT4_PER_TOKEN_HEAD, 128, 4)],
                         ids=["bf16-hd64-g8", "fp8-hd128-g8", "int4-hd64-g4-tquads", "int4-hd128-g4-tquads"])
def test_attention_hundreds_of_splits(kvq, orc, mode, hd, group):
    """One sequence of 40000 tokens on one KV head: the one-head kernel (groups
    of 8) takes 313 split ranges of 8 tiles, more than the wide merge's 256
    threads hold in one pass of (m, l) pairs and several passes of its O
    loads; the 8-wave INT4 tile quads (groups of 4) take 125 ranges of 20
    tiles.  Every query head against the oracle."""
    what = f"hundreds of splits mode {W.MODE_NAMES[mode]} hd {hd} group {group}"
    _flush(f"[attention] {what}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=1, bs=16, lens=[40000], group=group, seed=170 + hd + mode)
    try:
        bt = sc.bt.copy()
        bt[0, 1000:1003] = -1                # three blocks of one range take no part
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, what)
    finally:
        sc.close()


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.BF16, W.INT4_PER_TOKEN_HEAD])
def test_attention_one_long_sequence(kvq, orc, mode, hd):
    """Batch 1: a single long sequence split into dozens of ranges, merged by
    the workgroup-wide combine; one range's blocks are outside the layer."""
    what = f"one long sequence mode {W.MODE_NAMES[mode]} hd {hd}"
    _flush(f"[attention] {what}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=2, bs=16, lens=[6001], group=8, seed=130 + hd + mode)
    try:
        bt = sc.bt.copy()
        bt[0, 40:48] = -1                    # 128 tokens of one split range take no part
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, what)
    finally:
        sc.close()


@pytest.mark.parametrize("mode,hd", [(W.FP8_PER_TOKEN_HEAD, 64), (W.INT4_PER_TOKEN_HEAD, 64),
                                     (W.INT4_PER_TOKEN_HEAD, 128)],
                         ids=["fp8_per_token_head-hd64", "int4_per_token_head-hd64", "int4_per_token_head-hd128"])
def test_attention_head_quads_one_long_sequence(kvq, orc, mode, hd):
    """Batch 1 on the head-quad kernel: one sequence of 8 KV heads split into
    dozens of ranges (the workgroup-wide combine merges the quads'
    partials); one range's blocks are outside the layer."""
    what = f"quads one long sequence mode {W.MODE_NAMES[mode]} hd {hd}"
    _flush(f"[attention] {what}")
    sc = Scenario(kvq, orc, mode=mode, hd=hd, hkv=8, bs=16, lens=[6001], group=4, seed=150 + hd + mode)
    try:
        bt = sc.bt.copy()
        bt[0, 40:48] = -1
        out = sc.run_gpu(bt=bt)
        ref, tol = sc.reference(bt=bt)
        sc.check(out, ref, tol, what)
    finally:
        sc.close()
