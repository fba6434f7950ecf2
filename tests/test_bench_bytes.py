"""The benchmark's algorithmic-byte formulas (what every roofline figure
divides by) against the byte counts written out by hand: per token-head, a
store reads 4 hd bytes of BF16 K and V and the slot (8 bytes shared by the
token's KV heads) and writes 2 row_bytes of codes plus 8 bytes of scales in
per-token-head modes; a gather reads the codes, scales and the block-table
entry (4 bytes per block per KV head) and writes 4 hd bytes of BF16."""
import pytest

import bench

FP8_PTH, INT4_PTH, FP8_PT, BF16 = 3, 4, 1, 0


@pytest.mark.parametrize("mode,hd,store,gather", [
    (FP8_PTH, 128, 777, 776.03125),
    (FP8_PTH, 64, 393, 392.03125),
    (FP8_PT, 128, 769, 768.03125),
    (INT4_PTH, 128, 649, 648.03125),
    (INT4_PTH, 64, 329, 328.03125),
    (BF16, 64, 513, 512.03125),
])
def test_bytes_per_token_head(mode, hd, store, gather):
    s, g = bench.algorithmic_bytes(mode, hd, 8, 16, 1)
    assert s == pytest.approx(store, abs=1e-9)
    assert g == pytest.approx(gather, abs=1e-9)


def test_per_launch_totals_of_the_workloads():
    # GQA-32 layer call: 32768 tokens x 8 KV heads
    s, g = bench.algorithmic_bytes(FP8_PTH, 128, 8, 16, 32768 * 8)
    assert s == 203_685_888 and g == 203_431_936
    # one tensor-parallel shard's share at one KV head: the slot is one head's alone
    s, _ = bench.algorithmic_bytes(FP8_PTH, 128, 1, 16, 32768)
    assert s == 32768 * (512 + 256 + 8 + 8)
    # long context layer: 131072 tokens x 8 KV heads
    s, _ = bench.algorithmic_bytes(FP8_PTH, 128, 8, 16, 131072 * 8)
    assert s == 131072 * 8 * 777


def test_attention_bytes_of_one_launch():
    # 2 sequences, 40 cached tokens in all, 8 KV heads, 32 query heads, hd 128, FP8 per-token-head:
    # codes and scales of every token-head, ceil(40 / 16) block-table entries, BF16 q and out
    assert bench.attention_bytes(FP8_PTH, 128, 8, 16, 32, 2, 40) == 40 * 8 * (256 + 8) + 3 * 4 + 2 * 32 * 128 * 4
    # INT4 at head_dim 64 halves the rows: 32 code bytes each, the same 8 scale bytes
    assert bench.attention_bytes(INT4_PTH, 64, 8, 16, 32, 1, 16) == 16 * 8 * (64 + 8) + 4 + 32 * 64 * 4


@pytest.mark.parametrize("name", ["fp8_per_token_head", "fp8_per_tensor", "fp8_per_head", "int4_per_token_head"])
def test_layout_geometry_matches_the_cache_layout(orc, name):
    """The layer bases the store-pattern ceiling writes at are the cache
    layout's (the oracle's own offsets), and its last layer ends inside a
    buffer of kvq_cache_bytes().total, so the ceiling kernel stays in bounds."""
    import quantized_fp8_int4_amd as kvq
    import workloads as W
    spec = W.WORKLOADS["gqa32"]
    L, hkv, hd, bs = spec["num_layers"], spec["hkv"], spec["hd"], spec["block_size"]
    n = spec["num_seqs"] * spec["seq_len"]
    I = dict(L=L, hkv=hkv, hd=hd, bs=bs, n=n, nblocks=n // bs)
    geo = bench.layout_geometry(kvq, W, I, name)
    g = orc.Geometry(bs, hkv, hd, [geo["mode"]] * L, [n // bs] * L)
    assert [int(x) for x in orc.layer_offsets(g)[0]] == geo["layer_base"]
    block = bs * hkv * (2 * bench.row_bytes(geo["mode"], hd) + (8 if geo["dynamic"] else 0))
    total = kvq.kvq_cache_bytes(kvq.CacheConfig(bs, hkv, hd, [geo["mode"]] * L, [n // bs] * L))["total"]
    assert geo["layer_base"][-1] + (n // bs) * block <= total
