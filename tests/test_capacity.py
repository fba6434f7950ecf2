"""Byte accounting against the numbers printed on the pages
(tests/golden/capacity_pins.txt), computed both by the oracle's own layout and
by the library's kvq_cache_bytes (pure host arithmetic, no GPU needed)."""
import pytest

import workloads as W
from tests._golden import load as load_golden

GiB, MiB, KiB = 1 << 30, 1 << 20, 1 << 10
G = load_golden("capacity_pins.txt")


def _oracle_bytes(orc):
    def f(bs, hkv, hd, modes, nblocks):
        return orc.cache_bytes(orc.Geometry(bs, hkv, hd, modes, nblocks))
    return f


def _library_bytes():
    import quantized_fp8_int4_amd as kvq

    def f(bs, hkv, hd, modes, nblocks):
        return kvq.kvq_cache_bytes(kvq.CacheConfig(bs, hkv, hd, modes, nblocks))
    return f


@pytest.fixture(params=["oracle", "library"])
def cache_bytes(request, orc):
    if request.param == "oracle":
        return _oracle_bytes(orc)
    return _library_bytes()


def test_80_layer_128k_example(cache_bytes):
    """80 layers, 8 KV heads, head_dim 128, 131072 tokens (blocks of 16)."""
    L, nb = 80, 131072 // 16
    dyn = cache_bytes(16, 8, 128, [W.FP8_PER_TOKEN_HEAD] * L, [nb] * L)
    assert dyn["payload"] == G["p1_fp8_payload_80L_128K_GiB"] * GiB
    assert dyn["token_scales"] == G["p1_scales_80L_128K_MiB"] * MiB
    assert dyn["total"] == G["p1_total_80L_128K_GiB"] * GiB
    assert dyn["padding"] == 0 and dyn["static_scales"] == 0
    pairs = L * 8 * 131072
    assert dyn["payload"] / pairs == G["p1_token_head_data_bytes_hd128"]
    assert dyn["token_scales"] / pairs == G["p1_token_head_scale_bytes"]
    assert 100 * dyn["token_scales"] / dyn["payload"] == G["p1_scale_tax_hd128_percent"]
    bf = cache_bytes(16, 8, 128, [W.BF16] * L, [nb] * L)
    assert bf["total"] == G["p1_bf16_80L_128K_GiB"] * GiB
    pt = cache_bytes(16, 8, 128, [W.FP8_PER_TENSOR] * L, [nb] * L)
    ph = cache_bytes(16, 8, 128, [W.FP8_PER_HEAD] * L, [nb] * L)
    assert pt["static_scales"] == G["p1_static_per_tensor_80L_bytes"]
    assert ph["static_scales"] == G["p1_static_per_head_80L_bytes"]
    assert ph["total"] - pt["total"] == G["p1_static_difference_80L_bytes"]
    assert pt["payload"] == ph["payload"] == G["p1_fp8_payload_80L_128K_GiB"] * GiB


@pytest.mark.parametrize("hd,data_key,tax_key", [
    (64, "p1_token_head_data_bytes_hd64", "p1_scale_tax_hd64_percent"),
    (256, None, "p1_scale_tax_hd256_percent"),
])
def test_scale_tax_other_head_dims(cache_bytes, hd, data_key, tax_key):
    r = cache_bytes(16, 8, hd, [W.FP8_PER_TOKEN_HEAD], [100])
    pairs = 100 * 16 * 8
    if data_key:
        assert r["payload"] / pairs == G[data_key]
    assert 100 * r["token_scales"] / r["payload"] == G[tax_key]


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_fp8_tax_is_4_over_head_size(cache_bytes, hd):
    r = cache_bytes(16, 8, hd, [W.FP8_PER_TOKEN_HEAD] * 4, [10] * 4)
    assert r["token_scales"] / r["payload"] == 4 / hd
    pct = {64: "p2_fp8_tax_hd64_percent", 128: "p2_fp8_tax_hd128_percent", 256: "p2_fp8_tax_hd256_percent"}
    assert 100 * 4 / hd == G[pct[hd]]


@pytest.mark.parametrize("hd,key", [(128, "p2_int4_tax_hd128_percent"), (64, "p2_int4_tax_hd64_percent")])
def test_int4_tax_is_8_over_head_size(cache_bytes, hd, key):
    r = cache_bytes(16, 8, hd, [W.INT4_PER_TOKEN_HEAD] * 4, [10] * 4)
    assert r["token_scales"] / r["payload"] == 8 / hd
    assert 100 * r["token_scales"] / r["payload"] == G[key]
    assert r["payload"] == 4 * 10 * 16 * 8 * hd      # packed K and V: hd bytes per pair


def test_32_layer_gqa_per_token(cache_bytes):
    """One retained token of the 32-layer, 8-KV-head, head_dim-128 model."""
    r = cache_bytes(1, 8, 128, [W.FP8_PER_TOKEN_HEAD] * 32, [1] * 32)
    assert r["payload"] == G["p2_fp8_payload_per_token_32L_bytes"] == G["p2_fp8_payload_per_token_32L_KiB"] * KiB
    assert r["token_scales"] == G["p2_scales_per_token_32L_bytes"] == G["p2_scales_per_token_32L_KiB"] * KiB
    per_token = r["payload"] + r["token_scales"]       # before block-level rounding
    assert per_token == G["p2_total_per_token_32L_KiB"] * KiB
    bf = cache_bytes(1, 8, 128, [W.BF16] * 32, [1] * 32)
    assert bf["payload"] == G["p2_bf16_per_token_32L_KiB"] * KiB
    assert round(bf["payload"] / per_token, 2) == G["p2_compression_vs_bf16_32L"]


def test_32_layer_gqa_128k_and_blocks(cache_bytes):
    nb = 131072 // 16
    r = cache_bytes(16, 8, 128, [W.FP8_PER_TOKEN_HEAD] * 32, [nb] * 32)
    assert r["payload"] == G["p2_fp8_payload_32L_128Ki_GiB"] * GiB
    assert r["token_scales"] == G["p2_scales_32L_128Ki_MiB"] * MiB
    assert r["total"] == G["p2_total_32L_128Ki_GiB"] * GiB
    bf = cache_bytes(16, 8, 128, [W.BF16] * 32, [nb] * 32)
    assert bf["total"] == G["p2_bf16_32L_128Ki_GiB"] * GiB
    one_block = cache_bytes(16, 8, 128, [W.FP8_PER_TOKEN_HEAD] * 32, [1] * 32)
    assert one_block["total"] == G["p2_block16_32L_KiB"] * KiB
    ph = cache_bytes(16, 8, 128, [W.FP8_PER_HEAD] * 32, [nb] * 32)
    assert ph["static_scales"] == G["p2_static_per_head_32L_bytes"]


def test_static_per_head_worksheet(cache_bytes):
    """The pages count H query-head scales too; Q is not cached, so the cache
    holds the 2*Hkv K/V part and the query part is added here as 4*H bytes."""
    H, hkv = 64, 8
    ph = cache_bytes(16, hkv, 64, [W.FP8_PER_HEAD], [1])["static_scales"]
    pt = cache_bytes(16, hkv, 64, [W.FP8_PER_TENSOR], [1])["static_scales"]
    assert (ph + 4 * H) // 4 == G["p3_static_scale_values_H64_Hkv8"]
    assert ph + 4 * H == G["p3_static_scale_bytes_H64_Hkv8"]
    assert (ph + 4 * H) - (pt + 4) == G["p3_static_extra_bytes_H64_Hkv8"]
    ph24 = cache_bytes(16, hkv, 64, [W.FP8_PER_HEAD] * 24, [1] * 24)["static_scales"]
    pt24 = cache_bytes(16, hkv, 64, [W.FP8_PER_TENSOR] * 24, [1] * 24)["static_scales"]
    assert (ph24 + 24 * 4 * H) - (pt24 + 24 * 4) == G["p3_static_extra_bytes_24L"]


def _gptoss(full_mode, sliding_mode):
    modes, nb = [], []
    for layer in range(24):
        if W.gptoss_layer_is_sliding(layer):
            modes.append(sliding_mode)
            nb.append(128 // 16)
        else:
            modes.append(full_mode)
            nb.append(32768 // 16)
    return modes, nb


def test_gptoss_layer_skipping(cache_bytes):
    modes, nb = _gptoss(W.FP8_PER_TENSOR, W.BF16)
    A = sum(n * 16 for n in nb)
    S = sum(n * 16 for n, m in zip(nb, modes) if m == W.BF16)
    assert sum(n * 16 for n, m in zip(nb, modes) if m != W.BF16) == G["p3_gptoss_full_positions"]
    assert A == G["p3_gptoss_A"] and S == G["p3_gptoss_S"]
    all_bf16 = cache_bytes(16, 8, 64, [W.BF16] * 24, nb)
    all_fp8 = cache_bytes(16, 8, 64, [W.FP8_PER_TENSOR] * 24, nb)
    skip = cache_bytes(16, 8, 64, modes, nb)
    assert all_bf16["payload"] / A == G["p3_gptoss_bf16_bytes_per_position"]
    assert all_bf16["payload"] / MiB == G["p3_gptoss_all_bf16_MiB"]
    assert all_fp8["payload"] / MiB == G["p3_gptoss_all_fp8_MiB"]
    assert skip["payload"] / MiB == G["p3_gptoss_skip_sliding_MiB"]
    assert (skip["payload"] - all_fp8["payload"]) / MiB == G["p3_gptoss_skip_cost_MiB"]
    ratio = all_bf16["payload"] / skip["payload"]
    assert ratio == 2 * A / (A + S)
    assert round(ratio, 3) == G["p3_gptoss_compression"]
    # With per-token-head scales on the full layers the scale bytes are added
    # (the pages' ratio leaves them out on purpose).
    dyn_modes, _ = _gptoss(W.FP8_PER_TOKEN_HEAD, W.BF16)
    dyn = cache_bytes(16, 8, 64, dyn_modes, nb)
    assert dyn["total"] == 430964736 == 411 * MiB
    assert round(all_bf16["payload"] / dyn["total"], 3) == 1.876


def test_half_skipped_equal_retention(cache_bytes):
    mixed = cache_bytes(16, 8, 128, [W.BF16, W.FP8_PER_TENSOR], [64, 64])
    bf = cache_bytes(16, 8, 128, [W.BF16, W.BF16], [64, 64])
    assert round(bf["payload"] / mixed["payload"], 2) == G["p3_half_skipped_equal_retention_ratio"]


def test_layer_bases_are_256_byte_aligned(orc):
    g = orc.Geometry(1, 1, 64, [W.INT4_PER_TOKEN_HEAD, W.FP8_PER_HEAD, W.BF16], [3, 5, 1])
    lb, sb, total = orc.layer_offsets(g)
    assert list(lb) == [0, 256, 1024]            # 3*72=216 -> 256; 256+5*128=896 -> 1024
    assert sb[1] == 1280 and total == 1280 + 8
