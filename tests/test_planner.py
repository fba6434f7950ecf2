"""Capacity planner (kvq_plan_capacity, host code) against the numbers the
pages print (tests/golden/capacity_pins.txt) and against the oracle's own
planner, which prices blocks with the oracle's independent layout."""
import pytest

import workloads as W
from tests._golden import load as load_golden

GiB, MiB, KiB = 1 << 30, 1 << 20, 1 << 10
G = load_golden("capacity_pins.txt")


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    return kvq


def _gptoss(full_mode, sliding_mode):
    modes = [sliding_mode if W.gptoss_layer_is_sliding(l) else full_mode for l in range(24)]
    wins = [128 if W.gptoss_layer_is_sliding(l) else 0 for l in range(24)]
    return modes, wins


def _both(kvq, orc, bs, hkv, hd, modes, wins, context, pool):
    lib, blocks = kvq.kvq_plan_capacity(kvq.ModelConfig(bs, hkv, hd, modes, wins), context, pool)
    ref = orc.plan_capacity(bs, hkv, hd, modes, wins, context, pool)
    for k in ("retained_positions", "skipped_positions", "sequence_bytes", "max_sequences", "max_tokens",
              "buffer_bytes"):
        assert lib[k] == ref[k], k
    assert blocks == ref["layer_num_blocks"]
    return lib, blocks


def test_gptoss_retention_and_compression(kvq, orc):
    """24 alternating layers, 8 KV heads, head_dim 64, window 128, one 32,768-token sequence."""
    skip, wins = _gptoss(W.FP8_PER_TENSOR, W.BF16)
    p, _ = _both(kvq, orc, 16, 8, 64, skip, wins, 32768, 1 << 40)
    assert p["retained_positions"] == G["p3_gptoss_A"] and p["skipped_positions"] == G["p3_gptoss_S"]
    A, S = p["retained_positions"], p["skipped_positions"]
    assert p["sequence_bytes"] / MiB == G["p3_gptoss_skip_sliding_MiB"]
    fp8, _ = _both(kvq, orc, 16, 8, 64, [W.FP8_PER_TENSOR] * 24, wins, 32768, 1 << 40)
    bf16, _ = _both(kvq, orc, 16, 8, 64, [W.BF16] * 24, wins, 32768, 1 << 40)
    assert fp8["sequence_bytes"] / MiB == G["p3_gptoss_all_fp8_MiB"]
    assert bf16["sequence_bytes"] / MiB == G["p3_gptoss_all_bf16_MiB"]
    assert bf16["sequence_bytes"] / p["sequence_bytes"] == 2 * A / (A + S)
    assert round(2 * A / (A + S), 3) == G["p3_gptoss_compression"]
    assert bf16["skipped_positions"] == A and fp8["skipped_positions"] == 0


def test_half_skipped_equal_retention(kvq, orc):
    p, _ = _both(kvq, orc, 16, 8, 128, [W.BF16, W.FP8_PER_TENSOR], [0, 0], 4096, 1 << 34)
    A, S = p["retained_positions"], p["skipped_positions"]
    assert S * 2 == A and round(2 * A / (A + S), 2) == G["p3_half_skipped_equal_retention_ratio"]


def test_32_layer_block_capacity(kvq, orc):
    """66 KiB per token and 1,056 KiB per 16-token block; the pool divided by
    the rounded block bytes."""
    modes, wins = [W.FP8_PER_TOKEN_HEAD] * 32, [0] * 32
    one, _ = _both(kvq, orc, 16, 8, 128, modes, wins, 16, 1 << 40)
    assert one["sequence_bytes"] / KiB == G["p2_block16_32L_KiB"]
    assert one["sequence_bytes"] / 16 / KiB == G["p2_total_per_token_32L_KiB"]
    long, _ = _both(kvq, orc, 16, 8, 128, modes, wins, 128 * 1024, 1 << 40)
    assert long["sequence_bytes"] / GiB == G["p2_total_32L_128Ki_GiB"]
    block = one["sequence_bytes"]
    for k in (1, 7, 1000):
        exact, blocks = _both(kvq, orc, 16, 8, 128, modes, wins, 16, k * block)
        assert exact["max_sequences"] == k and blocks == [k] * 32
        short, _ = _both(kvq, orc, 16, 8, 128, modes, wins, 16, k * block - 1)
        assert short["max_sequences"] == k - 1


@pytest.mark.parametrize("seed", range(6))
def test_plan_is_the_largest_buffer_that_fits(kvq, orc, seed):
    """For mixed modes and windows, the plan's buffer fits the pool and one
    more sequence would not (layer alignment and static tables included)."""
    import random
    rng = random.Random(seed)
    bs = rng.choice([1, 4, 16, 64])
    hkv, hd = rng.choice([1, 3, 8]), rng.choice([64, 128, 256])
    L = rng.randint(1, 9)
    modes = [rng.randrange(5) for _ in range(L)]
    wins = [rng.choice([0, 0, bs, 4 * bs, 32 * bs]) for _ in range(L)]
    context = rng.randint(1, 5000)
    pool = rng.randint(1, 1 << 31)
    p, blocks = _both(kvq, orc, bs, hkv, hd, modes, wins, context, pool)
    per_seq = [-(-min(context, w if w else context) // bs) for w in wins]
    n = p["max_sequences"]
    assert blocks == [n * b for b in per_seq]
    nxt = kvq.kvq_cache_bytes(kvq.CacheConfig(bs, hkv, hd, modes, [(n + 1) * b for b in per_seq]))["total"]
    assert nxt > pool
    if n:
        assert kvq.kvq_cache_bytes(kvq.CacheConfig(bs, hkv, hd, modes, blocks))["total"] == p["buffer_bytes"] <= pool


def test_plan_argument_checks(kvq):
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_plan_capacity(kvq.ModelConfig(16, 8, 64, [W.BF16], [100]), 1000, 1 << 30)   # window not whole blocks
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_plan_capacity(kvq.ModelConfig(16, 8, 64, [W.BF16], [0]), 0, 1 << 30)
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_plan_capacity(kvq.ModelConfig(16, 8, 96, [W.BF16], [0]), 10, 1 << 30)
    assert e.value.status == kvq.ERR_UNSUPPORTED
    p, blocks = kvq.kvq_plan_capacity(kvq.ModelConfig(16, 8, 64, [W.BF16], [0]), 10, 100)   # pool too small
    assert p["max_sequences"] == 0 and blocks == [0] and p["buffer_bytes"] == 0
