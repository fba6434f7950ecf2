"""Host-side checks of the C-ABI library that need no GPU: it loads, it
exports every function include/kvq.h declares, and every argument check
returns its status before any HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_DEV = 0x7F0000000000          # 256-byte aligned; never dereferenced by these calls


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    return kvq


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"KVQ_API\s+[\w\s\*]+?\b(kvq_\w+)\s*\(", text)))


def test_header_declarations_are_exported(kvq):
    declared = _declared_functions()
    assert declared == sorted(kvq.EXPORTED_SYMBOLS)
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_library_exports_nothing_else(kvq):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    public = {n for n in names if n.startswith("kvq")}
    assert public == set(kvq.EXPORTED_SYMBOLS)


def test_status_strings(kvq):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert kvq._lib.kvq_status_string(s)
    assert b"unknown" in kvq._lib.kvq_status_string(-99)


def _cfg(kvq, modes, hd=64, bs=16, hkv=2, nblocks=4):
    return kvq.CacheConfig(bs, hkv, hd, modes, [nblocks] * len(modes))


def _handle(kvq, cfg):
    return kvq.kvq_create_cache(cfg, FAKE_DEV, kvq.kvq_cache_bytes(cfg)["total"])


def test_cache_bytes_rejects_bad_geometry(kvq):
    for hd in (32, 96, 512):
        with pytest.raises(kvq.KVQError) as e:
            kvq.kvq_cache_bytes(_cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD], hd=hd))
        assert e.value.status == kvq.ERR_UNSUPPORTED
    for bs in (3, 2048):
        with pytest.raises(kvq.KVQError) as e:
            kvq.kvq_cache_bytes(_cfg(kvq, [kvq.BF16], bs=bs))
        assert e.value.status == kvq.ERR_UNSUPPORTED
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_cache_bytes(_cfg(kvq, [7]))
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_cache_bytes(kvq.CacheConfig(16, 2, 64, [kvq.BF16], [-1]))
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_cache_bytes(kvq.CacheConfig(16, 0, 64, [kvq.BF16], [1]))
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_cache_bytes(kvq.CacheConfig(16, 300, 64, [kvq.FP8_PER_HEAD], [1]))
    assert e.value.status == kvq.ERR_UNSUPPORTED
    assert kvq._lib.kvq_cache_bytes(None, None) == kvq.ERR_INVALID_ARG


def test_create_cache_checks(kvq):
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD])
    total = kvq.kvq_cache_bytes(cfg)["total"]
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_create_cache(cfg, FAKE_DEV, total - 1)
    assert e.value.status == kvq.ERR_BUFFER_TOO_SMALL
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_create_cache(cfg, FAKE_DEV + 16, total)
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_create_cache(cfg, 0, total)
    assert e.value.status == kvq.ERR_INVALID_ARG
    h = kvq.kvq_create_cache(cfg, FAKE_DEV, total)
    kvq.kvq_destroy_cache(h)
    assert kvq._lib.kvq_destroy_cache(None) == kvq.OK


def _store(kvq, h, layer, n, mode, scales=None, keys=FAKE_DEV, values=FAKE_DEV, slots=FAKE_DEV):
    sc = None
    if scales is not None:
        sc = (ctypes.c_float * len(scales))(*scales)
    return kvq._lib.kvq_store(h, layer, ctypes.c_void_p(keys), ctypes.c_void_p(values), ctypes.c_void_p(slots),
                              n, mode, sc, None)


def _gather(kvq, h, layer, nseq, maxb=4, out=FAKE_DEV, rows=64):
    return kvq._lib.kvq_gather_dequant(h, layer, ctypes.c_void_p(FAKE_DEV), maxb, ctypes.c_void_p(FAKE_DEV),
                                       nseq, ctypes.c_void_p(out), ctypes.c_void_p(out), rows, None)


def test_store_argument_checks(kvq):
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD, kvq.FP8_PER_TENSOR, kvq.FP8_PER_HEAD, kvq.BF16])
    h = _handle(kvq, cfg)
    try:
        assert _store(kvq, h, 4, 1, kvq.BF16) == kvq.ERR_INVALID_ARG              # layer out of range
        assert _store(kvq, h, -1, 1, kvq.BF16) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 1, kvq.INT4_PER_TOKEN_HEAD) == kvq.ERR_MODE_MISMATCH
        assert _store(kvq, h, 3, 1, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_MODE_MISMATCH
        assert _store(kvq, h, 0, -1, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 0, kvq.FP8_PER_TOKEN_HEAD) == kvq.OK              # no-op, no HIP call
        assert _store(kvq, h, 0, 1, kvq.FP8_PER_TOKEN_HEAD, [1.0, 1.0]) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 1, kvq.FP8_PER_TOKEN_HEAD, keys=0) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 1, kvq.FP8_PER_TOKEN_HEAD, values=FAKE_DEV + 8) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 1, kvq.FP8_PER_TOKEN_HEAD, slots=FAKE_DEV + 4) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 0, 1 << 30, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_UNSUPPORTED
        # static layers: first call needs positive finite scales of the right count
        assert _store(kvq, h, 1, 1, kvq.FP8_PER_TENSOR) == kvq.ERR_INVALID_ARG
        for bad in ([0.0, 1.0], [1.0, -2.0], [float("nan"), 1.0], [1.0, float("inf")]):
            assert _store(kvq, h, 1, 1, kvq.FP8_PER_TENSOR, bad) == kvq.ERR_INVALID_ARG
        assert _store(kvq, h, 2, 1, kvq.FP8_PER_HEAD, [1.0, 1.0, 1.0, 0.0]) == kvq.ERR_INVALID_ARG
        # gather: a static layer never stored to has no scales yet
        assert _gather(kvq, h, 1, 1) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 0) == kvq.OK                                    # no-op
        assert _gather(kvq, h, 0, -1) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1, maxb=0) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1, out=FAKE_DEV + 2) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 9, 1) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1 << 20, maxb=1 << 12) == kvq.ERR_UNSUPPORTED
        # output capacity: negative or absurd row counts, null outputs with rows
        assert _gather(kvq, h, 0, 1, rows=-1) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1, rows=(1 << 46) + 1) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1, out=0) == kvq.ERR_INVALID_ARG
        assert _gather(kvq, h, 0, 1, out=0, rows=0) == kvq.OK                     # nothing to write: no launch
    finally:
        kvq.kvq_destroy_cache(h)


def test_ordered_store_argument_checks(kvq):
    """kvq_store_ordered: kvq_store's checks, plus a 4-byte aligned order that
    may be NULL only for an empty call; and the host query of which layers
    follow the order."""
    lib = kvq._lib
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD, kvq.FP8_PER_TENSOR, kvq.FP8_PER_HEAD, kvq.BF16])
    h = _handle(kvq, cfg)
    P = ctypes.c_void_p

    def st(layer, n, mode, order=FAKE_DEV + 4096):
        return lib.kvq_store_ordered(h, layer, P(FAKE_DEV), P(FAKE_DEV + 1024), P(FAKE_DEV + 2048), P(order), n,
                                     mode, None, None)
    try:
        assert st(0, 1, kvq.FP8_PER_TOKEN_HEAD, order=0) == kvq.ERR_INVALID_ARG        # no order
        assert st(0, 1, kvq.FP8_PER_TOKEN_HEAD, order=FAKE_DEV + 2) == kvq.ERR_INVALID_ARG
        assert st(0, 0, kvq.FP8_PER_TOKEN_HEAD, order=0) == kvq.OK                    # empty: no order needed
        assert st(4, 1, kvq.BF16) == kvq.ERR_INVALID_ARG
        assert st(0, 1, kvq.INT4_PER_TOKEN_HEAD) == kvq.ERR_MODE_MISMATCH
        assert st(0, -1, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_INVALID_ARG
        assert st(0, 1 << 30, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_UNSUPPORTED
    finally:
        kvq.kvq_destroy_cache(h)
    follows = lib.kvq_store_follows_order
    for hd in (128, 256):
        for m in (kvq.BF16, kvq.FP8_PER_TENSOR, kvq.FP8_PER_HEAD, kvq.FP8_PER_TOKEN_HEAD):
            assert follows(m, hd) == 1, (m, hd)
    for m in (kvq.BF16, kvq.FP8_PER_TENSOR, kvq.FP8_PER_HEAD, kvq.FP8_PER_TOKEN_HEAD, kvq.INT4_PER_TOKEN_HEAD):
        assert follows(m, 64) == 0
    assert follows(kvq.INT4_PER_TOKEN_HEAD, 128) == 0 and follows(kvq.INT4_PER_TOKEN_HEAD, 256) == 0
    assert follows(kvq.FP8_PER_TOKEN_HEAD, 96) == 0 and follows(7, 128) == 0 and follows(-1, 128) == 0


def test_odd_block_with_scales_is_unsupported(kvq):
    """An odd block_size * num_kv_heads makes per-token-head blocks 8 mod 16
    bytes long; the kernels' 16-byte accesses need 16-byte blocks."""
    cfg = kvq.CacheConfig(1, 1, 64, [kvq.FP8_PER_TOKEN_HEAD], [4])
    h = _handle(kvq, cfg)
    try:
        assert _store(kvq, h, 0, 1, kvq.FP8_PER_TOKEN_HEAD) == kvq.ERR_UNSUPPORTED
        assert _gather(kvq, h, 0, 1) == kvq.ERR_UNSUPPORTED
    finally:
        kvq.kvq_destroy_cache(h)


def test_static_scales_match_ieee_float32_division(kvq):
    import numpy as np
    rng = np.random.default_rng(3)
    amax = rng.uniform(0, 40, 16).astype(np.float32)
    amax[3] = 0.0
    amax[5] = np.float32(2.0 ** -130)
    got = np.array(kvq.kvq_static_scales(amax, 8, kvq.FP8_PER_HEAD), np.float32)
    want = amax / np.float32(448.0)
    want[3] = np.float32(1e-45)                      # zero maximum -> smallest positive float
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    pt = np.array(kvq.kvq_static_scales(amax, 8, kvq.FP8_PER_TENSOR), np.float32)
    assert np.array_equal(pt, np.array([amax[:8].max(), amax[8:].max()], np.float32) / np.float32(448.0))
    with pytest.raises(kvq.KVQError):
        kvq.kvq_static_scales([1.0, float("nan")], 1, kvq.FP8_PER_HEAD)
    with pytest.raises(kvq.KVQError):
        kvq.kvq_static_scales([1.0, -1.0], 1, kvq.FP8_PER_TENSOR)
    with pytest.raises(kvq.KVQError):
        kvq.kvq_static_scales([1.0, 1.0], 1, kvq.FP8_PER_TOKEN_HEAD)


def test_calibrate_argument_checks(kvq):
    lib = kvq._lib
    P = ctypes.c_void_p
    assert lib.kvq_calibrate_amax(P(FAKE_DEV), P(FAKE_DEV), 4, 8, 128, None, 0, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_calibrate_amax(P(FAKE_DEV), P(FAKE_DEV), 4, 8, 96, P(FAKE_DEV), 0, None) == kvq.ERR_UNSUPPORTED
    assert lib.kvq_calibrate_amax(P(FAKE_DEV), P(FAKE_DEV), 4, 300, 128, P(FAKE_DEV), 0, None) == kvq.ERR_UNSUPPORTED
    assert lib.kvq_calibrate_amax(P(FAKE_DEV), P(FAKE_DEV), -1, 8, 128, P(FAKE_DEV), 0, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_calibrate_amax(P(FAKE_DEV + 8), P(FAKE_DEV), 4, 8, 128, P(FAKE_DEV), 0, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_calibrate_amax(P(FAKE_DEV), P(FAKE_DEV), 4, 8, 128, P(FAKE_DEV + 2), 0, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_calibrate_amax(None, None, 0, 8, 128, P(FAKE_DEV), 1, None) == kvq.OK     # no-op
    assert lib.kvq_calibrate_amax(None, None, 4, 8, 128, P(FAKE_DEV), 0, None) == kvq.ERR_INVALID_ARG


def _attn(kvq, h, layer, nseq, H=4, maxb=4, q=FAKE_DEV, out=FAKE_DEV, ws=0, wsb=0, sm=0.125):
    return kvq._lib.kvq_decode_attention(h, layer, ctypes.c_void_p(q), H, ctypes.c_void_p(FAKE_DEV), maxb,
                                         ctypes.c_void_p(FAKE_DEV), nseq, sm, ctypes.c_void_p(out),
                                         ctypes.c_void_p(ws), wsb, None)


def test_attention_argument_checks(kvq):
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD, kvq.FP8_PER_TENSOR, kvq.BF16], hd=128)
    h = _handle(kvq, cfg)
    try:
        assert _attn(kvq, h, 3, 1) == kvq.ERR_INVALID_ARG                 # layer out of range
        assert _attn(kvq, h, 0, 0) == kvq.OK                              # no-op, no HIP call
        assert _attn(kvq, h, 0, -1) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 0, 1, H=3) == kvq.ERR_INVALID_ARG            # not a multiple of Hkv
        assert _attn(kvq, h, 0, 1, H=0) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 0, 1, maxb=0) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 0, 1, q=0) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 0, 1, q=FAKE_DEV + 8) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 0, 1, out=FAKE_DEV + 2) == kvq.ERR_INVALID_ARG
        for sm in (float("nan"), float("inf")):
            assert _attn(kvq, h, 0, 1, sm=sm) == kvq.ERR_INVALID_ARG
        assert _attn(kvq, h, 1, 1) == kvq.ERR_INVALID_ARG                 # static layer never stored
        assert _attn(kvq, h, 0, 1, maxb=1 << 27) == kvq.ERR_UNSUPPORTED   # max_blocks * bs >= 2^31
        # a context of more than 8 tiles is split and needs the workspace
        need = kvq.kvq_decode_attention_workspace(h, 4, 64, 2)
        assert need > 0 and need % (2 * 4 * (128 + 2) * 4) == 0
        assert _attn(kvq, h, 0, 2, maxb=64) == kvq.ERR_BUFFER_TOO_SMALL
        assert _attn(kvq, h, 0, 2, maxb=64, ws=FAKE_DEV, wsb=need - 1) == kvq.ERR_BUFFER_TOO_SMALL
        assert _attn(kvq, h, 0, 2, maxb=64, ws=FAKE_DEV + 8, wsb=need) == kvq.ERR_INVALID_ARG
        # at most 8 tiles of context: one split, no workspace
        assert kvq.kvq_decode_attention_workspace(h, 4, 8, 2) == 0
        assert kvq.kvq_decode_attention_workspace(h, 4, 64, 0) == 0
        for args in ((3, 64, 2), (0, 64, 2), (4, 0, 2), (4, 64, -1)):
            with pytest.raises(kvq.KVQError) as e:
                kvq.kvq_decode_attention_workspace(h, *args)
            assert e.value.status == kvq.ERR_INVALID_ARG
        assert kvq._lib.kvq_decode_attention_workspace(h, 4, 64, 2, None) == kvq.ERR_INVALID_ARG
    finally:
        kvq.kvq_destroy_cache(h)



def test_blocks_of_2gib_or_more_are_unsupported(kvq):
    """The kernels address a block with 32-bit offsets, so a layer whose
    block (codes and scale trailer) reaches 2^31 bytes is refused."""
    ok = kvq.CacheConfig(1024, 1024, 256, [kvq.BF16], [1])            # 2^30-byte blocks
    assert kvq.kvq_cache_bytes(ok)["total"] == 1 << 30
    for hkv, mode in ((2048, kvq.BF16), (4096, kvq.FP8_PER_TOKEN_HEAD), (8192, kvq.INT4_PER_TOKEN_HEAD)):
        with pytest.raises(kvq.KVQError) as e:
            kvq.kvq_cache_bytes(kvq.CacheConfig(1024, hkv, 256, [mode], [1]))
        assert e.value.status == kvq.ERR_UNSUPPORTED


def test_noalloc_attention_argument_checks(kvq):
    """The allocation-free attention checks everything before any HIP call,
    and refuses a call shape whose split partials exceed its fixed array."""
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD, kvq.FP8_PER_TENSOR], hd=128)
    h = _handle(kvq, cfg)

    def call(layer, nseq=1, H=4, maxb=4, q=FAKE_DEV, out=FAKE_DEV, sm=0.125):
        return kvq._lib.kvq_decode_attention_noalloc(h, layer, ctypes.c_void_p(q), H, ctypes.c_void_p(FAKE_DEV),
                                                     maxb, ctypes.c_void_p(FAKE_DEV), nseq, sm,
                                                     ctypes.c_void_p(out), None)
    try:
        assert call(2) == kvq.ERR_INVALID_ARG                 # layer out of range
        assert call(0, nseq=0) == kvq.OK                      # no-op, no HIP call
        assert call(0, nseq=-1) == kvq.ERR_INVALID_ARG
        assert call(0, H=3) == kvq.ERR_INVALID_ARG
        assert call(0, q=0) == kvq.ERR_INVALID_ARG
        assert call(0, out=FAKE_DEV + 2) == kvq.ERR_INVALID_ARG
        assert call(0, sm=float("nan")) == kvq.ERR_INVALID_ARG
        assert call(1) == kvq.ERR_INVALID_ARG                 # static layer never stored
        assert call(0, maxb=1 << 27) == kvq.ERR_UNSUPPORTED
    finally:
        kvq.kvq_destroy_cache(h)
    # 1023 sequences of one KV head with 16 query heads at head_dim 256 take
    # two splits each: 1023 * 16 * 2 * 258 * 4 bytes of partials, above 32 MiB
    big = kvq.CacheConfig(16, 1, 256, [kvq.FP8_PER_TOKEN_HEAD], [4])
    h = _handle(kvq, big)
    try:
        need = kvq.kvq_decode_attention_workspace(h, 16, 16, 1023)
        assert need == 1023 * 16 * 2 * 258 * 4 > kvq.ATTENTION_SCRATCH_BYTES
        assert kvq._lib.kvq_decode_attention_noalloc(h, 0, ctypes.c_void_p(FAKE_DEV), 16, ctypes.c_void_p(FAKE_DEV),
                                                     16, ctypes.c_void_p(FAKE_DEV), 1023, 0.0625,
                                                     ctypes.c_void_p(FAKE_DEV), None) == kvq.ERR_UNSUPPORTED
    finally:
        kvq.kvq_destroy_cache(h)


def test_fp8_query_attention_argument_checks(kvq):
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD, kvq.INT4_PER_TOKEN_HEAD, kvq.BF16], hd=128)
    h = _handle(kvq, cfg)

    def call(layer, qs=FAKE_DEV, nseq=1):
        return kvq._lib.kvq_decode_attention_fp8q(h, layer, ctypes.c_void_p(FAKE_DEV), ctypes.c_void_p(qs), 4,
                                                  ctypes.c_void_p(FAKE_DEV), 4, ctypes.c_void_p(FAKE_DEV), nseq,
                                                  0.125, ctypes.c_void_p(FAKE_DEV), None, 0, None)
    try:
        assert call(0, qs=0) == kvq.ERR_INVALID_ARG                 # FP8 queries need their scales
        assert call(0, qs=FAKE_DEV + 2) == kvq.ERR_INVALID_ARG      # 4-byte aligned
        assert call(1) == kvq.ERR_UNSUPPORTED                       # INT4 layer
        assert call(2) == kvq.ERR_UNSUPPORTED                       # BF16 layer
        assert call(0, nseq=0) == kvq.OK                            # no-op
    finally:
        kvq.kvq_destroy_cache(h)


def test_check_slots_debug_helper(kvq):
    """The binding's debug check of a slot mapping: duplicates among stored
    slots raise; skipped tokens (negative or past the layer) are counted."""
    import types
    import torch
    cfg = _cfg(kvq, [kvq.FP8_PER_TOKEN_HEAD])
    fake = types.SimpleNamespace(cfg=cfg)
    nslots = cfg.layer_num_blocks[0] * cfg.block_size
    ok = torch.tensor([0, 5, -1, nslots, nslots - 1, -7], dtype=torch.int64)
    assert kvq.Cache.check_slots(fake, 0, ok) == 3
    with pytest.raises(ValueError):
        kvq.Cache.check_slots(fake, 0, torch.tensor([3, 4, 3], dtype=torch.int64))
    # repeated skipped slots are no duplicates: they are never written
    assert kvq.Cache.check_slots(fake, 0, torch.tensor([-1, -1, nslots + 2, nslots + 2], dtype=torch.int64)) == 4
