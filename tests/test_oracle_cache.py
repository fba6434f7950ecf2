"""Pins of the oracle's store and gather: an independent brute-force
statement of the method (tests/_brute.py), the pages' numeric examples,
invariants (power-of-two scaling, negation, top-of-range), error bounds and
special cases with a known exact answer."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import _brute
from tests import _calib as C
from tests._golden import load as load_golden

MODES = [W.BF16, W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _adversarial_kv(n, hkv, hd, seed):
    """Normal rows plus rows that are all zero, contain -0, are bf16-subnormal,
    are huge, or mix magnitudes across 60 binades."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(2):
        x = torch.randn((n, hkv, hd), generator=g)
        kinds = torch.randint(0, 6, (n, hkv), generator=g)
        scale = torch.ones((n, hkv))
        scale[kinds == 1] = 0.0
        scale[kinds == 2] = 2.0 ** -130
        scale[kinds == 3] = 2.0 ** 100
        x = x * scale[..., None]
        mixed = kinds == 4
        e = torch.randint(-30, 30, (n, hkv, hd), generator=g).float()
        x = torch.where(mixed[..., None], x * torch.exp2(e), x)
        negz = kinds == 5
        x = torch.where(negz[..., None] & (torch.rand((n, hkv, hd), generator=g) < 0.5), -0.0 * x.abs(), x)
        xb = x.to(torch.bfloat16)
        out.append(xb)
    return out


def _geometry(orc, mode, hkv, hd, bs=4, nblocks=12):
    modes = [W.FP8_PER_TOKEN_HEAD, mode, W.INT4_PER_TOKEN_HEAD]
    nb = [3, nblocks, 2]
    return orc.Geometry(bs, hkv, hd, modes, nb), modes, nb


def _static_scales(mode, hkv, rng):
    if mode == W.FP8_PER_TENSOR:
        return rng.uniform(0.001, 0.05, 2).astype(np.float32)
    if mode == W.FP8_PER_HEAD:
        return rng.uniform(0.001, 0.05, 2 * hkv).astype(np.float32)
    return None


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("hkv", [1, 3])
def test_store_and_gather_match_brute_force(orc, mode, hd, hkv):
    bs, nblocks = 4, 12
    g, modes, nb = _geometry(orc, mode, hkv, hd, bs, nblocks)
    n = 29
    rng = np.random.default_rng(hd * 10 + hkv + 100 * mode)
    k, v = _adversarial_kv(n, hkv, hd, seed=hd + hkv + mode)
    slots = rng.permutation(nblocks * bs)[:n].astype(np.int64)
    slots[3] = -1                                # skipped token
    slots[7] = nblocks * bs + 5                  # beyond the layer: not stored
    scales = _static_scales(mode, hkv, rng)
    buf_o = orc.new_cache(g)
    orc.store(g, buf_o, 1, _bits(k), _bits(v), slots, scales)
    buf_b = np.zeros_like(buf_o)
    _brute.store(buf_b, bs, hkv, hd, modes, nb, 1, _bits(k), _bits(v), slots, scales)
    assert np.array_equal(buf_o, buf_b)

    # Gather through a block table that covers every block in shuffled order,
    # with a ragged last block and an out-of-range entry.
    perm = rng.permutation(nblocks).astype(np.int32)
    bt = np.stack([perm[:6], perm[6:]])
    bt[1, 5] = nblocks + 3
    seq_lens = np.array([21, 24], np.int32)
    ko, vo = orc.gather(g, buf_o, 1, bt, seq_lens)
    kb, vb = _brute.gather(buf_b, bs, hkv, hd, modes, nb, 1, bt, seq_lens)
    assert np.array_equal(ko, kb) and np.array_equal(vo, vb)


def test_tiny_range_sharing_example(orc):
    """Shared scale 32/448: the head that stays below 2 decodes to at most 28,
    one sixteenth of 448; per-token-head scales put every head's maximum at 448."""
    gold = load_golden("range_examples.txt")
    k, v = W.tiny_kv(seed=0)
    kb, vb = _bits(k), _bits(v)
    assert float(k[:, 0].float().abs().max()) == gold["shared_scale_small_head_absmax"]
    assert float(k[:, 1].float().abs().max()) == gold["shared_scale_large_head_absmax"]
    s = np.float32(gold["shared_scale_large_head_absmax"]) / np.float32(448.0)
    g = orc.Geometry(16, 2, 64, [W.FP8_PER_TENSOR], [4])
    buf = orc.new_cache(g)
    orc.store(g, buf, 0, kb, vb, np.arange(64), np.array([s, s], np.float32))
    codes = buf[: 4 * 16 * 2 * 2 * 64].reshape(64, 2, 2, 64)      # [pos][h][K,V][hd]
    dec = orc.e4m3_decode(codes[:, 0, 0])
    assert np.abs(dec).max() / 448.0 == gold["small_head_range_fraction"]
    assert (codes[:, 1, 0] & 0x7F).max() == 0x7E

    g2 = orc.Geometry(16, 2, 64, [W.FP8_PER_TOKEN_HEAD], [4])
    buf2 = orc.new_cache(g2)
    orc.store(g2, buf2, 0, kb, vb, np.arange(64))
    blk = buf2[: 4 * (16 * 2 * 2 * 64 + 16 * 2 * 8)].reshape(4, -1)
    codes2 = blk[:, : 16 * 2 * 2 * 64].reshape(64, 2, 2, 64)
    assert ((codes2 & 0x7F).max(axis=3) == 0x7E).all()


def test_quiet_token_keeps_its_own_range(orc):
    """Two tokens of one head, absmax 0.5 and 2: per-token-head scales differ by
    exactly 4 and both reach 448; a scale fitted to 2 leaves the quiet token at
    448/4."""
    gold = load_golden("range_examples.txt")
    quiet, loud = gold["quiet_token_absmax"], gold["loud_token_absmax"]
    hd = 64
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, (2, 1, hd)).astype(np.float32)
    x[0, 0] *= quiet / np.abs(x[0, 0]).max()
    x[1, 0] *= loud / np.abs(x[1, 0]).max()
    xb = _bits(torch.from_numpy(x).to(torch.bfloat16))
    assert np.abs(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()).max(axis=2).ravel().tolist() == [quiet, loud]
    g = orc.Geometry(1, 1, hd, [W.FP8_PER_TOKEN_HEAD], [2])
    buf = orc.new_cache(g)
    orc.store(g, buf, 0, xb, xb, np.arange(2))
    blk = buf[: 2 * (2 * hd + 8)].reshape(2, -1)
    s = blk[:, 2 * hd:].copy().view(np.float32)[:, 0]
    assert s[1] / s[0] == 4.0
    assert ((blk[:, :hd] & 0x7F).max(axis=1) == 0x7E).all()

    g2 = orc.Geometry(1, 1, hd, [W.FP8_PER_HEAD], [2])
    buf2 = orc.new_cache(g2)
    sc = np.array([loud / 448.0, loud / 448.0], np.float32)
    orc.store(g2, buf2, 0, xb, xb, np.arange(2), sc)
    dec = orc.e4m3_decode(buf2[: 2 * 2 * hd].reshape(2, 2, hd)[:, 0])
    assert np.abs(dec[0]).max() == 112.0 and np.abs(dec[1]).max() == 448.0


def _store_rows(orc, mode, kb, vb, hkv, hd, scales=None):
    n = kb.shape[0]
    g = orc.Geometry(1, hkv, hd, [mode], [n])
    buf = orc.new_cache(g)
    orc.store(g, buf, 0, kb, vb, np.arange(n), scales)
    return g, buf


def _blocks(buf, n, mode, hkv, hd):
    """The layer-0 region of a block_size-1 cache as [n, block_bytes]."""
    rb = {W.BF16: 2 * hd, W.INT4_PER_TOKEN_HEAD: hd // 2}.get(mode, hd)
    bb = hkv * 2 * rb + (hkv * 8 if mode in (W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD) else 0)
    return buf[: n * bb].reshape(n, bb)


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD])
@pytest.mark.parametrize("k", [-20, 7])
def test_power_of_two_scaling_invariance(orc, mode, k):
    """Scaling the input by 2^k (no subnormal or overflow involved) leaves the
    codes unchanged and multiplies the stored scales by exactly 2^k."""
    hkv, hd, n = 2, 128, 50
    x = torch.randn((n, hkv, hd), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    y = (x.float() * 2.0 ** k).to(torch.bfloat16)
    assert torch.equal(y.float(), x.float() * 2.0 ** k)
    rb = hd if mode == W.FP8_PER_TOKEN_HEAD else hd // 2
    _, b1 = _store_rows(orc, mode, _bits(x), _bits(x), hkv, hd)
    _, b2 = _store_rows(orc, mode, _bits(y), _bits(y), hkv, hd)
    b1, b2 = _blocks(b1, n, mode, hkv, hd), _blocks(b2, n, mode, hkv, hd)
    cb = hkv * 2 * rb
    assert np.array_equal(b1[:, :cb], b2[:, :cb])
    s1 = b1[:, cb:].copy().view(np.float32)
    s2 = b2[:, cb:].copy().view(np.float32)
    assert np.array_equal(s1 * np.float32(2.0 ** k), s2)


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD, W.FP8_PER_TENSOR])
def test_negation_flips_codes_keeps_scales(orc, mode):
    hkv, hd, n = 2, 64, 40
    x = torch.randn((n, hkv, hd), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    sc = np.array([0.01, 0.02], np.float32) if mode == W.FP8_PER_TENSOR else None
    _, b1 = _store_rows(orc, mode, _bits(x), _bits(x), hkv, hd, sc)
    _, b2 = _store_rows(orc, mode, _bits(-x), _bits(-x), hkv, hd, sc)
    rb = hd // 2 if mode == W.INT4_PER_TOKEN_HEAD else hd
    cb = hkv * 2 * rb
    c1 = _blocks(b1, n, mode, hkv, hd)
    c2 = _blocks(b2, n, mode, hkv, hd)
    if mode == W.INT4_PER_TOKEN_HEAD:
        def signed(nib):
            nib = nib.astype(np.int16)
            return np.where(nib >= 8, nib - 16, nib)
        lo1, hi1 = signed(c1[:, :cb] & 0xF), signed(c1[:, :cb] >> 4)
        lo2, hi2 = signed(c2[:, :cb] & 0xF), signed(c2[:, :cb] >> 4)
        assert np.array_equal(lo1, -lo2) and np.array_equal(hi1, -hi2)
    else:
        assert np.array_equal(c1[:, :cb] ^ 0x80, c2[:, :cb])
    assert np.array_equal(c1[:, cb:], c2[:, cb:])


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD, W.FP8_PER_HEAD])
def test_round_trip_error_bound(orc, mode):
    """|x - x_hat| within the format's rounding bound.  E4M3 unsaturated:
    2^-4 |q| relative (3 fraction bits) or 2^-10 absolute below 2^-6, in units
    of s; INT4: s/2; plus the final BF16 rounding (2^-9 relative)."""
    hkv, hd, n = 4, 128, 64
    k, v = W.gqa_kv(n, hkv, hd, seed=9)
    kb, vb = _bits(k), _bits(v)
    sc = None
    if mode == W.FP8_PER_HEAD:
        sc = C.oracle_static_scales(orc, k, v, mode)
    g, buf = _store_rows(orc, mode, kb, vb, hkv, hd, sc)
    ko, vo = orc.gather(g, buf, 0, np.arange(n, dtype=np.int32)[None, :], np.array([n], np.int32))
    for x, xo, c in ((k, ko, 0), (v, vo, 1)):
        x = x.float().numpy().astype(np.float64)
        xh = torch.from_numpy(xo.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
        if mode == W.FP8_PER_HEAD:
            s = sc.reshape(2, hkv)[c][None, :, None].astype(np.float64)
        elif mode == W.FP8_PER_TOKEN_HEAD:
            s = np.abs(x).max(axis=2, keepdims=True) / 448.0
        else:
            s = np.abs(x).max(axis=2, keepdims=True) / 7.0
        if mode == W.INT4_PER_TOKEN_HEAD:
            bound = s / 2 * (1 + 1e-6)
        else:
            bound = (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s) * (1 + 1e-6)
        bound = bound + 2.0 ** -8 * np.abs(xh)
        assert (np.abs(x - xh) <= bound).all()


def test_unit_scale_round_trips_e4m3_values_exactly(orc):
    """Per-tensor scale 1.0: every E4M3-representable input comes back exactly."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = orc.e4m3_decode(codes)                  # 254 values
    x = np.resize(vals, 4 * 2 * 64).reshape(4, 2, 64)
    xb = _bits(torch.from_numpy(x).to(torch.bfloat16))
    g, buf = _store_rows(orc, W.FP8_PER_TENSOR, xb, xb, 2, 64, np.array([1.0, 1.0], np.float32))
    ko, vo = orc.gather(g, buf, 0, np.arange(4, dtype=np.int32)[None, :], np.array([4], np.int32))
    assert np.array_equal(ko, xb) and np.array_equal(vo, xb)


def test_bf16_layer_round_trip_is_bit_exact(orc):
    k, v = _adversarial_kv(33, 2, 64, seed=21)
    g, buf = _store_rows(orc, W.BF16, _bits(k), _bits(v), 2, 64)
    ko, vo = orc.gather(g, buf, 0, np.arange(33, dtype=np.int32)[None, :], np.array([33], np.int32))
    assert np.array_equal(ko, _bits(k)) and np.array_equal(vo, _bits(v))


def test_ring_buffer_keeps_last_window(orc):
    """A sliding layer retains at most W positions: storing T tokens through
    ring slots keeps exactly tokens T-W..T-1, token t at slot t mod W."""
    T, Wn, bs, hkv, hd = 100, 32, 16, 2, 64
    k, v = W.normal_kv(T, hkv, hd, seed=5)
    g = orc.Geometry(bs, hkv, hd, [W.BF16], [Wn // bs])
    buf = orc.new_cache(g)
    orc.store(g, buf, 0, _bits(k), _bits(v), W.ring_slots(T, Wn).numpy())
    ko, _ = orc.gather(g, buf, 0, W.ring_block_table(Wn, bs).numpy(), np.array([Wn], np.int32))
    kb = _bits(k)
    for r in range(Wn):
        t = [t for t in range(T - Wn, T) if t % Wn == r][0]
        assert np.array_equal(ko[r], kb[t])


def test_gather_packs_sequences_in_order(orc):
    """Output rows of sequence b start at sum of the previous seq_lens, and
    gather returns what store put in, for a block table in shuffled order."""
    bs, hkv, hd = 16, 2, 64
    lens = [5, 0, 33, 16]
    st = W.DecodeState(num_seqs=4, block_size=bs, num_blocks=10, max_blocks_per_seq=3, seed=3)
    slots = []
    for b, n in enumerate(lens):
        slots += st.append(b, n)
    n = sum(lens)
    x = torch.arange(n * hkv * hd, dtype=torch.float32).view(n, hkv, hd).to(torch.bfloat16)
    g = orc.Geometry(bs, hkv, hd, [W.BF16], [10])
    buf = orc.new_cache(g)
    orc.store(g, buf, 0, _bits(x), _bits(x), np.array(slots))
    ko, _ = orc.gather(g, buf, 0, st.block_table.numpy(), np.array(lens, np.int32))
    assert np.array_equal(ko, _bits(x))


def test_calibration_amax_vs_numpy(orc):
    """Running per-(K/V, head) absmax over two batches equals numpy's max of
    |x| over both batches; a per-tensor scale is the max over heads."""
    k1, v1 = W.gqa_kv(300, 3, 64, seed=41)
    k2, v2 = W.gqa_kv(77, 3, 64, seed=42)
    a = orc.calibrate_amax(_bits(k1), _bits(v1), 3, 64)
    a = orc.calibrate_amax(_bits(k2), _bits(v2), 3, 64, amax=a)
    kk = np.abs(np.concatenate([k1.float().numpy(), k2.float().numpy()]))
    vv = np.abs(np.concatenate([v1.float().numpy(), v2.float().numpy()]))
    want = np.concatenate([kk.max(axis=(0, 2)), vv.max(axis=(0, 2))]).astype(np.float32)
    assert np.array_equal(a, want)
    zero = orc.calibrate_amax(np.zeros((5, 3, 64), np.uint16), np.zeros((5, 3, 64), np.uint16), 3, 64)
    assert (zero == 0).all()
