"""Pins of the oracle's decode attention over the quantized cache: it equals
a plain numpy float64 softmax attention over independently dequantized
values (tests/_brute.py), and reduces to known answers in special cases."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import _brute


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _numpy_attention(q, kh, vh, lens, group, sm_scale):
    """Reference softmax attention (float64) over packed [sum(lens), hkv, hd] values."""
    nseq, nqh, hd = q.shape
    out = np.zeros((nseq, nqh, hd))
    row = 0
    for b, n in enumerate(lens):
        for qh in range(nqh):
            if n == 0:
                continue
            k = kh[row: row + n, qh // group]
            v = vh[row: row + n, qh // group]
            s = (k @ q[b, qh]) * sm_scale
            p = np.exp(s - s.max())
            out[b, qh] = (p / p.sum()) @ v
        row += n
    return out


def _setup(orc, mode, hkv=2, hd=64, bs=16, nblocks=12, lens=(37, 0, 80), seed=0, gen=W.gqa_kv):
    g = orc.Geometry(bs, hkv, hd, [mode], [nblocks])
    buf = orc.new_cache(g)
    st = W.DecodeState(len(lens), bs, nblocks, 6, seed=seed)
    slots = []
    for b, n in enumerate(lens):
        slots += st.append(b, n)
    k, v = gen(len(slots), hkv, hd, seed=seed + 1)
    sc = None
    if mode == W.FP8_PER_TENSOR:
        sc = np.array([0.05, 0.04], np.float32)
    elif mode == W.FP8_PER_HEAD:
        sc = np.linspace(0.02, 0.06, 2 * hkv).astype(np.float32)
    orc.store(g, buf, 0, _bits(k), _bits(v), np.array(slots), sc)
    return g, buf, st


@pytest.mark.parametrize("mode", [W.BF16, W.FP8_PER_TENSOR, W.FP8_PER_HEAD, W.FP8_PER_TOKEN_HEAD,
                                  W.INT4_PER_TOKEN_HEAD])
@pytest.mark.parametrize("group", [1, 4])
def test_attention_matches_numpy_over_brute_force_dequant(orc, mode, group):
    hkv, hd = 2, 64
    g, buf, st = _setup(orc, mode, hkv, hd)
    lens = st.seq_lens
    q = torch.randn((len(lens), hkv * group, hd), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    out = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), lens, 0.125)
    kh, vh = _brute.dequant_f64(buf, g.bs, hkv, hd, [mode], [12], 0, st.block_table.numpy(), lens)
    ref = _numpy_attention(q.double().numpy(), kh, vh, lens, group, 0.125)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases(orc):
    hkv, hd = 1, 64
    g, buf, st = _setup(orc, W.BF16, hkv, hd, lens=(1, 5))
    kh, vh = _brute.dequant_f64(buf, g.bs, hkv, hd, [W.BF16], [12], 0, st.block_table.numpy(), [1, 5])
    q = torch.randn((2, 1, hd), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    out = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), [1, 5], 0.3)
    assert np.array_equal(out[0, 0], vh[0, 0])                   # one token: its value
    uni = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), [1, 5], 0.0)
    assert np.allclose(uni[1, 0], vh[1:6, 0].mean(axis=0), rtol=1e-14, atol=1e-14)  # zero scale: mean
    empty = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), [0, 0], 0.3)
    assert not empty.any()
    out2, absv = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), [1, 5], 0.3, with_absv=True)
    assert np.array_equal(out2, out) and (absv >= np.abs(out) - 1e-12).all()


@pytest.mark.parametrize("mode,qmax", [(W.INT4_PER_TOKEN_HEAD, 7.0), (W.FP8_PER_TOKEN_HEAD, 448.0)])
def test_bound_reads_each_tokens_key_scale(orc, mode, qmax):
    """The error bound's INT4 term takes every token's K scale from the cache
    image; read back through the block table they are RN32(absmax / qmax) of
    the stored rows, computed here with numpy float32 division."""
    g, buf, st = _setup(orc, mode)
    lens = np.array(st.seq_lens)
    slots_k, _ = W.gqa_kv(int(lens.sum()), 2, 64, seed=1)
    amax = slots_k.float().abs().amax(dim=2).numpy().astype(np.float32)
    want = (amax / np.float32(qmax)).astype(np.float64)
    got = orc._token_key_scales(g, buf, 0, st.block_table.numpy(), lens)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_attention_skips_blocks_outside_the_layer(orc):
    """Tokens whose block-table entry is negative or past the layer's block
    count take no part; the rest is softmax attention over what remains."""
    hkv, hd, bs = 1, 64, 16
    g, buf, st = _setup(orc, W.FP8_PER_TOKEN_HEAD, hkv, hd, bs=bs, lens=(70,))
    bt = st.block_table.numpy().copy()
    lens = [70]
    kh, vh = _brute.dequant_f64(buf, bs, hkv, hd, [W.FP8_PER_TOKEN_HEAD], [12], 0, bt, lens)
    bt[0, 1] = -1
    bt[0, 3] = 12                                   # one past the last block
    keep = np.array([not (16 <= t < 32 or 48 <= t < 64) for t in range(70)])
    q = torch.randn((1, 2, hd), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    out = orc.decode_attention(g, buf, 0, _bits(q), bt, lens, 0.2)
    ref = _numpy_attention(q.double().numpy(), kh[keep], vh[keep], [int(keep.sum())], 2, 0.2)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    bt[0, :] = -1
    assert not orc.decode_attention(g, buf, 0, _bits(q), bt, lens, 0.2).any()


@pytest.mark.parametrize("mode", [W.FP8_PER_TENSOR, W.FP8_PER_TOKEN_HEAD])
def test_fp8_query_attention_matches_numpy(orc, mode):
    """With static FP8 query scales each query element is its E4M3 code under
    its head's scale, decoded back; here built from numpy float32 division and
    torch's float8_e4m3fn cast, independently of the oracle's codec."""
    hkv, hd, group = 2, 64, 4
    g, buf, st = _setup(orc, mode, hkv, hd)
    lens = st.seq_lens
    q = torch.randn((len(lens), hkv * group, hd), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    qf = q.float().numpy()
    sq = (np.abs(qf).max(axis=(0, 2)) / np.float32(448.0)).astype(np.float32) * np.float32(1.5)   # some saturate
    quo = (qf / sq[None, :, None]).astype(np.float32)
    qhat = _brute._e4m3(quo.reshape(-1)).reshape(quo.shape)
    qhat = torch.from_numpy(qhat).view(torch.float8_e4m3fn).double().numpy() * sq[None, :, None].astype(np.float64)
    out = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), lens, 0.125, q_scales=sq)
    kh, vh = _brute.dequant_f64(buf, g.bs, hkv, hd, [mode], [12], 0, st.block_table.numpy(), lens)
    ref = _numpy_attention(qhat, kh, vh, lens, group, 0.125)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(orc.query_values(_bits(q), sq), qhat)
    # a scale so large that every code is zero: uniform weights, the mean of V
    zero = orc.decode_attention(g, buf, 0, _bits(q), st.block_table.numpy(), lens, 0.125,
                                q_scales=np.full(hkv * group, 3e38, np.float32))
    row0 = 0
    for b, n in enumerate(lens):
        if n:
            assert np.allclose(zero[b], np.repeat(vh[row0: row0 + n].mean(axis=0), group, axis=0), rtol=1e-13, atol=1e-13)
        row0 += n


@pytest.mark.parametrize("mode", [W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD, W.BF16, W.FP8_PER_HEAD])
def test_error_bound_is_not_vacuous(orc, mode):
    """The tolerance the GPU attention tests use catches plausible mistakes,
    planted here in the oracle's own inputs: at the short lengths of those
    tests, dropping a sequence's last token, or giving a token the V row of
    its neighbour, moves some output element of that sequence beyond the
    bound; so does doubling a token's V scale in the per-token-head modes.
    N(0, 1) rows keep every token's softmax weight near 1/len (a token of
    negligible weight can take any value without any tolerance noticing)."""
    hkv, hd, bs = 2, 64, 16
    g, buf, st = _setup(orc, mode, hkv=hkv, hd=hd, bs=bs, lens=(5, 17, 33), gen=W.normal_kv)
    bt = st.block_table.numpy()
    lens = np.array(st.seq_lens, np.int32)
    q = torch.randn((3, 4 * hkv, hd), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    qb = _bits(q)
    sm = 1.0 / np.sqrt(hd)
    v_big = 1.0 if mode != W.FP8_PER_HEAD else 0.06
    ref, absv = orc.decode_attention(g, buf, 0, qb, bt, lens, sm, with_absv=True)
    tol = orc.attention_error_bound(g, buf, 0, qb, bt, lens, sm, ref, absv, v_big)

    def caught(wrong, rows):
        return all((np.abs(wrong[b] - ref[b]) > tol[b]).any() for b in rows)

    # a dropped token
    assert caught(orc.decode_attention(g, buf, 0, qb, bt, lens - 1, sm), range(3))

    # token 0 of each sequence takes the V row of token 1 (head 0), laid out as
    # block = codes[bs][hkv][K, V][row bytes] then, per-token-head, scales[bs][hkv][K, V]
    hb = {W.BF16: 2 * hd, W.INT4_PER_TOKEN_HEAD: hd // 2}.get(mode, hd)
    dyn = mode in (W.FP8_PER_TOKEN_HEAD, W.INT4_PER_TOKEN_HEAD)
    code_bytes = bs * hkv * 2 * hb
    block_bytes = code_bytes + (bs * hkv * 8 if dyn else 0)
    lb, _, _ = orc.layer_offsets(g)
    planted = buf.copy()
    for b in range(3):
        base = int(lb[0]) + int(bt[b, 0]) * block_bytes
        v0 = base + hb                                   # (pos 0, head 0) V row
        v1 = base + (1 * hkv + 0) * 2 * hb + hb          # (pos 1, head 0) V row
        planted[v0: v0 + hb] = buf[v1: v1 + hb]
        if dyn:
            s0 = base + code_bytes + 4
            s1 = base + code_bytes + (1 * hkv) * 8 + 4
            planted[s0: s0 + 4] = buf[s1: s1 + 4]
    assert caught(orc.decode_attention(g, planted, 0, qb, bt, lens, sm), range(3))

    if dyn:
        doubled = buf.copy()
        for b in range(3):
            s0 = int(lb[0]) + int(bt[b, 0]) * block_bytes + code_bytes + 4
            sv = doubled[s0: s0 + 4].view(np.float32)
            doubled[s0: s0 + 4] = (sv * np.float32(2.0)).view(np.uint8)
        assert caught(orc.decode_attention(g, doubled, 0, qb, bt, lens, sm), range(3))
