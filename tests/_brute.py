"""Pure-Python brute-force store and gather for tiny inputs.

A second, independently written statement of the same method, built from
library primitives (numpy float32 IEEE division, torch's float8_e4m3fn and
bfloat16 conversions, torch.round), used only to pin the C oracle.  Its slot
addressing is written out here from the layout description, not taken from
the oracle.

Layout (per layer, in bytes from the layer's base, 256-byte aligned bases):
  block b occupies [b * block_bytes, (b+1) * block_bytes)
  codes of (position p, head h, K/V c): ((p * Hkv + h) * 2 + c) * row_bytes
  FP32 scale of (p, h, c) (per-token-head modes): bs * Hkv * 2 * row_bytes + ((p * Hkv + h) * 2 + c) * 4
  static table after the last layer: per-tensor [sK, sV], per-head [sK[h]..., sV[h]...]
"""
import numpy as np
import torch

BF16, FP8_PER_TENSOR, FP8_PER_HEAD, FP8_PER_TOKEN_HEAD, INT4_PER_TOKEN_HEAD = range(5)


def row_bytes(mode, hd):
    return {BF16: 2 * hd, INT4_PER_TOKEN_HEAD: hd // 2}.get(mode, hd)


def dynamic(mode):
    return mode in (FP8_PER_TOKEN_HEAD, INT4_PER_TOKEN_HEAD)


def layout(bs, hkv, hd, modes, nblocks):
    bases, off = [], 0
    for m, n in zip(modes, nblocks):
        off = -(-off // 256) * 256
        bases.append(off)
        off += n * (bs * hkv * 2 * row_bytes(m, hd) + (bs * hkv * 8 if dynamic(m) else 0))
    off = -(-off // 256) * 256
    statics = []
    for m in modes:
        statics.append(off)
        off += {FP8_PER_TENSOR: 8, FP8_PER_HEAD: 8 * hkv}.get(m, 0)
    return bases, statics, off


def _e4m3(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32)).clamp(-448, 448)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def store(buf, bs, hkv, hd, modes, nblocks, layer, kbits, vbits, slots, scales=None):
    bases, statics, _ = layout(bs, hkv, hd, modes, nblocks)
    mode = modes[layer]
    rb = row_bytes(mode, hd)
    cb = bs * hkv * 2 * rb
    blk_bytes = cb + (bs * hkv * 8 if dynamic(mode) else 0)
    if mode == FP8_PER_TENSOR or mode == FP8_PER_HEAD:
        sc = np.asarray(scales, np.float32)
        buf[statics[layer]: statics[layer] + 4 * sc.size] = sc.view(np.uint8)
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0 or slot >= nblocks[layer] * bs:
            continue
        blk, pos = divmod(slot, bs)
        for h in range(hkv):
            for c, src in enumerate((kbits, vbits)):
                xb = np.asarray(src[t, h], np.uint16)
                x = (xb.astype(np.uint32) << 16).view(np.float32)
                row_off = bases[layer] + blk * blk_bytes + ((pos * hkv + h) * 2 + c) * rb
                if mode == BF16:
                    buf[row_off: row_off + rb] = xb.view(np.uint8)
                    continue
                if dynamic(mode):
                    a = np.abs(x).max()
                    s = np.float32(a) / np.float32(448.0 if mode == FP8_PER_TOKEN_HEAD else 7.0)
                    so = bases[layer] + blk * blk_bytes + cb + ((pos * hkv + h) * 2 + c) * 4
                    buf[so: so + 4] = np.array([s], np.float32).view(np.uint8)
                elif mode == FP8_PER_TENSOR:
                    s = np.float32(scales[c])
                else:
                    s = np.float32(scales[c * hkv + h])
                if s == 0:                      # only when every element is +-0
                    q = np.where(np.signbit(x), np.float32(-0.0), np.float32(0.0)).astype(np.float32)
                else:
                    q = x / s
                if mode == INT4_PER_TOKEN_HEAD:
                    n = torch.round(torch.from_numpy(q)).clamp(-8, 7).to(torch.int64).numpy()
                    if s == 0:
                        n = np.zeros_like(n)
                    nib = (n & 0xF).astype(np.uint8)
                    buf[row_off: row_off + rb] = nib[0::2] | (nib[1::2] << 4)
                else:
                    buf[row_off: row_off + rb] = _e4m3(q)


def gather(buf, bs, hkv, hd, modes, nblocks, layer, block_table, seq_lens):
    bases, statics, _ = layout(bs, hkv, hd, modes, nblocks)
    mode = modes[layer]
    rb = row_bytes(mode, hd)
    cb = bs * hkv * 2 * rb
    blk_bytes = cb + (bs * hkv * 8 if dynamic(mode) else 0)
    total = int(sum(max(int(n), 0) for n in seq_lens))
    outs = [np.zeros((total, hkv, hd), np.uint16), np.zeros((total, hkv, hd), np.uint16)]
    row = 0
    for b, n in enumerate(seq_lens):
        for t in range(max(int(n), 0)):
            j = t // bs
            if j >= block_table.shape[1]:
                continue
            blk = int(block_table[b, j])
            if blk < 0 or blk >= nblocks[layer]:
                continue
            pos = t % bs
            for h in range(hkv):
                for c in range(2):
                    off = bases[layer] + blk * blk_bytes + ((pos * hkv + h) * 2 + c) * rb
                    raw = buf[off: off + rb]
                    if mode == BF16:
                        outs[c][row + t, h] = raw.view(np.uint16)
                        continue
                    if dynamic(mode):
                        so = bases[layer] + blk * blk_bytes + cb + ((pos * hkv + h) * 2 + c) * 4
                        s = buf[so: so + 4].view(np.float32)[0]
                    elif mode == FP8_PER_TENSOR:
                        s = buf[statics[layer] + 4 * c: statics[layer] + 4 * c + 4].view(np.float32)[0]
                    else:
                        o = statics[layer] + 4 * (c * hkv + h)
                        s = buf[o: o + 4].view(np.float32)[0]
                    if mode == INT4_PER_TOKEN_HEAD:
                        nib = np.empty(hd, np.int64)
                        nib[0::2] = raw & 0xF
                        nib[1::2] = raw >> 4
                        dec = torch.from_numpy(np.where(nib >= 8, nib - 16, nib).astype(np.float32))
                    else:
                        dec = torch.from_numpy(raw.copy()).view(torch.float8_e4m3fn).to(torch.float32)
                    prod = dec * torch.tensor(s, dtype=torch.float32)
                    outs[c][row + t, h] = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        row += max(int(n), 0)
    return outs[0], outs[1]


def dequant_f64(buf, bs, hkv, hd, modes, nblocks, layer, block_table, seq_lens):
    """Exact dequantized K and V (float64 [sum(seq_lens), hkv, hd]): decode(code)
    times the slot's scale, read with this module's own layout arithmetic."""
    bases, statics, _ = layout(bs, hkv, hd, modes, nblocks)
    mode = modes[layer]
    rb = row_bytes(mode, hd)
    cb = bs * hkv * 2 * rb
    blk_bytes = cb + (bs * hkv * 8 if dynamic(mode) else 0)
    total = int(sum(max(int(n), 0) for n in seq_lens))
    outs = [np.zeros((total, hkv, hd)), np.zeros((total, hkv, hd))]
    row = 0
    for b, n in enumerate(seq_lens):
        for t in range(max(int(n), 0)):
            blk, pos = int(block_table[b, t // bs]), t % bs
            for h in range(hkv):
                for c in range(2):
                    off = bases[layer] + blk * blk_bytes + ((pos * hkv + h) * 2 + c) * rb
                    raw = buf[off: off + rb]
                    if mode == BF16:
                        outs[c][row + t, h] = torch.from_numpy(raw.copy()).view(torch.bfloat16).double().numpy()
                        continue
                    if dynamic(mode):
                        so = bases[layer] + blk * blk_bytes + cb + ((pos * hkv + h) * 2 + c) * 4
                        s = float(buf[so: so + 4].view(np.float32)[0])
                    elif mode == FP8_PER_TENSOR:
                        s = float(buf[statics[layer] + 4 * c: statics[layer] + 4 * c + 4].view(np.float32)[0])
                    else:
                        o = statics[layer] + 4 * (c * hkv + h)
                        s = float(buf[o: o + 4].view(np.float32)[0])
                    if mode == INT4_PER_TOKEN_HEAD:
                        nib = np.empty(hd, np.int64)
                        nib[0::2] = raw & 0xF
                        nib[1::2] = raw >> 4
                        dec = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
                    else:
                        dec = torch.from_numpy(raw.copy()).view(torch.float8_e4m3fn).double().numpy()
                    outs[c][row + t, h] = dec * s
        row += max(int(n), 0)
    return outs[0], outs[1]
