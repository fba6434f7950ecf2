"""Seeded synthetic inputs for the KV-cache quantizer -- shared by the oracle
side and the HIP side of every test and benchmark.

This module draws numbers and lays out indices.  It holds none of the
method's arithmetic: no per-token-head absmax, no scale, no calibration, no
quantization and no layout addressing.  (The tiny draw rescales each head of
its FP32 sample to a chosen maximum before the BF16 cast; that shapes the
input, as the pages' range example does, and no result of the method comes
from it.)  Static scales for the static layouts are derived by each side's
own calibration (the library's kvq_calibrate_amax, the oracle's
calibrate_amax).  Everything is returned as torch tensors on the requested device;
callers copy to the host when the oracle needs them.

The shapes follow the pages' own geometries: the 32-layer, 8-KV-head,
head_dim-128 model and the 80-layer 128K-token example ("Per-token-head KV
cache scale overhead", "Work a 32-layer GQA model"; "Per-tensor vs per-head
FP8 KV cache scales", "Static per-head metadata is almost free"), and the
gpt-oss-20b shape with 128-token sliding windows ("FP8 KV cache layer skipping
vs per-head scales", "Work the gpt-oss-20b numbers").  The pages measure on no
public data set for this path; these draws stand in for their
"production-shaped data".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Mode numbering of the C ABI (kvq_mode); a plain enumeration.
BF16, FP8_PER_TENSOR, FP8_PER_HEAD, FP8_PER_TOKEN_HEAD, INT4_PER_TOKEN_HEAD = range(5)
MODE_NAMES = {
    BF16: "bf16",
    FP8_PER_TENSOR: "fp8_per_tensor",
    FP8_PER_HEAD: "fp8_per_head",
    FP8_PER_TOKEN_HEAD: "fp8_per_token_head",
    INT4_PER_TOKEN_HEAD: "int4_per_token_head",
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


# --------------------------------------------------------------------------
# Value distributions
# --------------------------------------------------------------------------

def normal_kv(n_tokens, hkv, hd, seed, device="cpu"):
    """K then V, each bf16 [n, hkv, hd] ~ N(0, 1) (fp32 draw, RNE cast)."""
    g = _gen(seed, device)
    k = _randn((n_tokens, hkv, hd), g, device).to(torch.bfloat16)
    v = _randn((n_tokens, hkv, hd), g, device).to(torch.bfloat16)
    return k, v


def tiny_kv(seed=0, device="cpu", n_tokens=64, hkv=2, hd=64, head_absmax=(2.0, 32.0)):
    """Tiny case: N(0,1) with head h rescaled so its absolute maximum is
    head_absmax[h] (2 and 32: the pages' range-sharing example)."""
    g = _gen(seed, device)
    out = []
    for _ in range(2):                      # K, then V
        z = _randn((n_tokens, hkv, hd), g, device)
        for h in range(hkv):
            z[:, h, :] *= head_absmax[h % len(head_absmax)] / z[:, h, :].abs().max()
        out.append(z.to(torch.bfloat16))
    return out[0], out[1]


def gqa_kv(n_tokens, hkv, hd, seed, device="cpu", sigma_lo=0.25, sigma_hi=16.0,
           outlier_p=1e-3, outlier_mult=20.0):
    """Per-(K/V, head) std drawn log-uniform in [sigma_lo, sigma_hi], x = std * z,
    with Bernoulli(outlier_p) elements multiplied by outlier_mult."""
    g = _gen(seed, device)
    out = []
    for _ in range(2):
        u = torch.rand((hkv,), generator=g, device=device, dtype=torch.float32)
        sigma = torch.exp(math.log(sigma_lo) + u * (math.log(sigma_hi) - math.log(sigma_lo)))
        z = _randn((n_tokens, hkv, hd), g, device) * sigma.view(1, hkv, 1)
        mask = torch.rand((n_tokens, hkv, hd), generator=g, device=device) < outlier_p
        z = torch.where(mask, z * outlier_mult, z)
        out.append(z.to(torch.bfloat16))
    return out[0], out[1]


def heavy_tail_kv(n_tokens, hkv, hd, seed, device="cpu"):
    """Even KV heads N(0,1); odd KV heads Student-t with 3 degrees of freedom,
    z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)."""
    g = _gen(seed, device)
    out = []
    for _ in range(2):
        z = _randn((n_tokens, hkv, hd), g, device)
        chi = (_randn((3, n_tokens, hkv, hd), g, device) ** 2).sum(0) / 3.0
        t3 = z / torch.sqrt(chi)
        odd = (torch.arange(hkv, device=device) % 2 == 1).view(1, hkv, 1)
        out.append(torch.where(odd, t3, z).to(torch.bfloat16))
    return out[0], out[1]


# --------------------------------------------------------------------------
# Slot mappings and block tables
# --------------------------------------------------------------------------

def identity_slots(n_tokens, device="cpu"):
    return torch.arange(n_tokens, dtype=torch.int64, device=device)


def permuted_block_table(num_seqs, blocks_per_seq, num_blocks, seed, device="cpu"):
    """block_table[b][j] = perm[b * blocks_per_seq + j] of a seeded permutation."""
    g = _gen(seed, "cpu")
    perm = torch.randperm(num_blocks, generator=g)[: num_seqs * blocks_per_seq]
    return perm.view(num_seqs, blocks_per_seq).to(torch.int32).to(device)


def slots_from_block_table(block_table, seq_lens, block_size, device="cpu"):
    """Prefill slot of every token, sequences packed in order."""
    bt = block_table.cpu().long()
    out = []
    for b, n in enumerate(seq_lens):
        t = torch.arange(int(n), dtype=torch.int64)
        out.append(bt[b, t // block_size] * block_size + t % block_size)
    return torch.cat(out).to(device)


def ring_slots(n_tokens, window, device="cpu"):
    """Sliding-window ring buffer: token t is kept at slot t mod window when it
    is among the last `window` tokens, else skipped (-1)."""
    t = torch.arange(n_tokens, dtype=torch.int64)
    s = torch.where(t >= n_tokens - window, t % window, torch.full_like(t, -1))
    return s.to(device)


def ring_block_table(window, block_size, device="cpu"):
    return torch.arange(window // block_size, dtype=torch.int32, device=device).view(1, -1)


@dataclass
class DecodeState:
    """Paged allocation for many sequences: a seeded random free list of blocks
    from which each sequence pops blocks as it grows."""
    num_seqs: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    seed: int
    free: list = field(default_factory=list)
    block_table: torch.Tensor = None
    seq_lens: list = field(default_factory=list)

    def __post_init__(self):
        g = _gen(self.seed, "cpu")
        self.free = torch.randperm(self.num_blocks, generator=g).tolist()
        self.free.reverse()                  # pop() takes perm[0] first
        self.block_table = torch.full((self.num_seqs, self.max_blocks_per_seq), -1, dtype=torch.int32)
        self.seq_lens = [0] * self.num_seqs

    def append(self, b: int, n: int):
        """Reserve n more tokens for sequence b; returns their slots (int64)."""
        t0 = self.seq_lens[b]
        t = torch.arange(t0, t0 + n, dtype=torch.int64)
        j = t // self.block_size
        first_new = (t0 + self.block_size - 1) // self.block_size    # first block index not yet held
        last = (t0 + n - 1) // self.block_size if n > 0 else first_new - 1
        for jj in range(first_new, last + 1):
            self.block_table[b, jj] = self.free.pop()
        self.seq_lens[b] = t0 + n
        return (self.block_table[b].to(torch.int64)[j] * self.block_size + t % self.block_size).tolist()


# --------------------------------------------------------------------------
# The five workloads (sizes as named; the first is small enough for the oracle)
# --------------------------------------------------------------------------

WORKLOADS = {
    "tiny": dict(num_layers=1, hkv=2, hd=64, block_size=16, n_tokens=64,
                 desc="1 layer, 2 KV heads, head_dim 64, 64 tokens, block 16, heads at absmax 2 and 32"),
    "gqa32": dict(num_layers=32, hkv=8, hd=128, block_size=16, num_seqs=8, seq_len=4096,
                  desc="32 layers, 8 KV heads, head_dim 128, block 16, prefill 8 x 4096 tokens per layer call"),
    "long80": dict(num_layers=80, hkv=8, hd=128, block_size=16, num_seqs=1, seq_len=131072,
                   desc="80 layers, 8 KV heads, head_dim 128, one 131072-token sequence"),
    "gptoss": dict(num_layers=24, hkv=8, hd=64, block_size=16, seq_len=32768, window=128,
                   desc="24 layers alternating sliding (W=128, BF16 ring) and full (per-token-head FP8), 8 KV heads, head_dim 64, 32768 tokens"),
    "decode": dict(num_layers=32, hkv=8, block_size=16, num_seqs=256, context=8192, steps=16,
                   desc="256 sequences x 8192-token context, 8 KV heads, 32 layers, 1 token appended per step"),
}


def gptoss_layer_is_sliding(layer: int) -> bool:
    """Even layers sliding, odd layers full (the pages say only that they alternate)."""
    return layer % 2 == 0
