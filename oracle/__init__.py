"""CPU oracle for the quantized paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it.

The arithmetic lives in ``kvq_oracle.c`` (plain scalar C, compiled with gcc);
this module only builds it and marshals numpy arrays through ctypes.  Each
function's docstring names the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libkvq_oracle.so")

# Mode numbering shared by the tests' inputs (a plain enumeration, no arithmetic).
BF16, FP8_PER_TENSOR, FP8_PER_HEAD, FP8_PER_TOKEN_HEAD, INT4_PER_TOKEN_HEAD = range(5)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no contraction)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
               "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int
    lib.orc_cache_bytes.argtypes = [I32, I64, I64, I64, P, P, P]
    lib.orc_layer_offsets.argtypes = [I32, I64, I64, I64, P, P, P, P]
    lib.orc_layer_offsets.restype = I64
    lib.orc_store.argtypes = [I32, I64, I64, I64, P, P, P, I32, P, P, P, I64, P]
    lib.orc_gather.argtypes = [I32, I64, I64, I64, P, P, P, I32, P, I64, P, I64, P, P]
    for name in ("orc_e4m3_encode_n", "orc_e4m3_decode_n", "orc_int4_encode_n",
                 "orc_float_to_bf16_n"):
        getattr(lib, name).argtypes = [P, P, I64]
    lib.orc_quotient_n.argtypes = [P, P, P, I64]
    lib.orc_dequant_fp8_n.argtypes = [P, P, P, I64]
    lib.orc_dynamic_scale_n.argtypes = [P, ctypes.c_double, P, I64]
    lib.orc_num_threads.restype = I32
    lib.orc_set_num_threads.argtypes = [I32]
    lib.orc_set_num_threads.restype = None
    lib.orc_calibrate_amax.argtypes = [P, P, I64, I64, I64, P, I32]
    lib.orc_decode_attention.argtypes = [I32, I64, I64, I64, P, P, P, I32, P, I64, P, I64, P, I64,
                                         ctypes.c_double, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Geometry:
    """Cache geometry: layers, block size, KV heads, head_dim, per-layer mode and block count."""

    def __init__(self, block_size, num_kv_heads, head_dim, layer_modes, layer_num_blocks):
        self.bs = int(block_size)
        self.hkv = int(num_kv_heads)
        self.hd = int(head_dim)
        self.modes = _c(layer_modes, np.int32)
        self.nblocks = _c(layer_num_blocks, np.int64)
        assert self.modes.shape == self.nblocks.shape
        self.num_layers = int(self.modes.shape[0])

    def _args(self):
        return (self.num_layers, self.bs, self.hkv, self.hd, _ptr(self.modes), _ptr(self.nblocks))


def cache_bytes(g: Geometry) -> dict:
    """Byte accounting.  Payload and per-slot scale formulas: "Per-token-head KV
    cache scale overhead", sections "Per-token-head KV cache scale overhead" and
    "INT4 makes the metadata fraction larger"; static scale tables: "Per-tensor
    vs per-head FP8 KV cache scales", "Static per-head metadata is almost free";
    BF16 layers: "FP8 KV cache layer skipping vs per-head scales"."""
    out = np.zeros(5, np.int64)
    _load().orc_cache_bytes(*g._args(), _ptr(out))
    return dict(zip(("payload", "token_scales", "static_scales", "padding", "total"),
                    (int(v) for v in out)))


def layer_offsets(g: Geometry):
    """(layer_base[], static_base[], total) of the oracle's own layout."""
    lb = np.zeros(g.num_layers, np.int64)
    sb = np.zeros(g.num_layers, np.int64)
    total = _load().orc_layer_offsets(*g._args(), _ptr(lb), _ptr(sb))
    return lb, sb, int(total)


def new_cache(g: Geometry) -> np.ndarray:
    """A zeroed host image of the whole cache buffer."""
    return np.zeros(cache_bytes(g)["total"], np.uint8)


def store(g: Geometry, buf: np.ndarray, layer: int, keys_bits, values_bits,
          slot_mapping, scales=None) -> None:
    """Quantize-and-store of one layer call ("Per-tensor vs per-head FP8 KV cache
    scales", "Dynamic per-token-head scales add 3.125 percent": reduce over each
    new head vector, write the scales, write the codes into the slot)."""
    assert buf.dtype == np.uint8 and buf.flags.c_contiguous
    k = _c(keys_bits, np.uint16)
    v = _c(values_bits, np.uint16)
    sm = _c(slot_mapping, np.int64)
    n = int(sm.shape[0])
    assert k.size == n * g.hkv * g.hd and v.size == k.size
    mode = int(g.modes[layer])
    if mode in (FP8_PER_TENSOR, FP8_PER_HEAD):
        sc = _c(scales, np.float32)
        assert sc.size == (2 if mode == FP8_PER_TENSOR else 2 * g.hkv)
        sp = _ptr(sc)
    else:
        sc = None
        sp = None
    _load().orc_store(*g._args(), _ptr(buf), int(layer), _ptr(k), _ptr(v), _ptr(sm), n, sp)


def gather(g: Geometry, buf: np.ndarray, layer: int, block_table, seq_lens):
    """Dequantizing paged read of one layer: returns (keys, values) as BF16 bits
    [sum(seq_lens), hkv, hd] ("Per-tensor vs per-head FP8 KV cache scales",
    "Dynamic per-token-head scales add 3.125 percent": scales are read back
    when attention consumes the cache)."""
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    nseq = int(sl.shape[0])
    maxb = int(bt.shape[1]) if bt.ndim == 2 else 0
    total = int(np.clip(sl, 0, None).sum())
    ok = np.zeros((total, g.hkv, g.hd), np.uint16)
    ov = np.zeros((total, g.hkv, g.hd), np.uint16)
    _load().orc_gather(*g._args(), _ptr(buf), int(layer), _ptr(bt), maxb, _ptr(sl), nseq,
                       _ptr(ok), _ptr(ov))
    return ok, ov


def decode_attention(g: Geometry, buf: np.ndarray, layer: int, q_bits, block_table, seq_lens,
                     sm_scale: float, with_absv: bool = False, q_scales=None):
    """Attention of one query token per sequence over its cached tokens, from
    the dequantized cache values, all in double ("Per-tensor vs per-head FP8 KV
    cache scales", "Dynamic per-token-head scales add 3.125 percent": scales
    are read during attention).  q_bits: BF16 bits [num_seqs, H, hd].  Returns
    out [num_seqs, H, hd] (float64) and, if asked, sum_t p_t |V^_t| alike.
    With q_scales ([H] static FP8 query scales, "FP8 KV cache layer skipping vs
    per-head scales", "Per-head scales have fixed overhead"), each query
    element is its E4M3 code under its head's scale, decoded back."""
    q = _c(q_bits, np.uint16)
    nseq, nqh = int(q.shape[0]), int(q.shape[1])
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.zeros((nseq, nqh, g.hd), np.float64)
    absv = np.zeros_like(out) if with_absv else None
    qs = None if q_scales is None else _c(q_scales, np.float32)
    assert qs is None or (qs.size == nqh and (qs > 0).all())
    _load().orc_decode_attention(*g._args(), _ptr(buf), int(layer), _ptr(q), nqh, _ptr(bt), int(bt.shape[1]),
                                 _ptr(sl), nseq, float(sm_scale), _ptr(qs) if qs is not None else None, _ptr(out),
                                 _ptr(absv) if absv is not None else None)
    return (out, absv) if with_absv else out


def query_values(q_bits, q_scales=None) -> np.ndarray:
    """Query elements as attention uses them (float64): BF16 values, or with
    q_scales [H] their E4M3 codes under each head's scale, decoded back."""
    q = _c(q_bits, np.uint16)
    x = (q.astype(np.uint32) << 16).view(np.float32)
    if q_scales is None:
        return x.astype(np.float64)
    s = _c(q_scales, np.float32).reshape(1, -1, 1)
    codes = e4m3_encode(quotient(x, np.broadcast_to(s, x.shape)))
    return e4m3_decode(codes).astype(np.float64) * s.astype(np.float64)


def _token_key_scales(g: Geometry, buf: np.ndarray, layer: int, bt: np.ndarray, lens: np.ndarray,
                      which: int = 0) -> np.ndarray:
    """FP32 K (which = 0) or V (which = 1) scale of every token-head a gather
    of a per-token-head layer reads, [sum(lens), hkv] in the gather's order,
    from the scale trailer of this module's own block layout; 0 for tokens
    whose block is not in the layer."""
    lb, _, _ = layer_offsets(g)
    rb = g.hd // 2 if int(g.modes[layer]) == INT4_PER_TOKEN_HEAD else g.hd
    code_bytes = g.bs * g.hkv * 2 * rb
    block_bytes = code_bytes + g.bs * g.hkv * 8
    out = np.zeros((int(lens.sum()), g.hkv))
    row = 0
    for i, n in enumerate(lens):
        for t in range(int(n)):
            blk = int(bt[i, t // g.bs])
            if 0 <= blk < int(g.nblocks[layer]):
                base = int(lb[layer]) + blk * block_bytes + code_bytes + (t % g.bs) * g.hkv * 8
                out[row] = buf[base: base + g.hkv * 8].view(np.float32).reshape(g.hkv, 2)[:, which]
            row += 1
    return out


def attention_error_bound(g: Geometry, buf: np.ndarray, layer: int, q_bits, block_table, seq_lens,
                          sm_scale: float, ref, absv, static_v_max: float = 1.0, q_scales=None):
    """Per-element bound on |o_kernel - o_exact| for an attention kernel that
    takes the dequantized-cache attention with FP32 accumulation, BF16
    softmax weights (times per-token V scales) in the value product and a
    BF16 output:
      (2^-8 + 2.5 eps_S) * sum_t p_t |V^_t| + 2^-8 |o| + (n + 16) 2^-120 max(1, s_V)
    eps_S = (hd + 4) 2^-24 max_t (sum_d |K^_t[d] q[d]| + b_t) * sm_scale bounds
    the score error of an FP32 dot product of hd exact products (a score
    error e moves each weight by a factor within exp(+-2e)).  b_t is 0 except
    in INT4 layers, whose keys enter the products biased, as n + 8, with the
    FP32 sum (8 / 16) sum(q) subtracted through the initial accumulator:
    the biased terms, the subtracted sum and that sum's own rounding add at
    most 24 s_t sum_d |q[d]| (s_t the token's K scale) to what the rounding
    acts on.  2^-8 covers the BF16 rounding of the weights (2^-9) and of the
    output (2^-9) plus FP32 accumulation and rescaling over fewer than 2^11
    tiles (2^-9); the last term is the FP32 underflow floor (products below
    2^-126 may be lost).  INT4 layers' values enter the value product biased
    too, as (n + 8) / 16, with (8 / 16) sum_t P'_t (the same BF16 weights)
    accumulated beside them and subtracted at the end: the weights' rounding
    cancels between the two, and the FP32 accumulation and rescaling (2^-9
    relative, as above) act on sum_t p_t s_t (|n_t| + 16) / 16 in units of
    the code (s_t the token's V scale), which adds at most
    2^-9 * 16 * sum_t p_t s_t <= 2^-5 max_t s_t to each element.  ref and
    absv are this module's decode_attention results for the same inputs."""
    q = _c(q_bits, np.uint16)
    bt = _c(block_table, np.int32)
    lens = np.clip(_c(seq_lens, np.int64), 0, int(bt.shape[1]) * g.bs)
    nqh = int(q.shape[1])
    group = nqh // g.hkv
    kb, _ = gather(g, buf, layer, bt, lens)
    kabs = np.abs((kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) * (1 + 2.0 ** -8)
    qabs = np.abs(query_values(q, q_scales))
    biased = int(g.modes[layer]) == INT4_PER_TOKEN_HEAD
    ks = _token_key_scales(g, buf, layer, bt, lens) if biased else None
    vs = _token_key_scales(g, buf, layer, bt, lens, which=1) if biased else None
    eps = np.zeros((q.shape[0], nqh))
    vbias = np.zeros((q.shape[0], nqh))
    row0 = 0
    for i, n in enumerate(lens):
        if n:
            kk = kabs[row0: row0 + n]
            for qh in range(nqh):
                dot = kk[:, qh // group, :] @ qabs[i, qh]
                if biased:
                    dot = dot + 24.0 * ks[row0: row0 + n, qh // group] * qabs[i, qh].sum()
                    vbias[i, qh] = 2.0 ** -5 * vs[row0: row0 + n, qh // group].max()
                eps[i, qh] = (g.hd + 4) * 2.0 ** -24 * dot.max() * sm_scale
        row0 += int(n)
    floor = (lens.astype(np.float64)[:, None, None] + 16) * 2.0 ** -120 * max(1.0, float(static_v_max))
    return ((2.0 ** -8 + 2.5 * eps[:, :, None]) * absv + 2.0 ** -8 * np.abs(ref) + vbias[:, :, None] + floor)

def retained_positions(layer_windows, context: int):
    """Retained token-layer positions of one sequence per layer: a
    full-attention layer (window 0) retains the whole context, a sliding layer
    at most its window ("FP8 KV cache layer skipping vs per-head scales",
    "Layer skipping follows retained-token footprint")."""
    return [min(int(context), int(w)) if int(w) > 0 else int(context) for w in layer_windows]


def plan_capacity(bs: int, hkv: int, hd: int, layer_modes, layer_windows, context: int, pool_bytes: int) -> dict:
    """Capacity plan from the pages: A and S ("Layer skipping follows
    retained-token footprint"); each layer's retained positions rounded up to
    whole blocks and priced with this module's own layout; the usable pool
    divided by one sequence's bytes, stepped down until the whole buffer
    (alignment and static scales included) fits ("Per-token-head KV cache
    scale overhead", "Convert bytes into block capacity")."""
    r = retained_positions(layer_windows, context)
    A = sum(r)
    S = sum(x for x, m in zip(r, layer_modes) if int(m) == BF16)
    per_seq = [-(-x // bs) for x in r]
    one = cache_bytes(Geometry(bs, hkv, hd, layer_modes, per_seq))
    seq_bytes = one["payload"] + one["token_scales"]
    n = int(pool_bytes) // seq_bytes

    def total(k):
        return cache_bytes(Geometry(bs, hkv, hd, layer_modes, [k * b for b in per_seq]))["total"]
    while n > 0 and total(n) > pool_bytes:
        n -= 1
    return {"retained_positions": A, "skipped_positions": S, "sequence_bytes": seq_bytes, "max_sequences": n,
            "max_tokens": n * int(context), "buffer_bytes": total(n) if n > 0 else 0,
            "layer_num_blocks": [n * b for b in per_seq]}

def calibrate_amax(keys_bits, values_bits, hkv: int, hd: int, amax=None) -> np.ndarray:
    """Per-(K/V, head) absolute maximum over a batch, float32 [2 * hkv]
    (K heads, then V heads); with amax given, the running maximum continues
    from it ("Per-tensor vs per-head FP8 KV cache scales", "Calibration
    changes which scale layout exists")."""
    k = _c(keys_bits, np.uint16)
    v = _c(values_bits, np.uint16)
    n = k.size // (hkv * hd)
    out = np.zeros(2 * hkv, np.float32) if amax is None else np.array(amax, np.float32).copy()
    _load().orc_calibrate_amax(_ptr(k), _ptr(v), n, hkv, hd, _ptr(out), 0 if amax is None else 1)
    return out


def e4m3_encode(v) -> np.ndarray:
    """Float -> OCP E4M3FN code, nearest with ties to even, saturating at 448."""
    a = _c(v, np.float32)
    out = np.zeros(a.shape, np.uint8)
    _load().orc_e4m3_encode_n(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_decode(c) -> np.ndarray:
    a = _c(c, np.uint8)
    out = np.zeros(a.shape, np.float32)
    _load().orc_e4m3_decode_n(_ptr(a), _ptr(out), a.size)
    return out


def int4_encode(v) -> np.ndarray:
    a = _c(v, np.float32)
    out = np.zeros(a.shape, np.int8)
    _load().orc_int4_encode_n(_ptr(a), _ptr(out), a.size)
    return out


def quotient(x, s) -> np.ndarray:
    """RN32(x / s)."""
    x = _c(x, np.float32)
    s = _c(np.broadcast_to(s, x.shape), np.float32)
    out = np.zeros(x.shape, np.float32)
    _load().orc_quotient_n(_ptr(x), _ptr(s), _ptr(out), x.size)
    return out


def dynamic_scale(a, qmax: float) -> np.ndarray:
    """RN32(a / qmax): 448 for FP8, 7 for INT4."""
    a = _c(a, np.float32)
    out = np.zeros(a.shape, np.float32)
    _load().orc_dynamic_scale_n(_ptr(a), float(qmax), _ptr(out), a.size)
    return out


def float_to_bf16(v) -> np.ndarray:
    a = _c(v, np.float32)
    out = np.zeros(a.shape, np.uint16)
    _load().orc_float_to_bf16_n(_ptr(a), _ptr(out), a.size)
    return out


def dequant_fp8(codes, s) -> np.ndarray:
    """BF16_RNE(RN32(decode(code) * s)) as BF16 bits."""
    c = _c(codes, np.uint8)
    s = _c(np.broadcast_to(s, c.shape), np.float32)
    out = np.zeros(c.shape, np.uint16)
    _load().orc_dequant_fp8_n(_ptr(c), _ptr(s), _ptr(out), c.size)
    return out


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from here on (used to time it)."""
    _load().orc_set_num_threads(int(n))
