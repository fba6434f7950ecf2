"""MI355X-native quantized paged KV cache (kvq): Python binding of libkvq.so.

The binding marshals arguments to the C ABI declared in include/kvq.h and
nothing else: every step of store and gather runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built, importing the binding raises; there is no CPU
fallback.

    import quantized_fp8_int4_amd as kvq
    cfg = kvq.CacheConfig(block_size=16, num_kv_heads=8, head_dim=128,
                          layer_modes=[kvq.FP8_PER_TOKEN_HEAD] * 32,
                          layer_num_blocks=[2048] * 32)
    cache = kvq.Cache(cfg, device="cuda")
    cache.store(layer, keys, values, slot_mapping)
    k, v = cache.gather_dequant(layer, block_table, seq_lens)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch  # loads the HIP runtime that libkvq.so then shares

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libkvq.so")

# kvq_mode
BF16 = 0
FP8_PER_TENSOR = 1
FP8_PER_HEAD = 2
FP8_PER_TOKEN_HEAD = 3
INT4_PER_TOKEN_HEAD = 4
MODE_NAMES = {BF16: "bf16", FP8_PER_TENSOR: "fp8_per_tensor", FP8_PER_HEAD: "fp8_per_head",
              FP8_PER_TOKEN_HEAD: "fp8_per_token_head", INT4_PER_TOKEN_HEAD: "int4_per_token_head"}

# kvq_status
OK, ERR_INVALID_ARG, ERR_MODE_MISMATCH, ERR_BUFFER_TOO_SMALL, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_SPACE = \
    0, -1, -2, -3, -4, -5, -6

EXPORTED_SYMBOLS = ("kvq_cache_bytes", "kvq_create_cache", "kvq_destroy_cache", "kvq_store", "kvq_store_ordered",
                    "kvq_store_follows_order",
                    "kvq_gather_dequant", "kvq_calibrate_amax", "kvq_static_scales",
                    "kvq_decode_attention_workspace", "kvq_decode_attention", "kvq_decode_attention_fp8q",
                    "kvq_decode_attention_noalloc",
                    "kvq_plan_capacity",
                    "kvq_manager_create", "kvq_manager_destroy", "kvq_manager_num_groups", "kvq_manager_layer_group",
                    "kvq_manager_append", "kvq_manager_release", "kvq_manager_tables", "kvq_status_string")


class _Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("layer_mode", ctypes.POINTER(ctypes.c_int32)),
                ("layer_num_blocks", ctypes.POINTER(ctypes.c_int64))]


class _Model(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("layer_mode", ctypes.POINTER(ctypes.c_int32)),
                ("layer_window", ctypes.POINTER(ctypes.c_int32))]


class _Plan(ctypes.Structure):
    _fields_ = [("retained_positions", ctypes.c_int64), ("skipped_positions", ctypes.c_int64),
                ("sequence_bytes", ctypes.c_uint64), ("max_sequences", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64), ("buffer_bytes", ctypes.c_uint64)]


class _Bytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("payload", "token_scales", "static_scales", "padding", "total")]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkvq.so is not built ({LIB_PATH}); run `python quantized_fp8_int4_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kvq_cache_bytes.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Bytes)]
    lib.kvq_create_cache.argtypes = [ctypes.POINTER(_Config), P, ctypes.c_uint64, ctypes.POINTER(P)]
    lib.kvq_destroy_cache.argtypes = [P]
    lib.kvq_store.argtypes = [P, I32, P, P, P, I64, ctypes.c_int, P, P]
    lib.kvq_store_ordered.argtypes = [P, I32, P, P, P, P, I64, ctypes.c_int, P, P]
    lib.kvq_store_follows_order.argtypes = [ctypes.c_int, I32]
    lib.kvq_store_follows_order.restype = I32
    lib.kvq_gather_dequant.argtypes = [P, I32, P, I32, P, I32, P, P, I64, P]
    lib.kvq_calibrate_amax.argtypes = [P, P, I64, I32, I32, P, I32, P]
    lib.kvq_static_scales.argtypes = [P, I32, ctypes.c_int, P]
    lib.kvq_decode_attention_workspace.argtypes = [P, I32, I32, I32, ctypes.POINTER(ctypes.c_uint64)]
    lib.kvq_decode_attention.argtypes = [P, I32, P, I32, P, I32, P, I32, ctypes.c_float, P, P, ctypes.c_uint64, P]
    lib.kvq_decode_attention_fp8q.argtypes = [P, I32, P, P, I32, P, I32, P, I32, ctypes.c_float, P, P,
                                              ctypes.c_uint64, P]
    lib.kvq_decode_attention_noalloc.argtypes = [P, I32, P, I32, P, I32, P, I32, ctypes.c_float, P, P]
    lib.kvq_plan_capacity.argtypes = [ctypes.POINTER(_Model), I64, ctypes.c_uint64, ctypes.POINTER(_Plan), P]
    lib.kvq_manager_create.argtypes = [ctypes.POINTER(_Model), P, I32, ctypes.POINTER(P)]
    lib.kvq_manager_destroy.argtypes = [P]
    lib.kvq_manager_num_groups.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.kvq_manager_layer_group.argtypes = [P, I32, ctypes.POINTER(ctypes.c_int32)]
    lib.kvq_manager_append.argtypes = [P, I32, I32, P]
    lib.kvq_manager_release.argtypes = [P, I32]
    lib.kvq_manager_tables.argtypes = [P, I32, P, I32, I32, P, P]
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    for name in EXPORTED_SYMBOLS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load_library()


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.kvq_status_string(status).decode()} ({status})")


def _check(status: int, where: str) -> None:
    if status != OK:
        raise KVQError(status, where)


@dataclass
class CacheConfig:
    """kvq_cache_config: block_size (power of two <= 1024), num_kv_heads,
    head_dim (64/128/256), and per layer a mode and a block count."""
    block_size: int
    num_kv_heads: int
    head_dim: int
    layer_modes: Sequence[int]
    layer_num_blocks: Sequence[int]

    def _c(self):
        n = len(self.layer_modes)
        modes = (ctypes.c_int32 * n)(*[int(m) for m in self.layer_modes])
        blocks = (ctypes.c_int64 * n)(*[int(b) for b in self.layer_num_blocks])
        cfg = _Config(n, int(self.block_size), int(self.num_kv_heads), int(self.head_dim),
                      ctypes.cast(modes, ctypes.POINTER(ctypes.c_int32)),
                      ctypes.cast(blocks, ctypes.POINTER(ctypes.c_int64)))
        return cfg, (modes, blocks)          # keep the arrays alive with the struct


def kvq_cache_bytes(cfg: CacheConfig) -> dict:
    c, keep = cfg._c()
    out = _Bytes()
    _check(_lib.kvq_cache_bytes(ctypes.byref(c), ctypes.byref(out)), "kvq_cache_bytes")
    return {n: int(getattr(out, n)) for n, _ in _Bytes._fields_}


def kvq_create_cache(cfg: CacheConfig, dev_ptr: int, dev_bytes: int) -> ctypes.c_void_p:
    c, keep = cfg._c()
    h = ctypes.c_void_p()
    _check(_lib.kvq_create_cache(ctypes.byref(c), ctypes.c_void_p(dev_ptr), int(dev_bytes), ctypes.byref(h)),
           "kvq_create_cache")
    return h


def kvq_destroy_cache(handle) -> None:
    _check(_lib.kvq_destroy_cache(handle), "kvq_destroy_cache")


def _stream_ptr(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def kvq_store(handle, layer: int, keys: torch.Tensor, values: torch.Tensor, slot_mapping: torch.Tensor,
              mode: int, scales=None, stream=None, order=None) -> None:
    """keys/values: bf16 [N, Hkv, hd] on the device; slot_mapping: int64 [N] on
    the device; scales: host float32 values for static layers, else None;
    order: None, or int32 [N] on the device, a permutation of the tokens
    (kvq_store_ordered: the tokens taken in that order, the same result)."""
    n = int(slot_mapping.numel())
    kp = _dev(keys, torch.bfloat16, "keys") if n else 0
    vp = _dev(values, torch.bfloat16, "values") if n else 0
    sp = _dev(slot_mapping, torch.int64, "slot_mapping") if n else 0
    if n and (keys.shape != values.shape or keys.shape[0] != n):
        raise ValueError("keys, values and slot_mapping disagree in token count")
    op = 0
    if order is not None:
        if order.dim() != 1 or int(order.numel()) != n:
            raise ValueError("order must be int32 [num_tokens]")
        op = _dev(order, torch.int32, "order") if n else 0
    sc = None
    if scales is not None:
        if isinstance(scales, torch.Tensor):
            scales = scales.detach().cpu().to(torch.float32).reshape(-1).tolist()
        vals = [float(x) for x in scales]
        sc = (ctypes.c_float * len(vals))(*vals)
    if order is None:
        _check(_lib.kvq_store(handle, int(layer), ctypes.c_void_p(kp), ctypes.c_void_p(vp), ctypes.c_void_p(sp),
                              n, int(mode), sc, _stream_ptr(stream, keys.device if n else None)), "kvq_store")
    else:
        _check(_lib.kvq_store_ordered(handle, int(layer), ctypes.c_void_p(kp), ctypes.c_void_p(vp),
                                      ctypes.c_void_p(sp), ctypes.c_void_p(op), n, int(mode), sc,
                                      _stream_ptr(stream, keys.device if n else None)), "kvq_store_ordered")


def kvq_gather_dequant(handle, layer: int, block_table: torch.Tensor, seq_lens: torch.Tensor,
                       out_keys: torch.Tensor, out_values: torch.Tensor, stream=None) -> None:
    """block_table: int32 [num_seqs, max_blocks] on the device; seq_lens: int32
    [num_seqs] on the device; out_*: bf16 [rows, Hkv, hd] on the device.  The
    library writes at most `rows` token rows (out_keys.shape[0]): tokens past
    them are dropped, never written out of bounds."""
    num_seqs = int(seq_lens.numel())
    if num_seqs == 0:
        return
    if out_keys.dim() != 3 or out_keys.shape != out_values.shape:
        raise ValueError("out_keys and out_values must both be [rows, num_kv_heads, head_dim]")
    rows = int(out_keys.shape[0])
    bt = _dev(block_table, torch.int32, "block_table")
    sl = _dev(seq_lens, torch.int32, "seq_lens")
    # an output of zero rows has no device address to pass (and gets no writes)
    ok = _dev(out_keys, torch.bfloat16, "out_keys") if rows else 0
    ov = _dev(out_values, torch.bfloat16, "out_values") if rows else 0
    if block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    _check(_lib.kvq_gather_dequant(handle, int(layer), ctypes.c_void_p(bt), int(block_table.shape[1]),
                                   ctypes.c_void_p(sl), num_seqs, ctypes.c_void_p(ok), ctypes.c_void_p(ov), rows,
                                   _stream_ptr(stream, out_keys.device)), "kvq_gather_dequant")


def kvq_calibrate_amax(keys: torch.Tensor, values: torch.Tensor, amax: torch.Tensor,
                       accumulate: bool = False, stream=None) -> None:
    """Running per-(K/V, head) absolute maximum into amax (float32 [2 * Hkv] on
    the device); keys/values bf16 [N, Hkv, hd] on the device."""
    n = int(keys.shape[0]) if keys.dim() == 3 else 0
    hkv, hd = int(keys.shape[1]), int(keys.shape[2])
    kp = _dev(keys, torch.bfloat16, "keys") if n else 0
    vp = _dev(values, torch.bfloat16, "values") if n else 0
    ap = _dev(amax, torch.float32, "amax")
    if keys.shape != values.shape or amax.numel() != 2 * hkv:
        raise ValueError("keys/values must match and amax must hold 2 * num_kv_heads values")
    _check(_lib.kvq_calibrate_amax(ctypes.c_void_p(kp), ctypes.c_void_p(vp), n, hkv, hd, ctypes.c_void_p(ap),
                                   1 if accumulate else 0, _stream_ptr(stream, amax.device)), "kvq_calibrate_amax")


def kvq_static_scales(amax, num_kv_heads: int, mode: int) -> list:
    """Static scales (host floats) for kvq_store from calibrated maxima."""
    vals = [float(x) for x in (amax.detach().cpu().reshape(-1).tolist() if isinstance(amax, torch.Tensor) else amax)]
    if len(vals) != 2 * num_kv_heads:
        raise ValueError("amax must hold 2 * num_kv_heads values")
    a = (ctypes.c_float * len(vals))(*vals)
    n_out = 2 if mode == FP8_PER_TENSOR else 2 * num_kv_heads
    out = (ctypes.c_float * n_out)()
    _check(_lib.kvq_static_scales(a, int(num_kv_heads), int(mode), out), "kvq_static_scales")
    return [float(x) for x in out]


def kvq_decode_attention_workspace(handle, num_q_heads: int, max_blocks_per_seq: int, num_seqs: int) -> int:
    """Device workspace bytes kvq_decode_attention needs for this call shape."""
    n = ctypes.c_uint64(0)
    _check(_lib.kvq_decode_attention_workspace(handle, int(num_q_heads), int(max_blocks_per_seq), int(num_seqs),
                                               ctypes.byref(n)), "kvq_decode_attention_workspace")
    return int(n.value)


def kvq_decode_attention(handle, layer: int, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                         sm_scale: float, out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                         stream=None, q_scales: Optional[torch.Tensor] = None) -> None:
    """q: bf16 [num_seqs, H, hd] on the device; block_table int32 [num_seqs,
    max_blocks]; seq_lens int32 [num_seqs]; out: bf16 [num_seqs, H, hd];
    workspace: a device tensor of at least kvq_decode_attention_workspace()
    bytes (None when that is 0).  q_scales: float32 [H] on the device for FP8
    queries (kvq_decode_attention_fp8q), else None."""
    num_seqs = int(seq_lens.numel())
    if num_seqs == 0:
        return
    qp = _dev(q, torch.bfloat16, "q")
    op = _dev(out, torch.bfloat16, "out")
    bt = _dev(block_table, torch.int32, "block_table")
    sl = _dev(seq_lens, torch.int32, "seq_lens")
    if q.dim() != 3 or q.shape[0] != num_seqs or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    wp, wb = 0, 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if q_scales is None:
        _check(_lib.kvq_decode_attention(handle, int(layer), ctypes.c_void_p(qp), int(q.shape[1]), ctypes.c_void_p(bt),
                                         int(block_table.shape[1]), ctypes.c_void_p(sl), num_seqs, float(sm_scale),
                                         ctypes.c_void_p(op), ctypes.c_void_p(wp), wb, _stream_ptr(stream, q.device)),
               "kvq_decode_attention")
        return
    sp = _dev(q_scales, torch.float32, "q_scales")
    if q_scales.numel() != q.shape[1]:
        raise ValueError("q_scales must hold one scale per query head")
    _check(_lib.kvq_decode_attention_fp8q(handle, int(layer), ctypes.c_void_p(qp), ctypes.c_void_p(sp), int(q.shape[1]),
                                          ctypes.c_void_p(bt), int(block_table.shape[1]), ctypes.c_void_p(sl), num_seqs,
                                          float(sm_scale), ctypes.c_void_p(op), ctypes.c_void_p(wp), wb,
                                          _stream_ptr(stream, q.device)), "kvq_decode_attention_fp8q")


# Bytes of the fixed device array behind kvq_decode_attention_noalloc.
ATTENTION_SCRATCH_BYTES = 32 << 20


def kvq_decode_attention_noalloc(handle, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                                 seq_lens: torch.Tensor, sm_scale: float, out: torch.Tensor, stream=None) -> None:
    """kvq_decode_attention without a workspace: the library keeps the split
    partials in a fixed per-GPU device array and allocates nothing.  Calls
    that overlap on one GPU share that array and race."""
    num_seqs = int(seq_lens.numel())
    if num_seqs == 0:
        return
    qp = _dev(q, torch.bfloat16, "q")
    op = _dev(out, torch.bfloat16, "out")
    bt = _dev(block_table, torch.int32, "block_table")
    sl = _dev(seq_lens, torch.int32, "seq_lens")
    if q.dim() != 3 or q.shape[0] != num_seqs or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    _check(_lib.kvq_decode_attention_noalloc(handle, int(layer), ctypes.c_void_p(qp), int(q.shape[1]),
                                             ctypes.c_void_p(bt), int(block_table.shape[1]), ctypes.c_void_p(sl),
                                             num_seqs, float(sm_scale), ctypes.c_void_p(op),
                                             _stream_ptr(stream, q.device)), "kvq_decode_attention_noalloc")


@dataclass
class ModelConfig:
    """kvq_model_config: a cache geometry without block counts, plus each
    layer's window (0 = full attention, W > 0 = sliding window of W tokens)."""
    block_size: int
    num_kv_heads: int
    head_dim: int
    layer_modes: Sequence[int]
    layer_windows: Sequence[int]

    def _c(self):
        n = len(self.layer_modes)
        modes = (ctypes.c_int32 * n)(*[int(m) for m in self.layer_modes])
        wins = (ctypes.c_int32 * n)(*[int(w) for w in self.layer_windows])
        m = _Model(n, int(self.block_size), int(self.num_kv_heads), int(self.head_dim),
                   ctypes.cast(modes, ctypes.POINTER(ctypes.c_int32)), ctypes.cast(wins, ctypes.POINTER(ctypes.c_int32)))
        return m, (modes, wins)

    def cache_config(self, layer_num_blocks) -> CacheConfig:
        return CacheConfig(self.block_size, self.num_kv_heads, self.head_dim, list(self.layer_modes),
                           [int(b) for b in layer_num_blocks])


def kvq_plan_capacity(model: ModelConfig, context: int, pool_bytes: int):
    """Returns (plan dict, per-layer block counts) for sequences of `context`
    tokens in a usable pool of pool_bytes."""
    m, keep = model._c()
    out = _Plan()
    blocks = (ctypes.c_int64 * len(model.layer_modes))()
    _check(_lib.kvq_plan_capacity(ctypes.byref(m), int(context), int(pool_bytes), ctypes.byref(out), blocks),
           "kvq_plan_capacity")
    plan = {k: int(getattr(out, k)) for k, _ in _Plan._fields_}
    return plan, [int(b) for b in blocks]


class SeqManager:
    """The decode-time block manager (kvq_manager_*): slots for new tokens per
    layer group, and block tables / lengths per group."""

    def __init__(self, model: ModelConfig, layer_num_blocks, max_blocks_per_seq: int):
        m, keep = model._c()
        nb = (ctypes.c_int64 * len(layer_num_blocks))(*[int(b) for b in layer_num_blocks])
        h = ctypes.c_void_p()
        _check(_lib.kvq_manager_create(ctypes.byref(m), nb, int(max_blocks_per_seq), ctypes.byref(h)),
               "kvq_manager_create")
        self.handle = h
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        g = ctypes.c_int32()
        _check(_lib.kvq_manager_num_groups(self.handle, ctypes.byref(g)), "kvq_manager_num_groups")
        self.num_groups = int(g.value)

    def close(self):
        if getattr(self, "handle", None) is not None:
            _lib.kvq_manager_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def layer_group(self, layer: int) -> int:
        g = ctypes.c_int32()
        _check(_lib.kvq_manager_layer_group(self.handle, int(layer), ctypes.byref(g)), "kvq_manager_layer_group")
        return int(g.value)

    def append(self, seq: int, n: int):
        """Slots (list per group, n int64 each) of n new tokens of sequence seq."""
        buf = (ctypes.c_int64 * max(1, self.num_groups * int(n)))()
        _check(_lib.kvq_manager_append(self.handle, int(seq), int(n), buf), "kvq_manager_append")
        flat = list(buf)[: self.num_groups * int(n)]
        return [flat[g * n: (g + 1) * n] for g in range(self.num_groups)]

    def release(self, seq: int) -> None:
        _check(_lib.kvq_manager_release(self.handle, int(seq)), "kvq_manager_release")

    def tables(self, group: int, seqs, max_blocks=None):
        """(block_table [len(seqs)][max_blocks], seq_lens [len(seqs)]) as lists."""
        mb = int(max_blocks or self.max_blocks_per_seq)
        ns = len(seqs)
        sq = (ctypes.c_int32 * max(1, ns))(*[int(x) for x in seqs])
        bt = (ctypes.c_int32 * max(1, ns * mb))()
        sl = (ctypes.c_int32 * max(1, ns))()
        _check(_lib.kvq_manager_tables(self.handle, int(group), sq, ns, mb, bt, sl), "kvq_manager_tables")
        flat = list(bt)
        return [flat[i * mb: (i + 1) * mb] for i in range(ns)], list(sl)[:ns]

class Cache:
    """A cache buffer (zeroed torch uint8 tensor of kvq_cache_bytes().total
    bytes) plus its library handle."""

    def __init__(self, cfg: CacheConfig, device="cuda", buffer: Optional[torch.Tensor] = None):
        self.cfg = cfg
        self.bytes = kvq_cache_bytes(cfg)
        if buffer is None:
            buffer = torch.zeros(self.bytes["total"], dtype=torch.uint8, device=device)
        if buffer.dtype != torch.uint8 or buffer.numel() < self.bytes["total"]:
            raise ValueError("buffer must be uint8 with at least kvq_cache_bytes().total elements")
        self.buffer = buffer
        self.device = buffer.device
        self.handle = kvq_create_cache(cfg, buffer.data_ptr(), buffer.numel())

    def close(self):
        if getattr(self, "handle", None) is not None:
            kvq_destroy_cache(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _rows(self, name, t, first=None):
        # the C ABI cannot see a device buffer's size: shapes are checked here,
        # before any launch, so a wrong one never reaches a kernel
        want = (self.cfg.num_kv_heads, self.cfg.head_dim)
        if t.dim() != 3 or tuple(t.shape[1:]) != want or (first is not None and t.shape[0] != first):
            lead = "N" if first is None else str(first)
            raise ValueError(f"{name} must be [{lead}, {want[0]}, {want[1]}], got {tuple(t.shape)}")

    def store(self, layer, keys, values, slot_mapping, scales=None, stream=None, order=None):
        """order: None, or a permutation of the tokens (int32 on the device)
        in which to take them; the slot order (argsort of slot_mapping),
        shared by every layer of a step, makes the writes sequential.  The
        cache contents are the same either way."""
        n = int(slot_mapping.numel())
        self._rows("keys", keys, n)
        self._rows("values", values, n)
        kvq_store(self.handle, layer, keys, values, slot_mapping, self.cfg.layer_modes[layer], scales, stream,
                  order)

    def check_slots(self, layer, slot_mapping) -> int:
        """Debug check of a store's slot_mapping, off the store path: raises
        ValueError when two tokens name the same slot of the layer (kvq_store
        leaves which one lands undefined); returns how many tokens the store
        will skip (negative slots or slots past the layer's blocks)."""
        s = slot_mapping.detach().to(torch.int64).flatten()
        nslots = int(self.cfg.layer_num_blocks[layer]) * int(self.cfg.block_size)
        kept = s[(s >= 0) & (s < nslots)]
        if torch.unique(kept).numel() != kept.numel():
            raise ValueError(f"layer {layer}: slot_mapping names a slot more than once")
        return int(s.numel() - kept.numel())

    def gather_dequant(self, layer, block_table, seq_lens, total_tokens=None, out=None, stream=None):
        """Returns (keys, values) bf16 [sum(seq_lens), Hkv, hd].  Pass
        total_tokens (or out) to avoid reading seq_lens back to the host.  The
        kernel writes at most as many token rows as the output holds; an out
        shorter than total_tokens, or one of zero rows without total_tokens=0
        (which states that every sequence is empty), is refused here, since
        it would silently drop tokens."""
        if out is not None:
            self._rows("out[0]", out[0])
            self._rows("out[1]", out[1], int(out[0].shape[0]))
            rows = int(out[0].shape[0])
            if total_tokens is not None and rows < int(total_tokens):
                raise ValueError(f"out holds {rows} rows, fewer than total_tokens={int(total_tokens)}")
            if rows == 0 and total_tokens is None and int(seq_lens.numel()) > 0:
                raise ValueError("out holds no rows: pass total_tokens=0 if every sequence is empty")
        else:
            if total_tokens is None:
                total_tokens = int(seq_lens.clamp(min=0).sum().item())
            shape = (int(total_tokens), self.cfg.num_kv_heads, self.cfg.head_dim)
            out = (torch.empty(shape, dtype=torch.bfloat16, device=self.device),
                   torch.empty(shape, dtype=torch.bfloat16, device=self.device))
        kvq_gather_dequant(self.handle, layer, block_table, seq_lens, out[0], out[1], stream)
        return out

    def decode_attention(self, layer, q, block_table, seq_lens, sm_scale, out=None, workspace=None, stream=None,
                         q_scales=None):
        """Fused decode attention over one layer; returns bf16 [num_seqs, H, hd].
        Allocates the workspace with torch when none is given.  q_scales
        (float32 [H] on the device) selects FP8 queries."""
        if q.dim() != 3 or q.shape[2] != self.cfg.head_dim or q.shape[1] % self.cfg.num_kv_heads:
            raise ValueError(f"q must be [num_seqs, H, {self.cfg.head_dim}] with H a multiple of "
                             f"{self.cfg.num_kv_heads}, got {tuple(q.shape)}")
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            nbytes = kvq_decode_attention_workspace(self.handle, q.shape[1], block_table.shape[1], seq_lens.numel())
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device) if nbytes else None
        kvq_decode_attention(self.handle, layer, q, block_table, seq_lens, sm_scale, out, workspace, stream, q_scales)
        return out
