#!/usr/bin/env python3
"""Benchmark of the quantized paged KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: quantize-and-store
of every layer's new K/V (kvq_store), then the dequantizing paged read of
every layer (kvq_gather_dequant).  Default workload: the 32-layer GQA shape
(8 KV heads, head_dim 128, blocks of 16 tokens), a prefill of 8 sequences x
4096 tokens per layer call, dynamic per-token-head FP8, synthetic inputs
(per-head std log-uniform in [0.25, 16], 0.1% outliers x20) resident in HBM
before timing.  Every layer has its own inputs, cache region and output
buffers, so a step streams ~10 GiB and nothing is served from the 256 MB
Infinity Cache.

Prints one JSON line (rank 0).  Algorithmic bytes per token-head (no
padding, no re-reads):
  store  = 4*hd (BF16 K+V in) + 2*row_bytes (codes out) + 8 (FP32 scales, per-token-head)
           + 8/Hkv (int64 slot)
  gather = 2*row_bytes + 8 + 4/(block_size*Hkv) (int32 block-table entry) + 4*hd (BF16 out)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_gqa32_all_layouts.md")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_fp8_int4_amd", "csrc", f)
                  for f in ("kvq_kernels.hip", "kvq_device.h", "kvq_exact.h")]
METRIC = "kvq_store/gather GB/s and % of HBM peak; cached tokens/s (per-token-head FP8)"
COPY_BYTES = 256 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def row_bytes(mode, hd):
    import quantized_fp8_int4_amd as kvq
    return {kvq.BF16: 2 * hd, kvq.INT4_PER_TOKEN_HEAD: hd // 2}.get(mode, hd)


def algorithmic_bytes(mode, hd, hkv, bs, token_heads):
    import quantized_fp8_int4_amd as kvq
    rb = row_bytes(mode, hd)
    sigma = 8 if mode in (kvq.FP8_PER_TOKEN_HEAD, kvq.INT4_PER_TOKEN_HEAD) else 0
    store = token_heads * (4 * hd + 2 * rb + sigma) + token_heads * 8 / hkv
    gather = token_heads * (2 * rb + sigma + 4 * hd) + token_heads * 4 / (bs * hkv)
    return store, gather


CEILING_LIB = os.path.join(ROOT, "ceiling", "_build", "libkvq_ceiling.so")


def _ceiling_lib():
    """The bench-only ceiling kernels (ceiling/copy_ceiling.hip, built by
    __graft_entry__.build()); not part of libkvq.so."""
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(CEILING_LIB)
    P = ctypes.c_void_p
    lib.ceil_linear_copy.argtypes = [P, P, ctypes.c_uint64, P]
    lib.ceil_store_pattern.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P]
    I32 = ctypes.c_int32
    lib.ceil_gather_pattern.argtypes = [P, P, I32, P, I32, P, P, I32, I32, I32, I32, I32, ctypes.c_int64, P]
    lib.ceil_empty.argtypes = [ctypes.c_int64, P]
    return lib


def _time_launches(torch, launches, reps, warmup=2):
    """Mean seconds per launch of a list of launch closures, run back to back
    `reps` times on the current stream between HIP events on that stream."""
    for _ in range(warmup):
        for f in launches:
            f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for f in launches:
            f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * len(launches))


def _rate(nbytes, sec):
    gbps = nbytes / sec / 1e9
    return {"bytes": int(nbytes), "us": round(sec * 1e6, 2), "GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def gather_pattern_ceiling(torch, I, LA, bt, reps, cache_buf):
    """The gather's exact loads and stores (block table, sequence offsets,
    code chunks and row scales of the layout's blocks, every layer's BF16
    output rows) with no arithmetic, reading a buffer laid out like the
    layout's cache."""
    import ctypes
    lib = _ceiling_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rb = row_bytes(LA["mode"], I["hd"])
    sc = 8 if LA["dynamic"] else 0

    def mk(layer):
        base = cache_buf.data_ptr() + LA["layer_base"][layer]
        ok, ov = I["outs"][layer]

        def f():
            if lib.ceil_gather_pattern(ctypes.c_void_p(base), ctypes.c_void_p(bt.data_ptr()), bt.shape[1],
                                       ctypes.c_void_p(I["seq_lens"].data_ptr()), I["nseq"],
                                       ctypes.c_void_p(ok.data_ptr()), ctypes.c_void_p(ov.data_ptr()), I["hkv"],
                                       I["hd"], rb, sc, I["bs"], I["nblocks"], stream):
                raise RuntimeError("ceil_gather_pattern failed")
        return f
    sec = _time_launches(torch, [mk(l) for l in range(I["L"])], reps)
    return _rate(LA["gather_bytes"], sec)


def linear_copy_ceiling(torch, nbytes, buffers, reps):
    """A non-temporal linear copy moving nbytes per launch (nbytes / 2 read,
    nbytes / 2 written), rotating over `buffers` source/destination pairs so
    that the 256 MB Infinity Cache holds none of them."""
    import ctypes
    lib = _ceiling_lib()
    half = (int(nbytes) // 2 + 15) // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"), torch.empty(half, dtype=torch.uint8, device="cuda"))
             for _ in range(buffers)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def mk(src, dst):
        def f():
            if lib.ceil_linear_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), half, stream):
                raise RuntimeError("ceil_linear_copy failed")
        return f
    sec = _time_launches(torch, [mk(s_, d_) for s_, d_ in pairs], reps)
    del pairs
    torch.cuda.empty_cache()
    return _rate(2 * half, sec)


def empty_launch_us(torch, grids, reps=200):
    """Microseconds per launch of a kernel that does nothing, launched back
    to back on the current stream, for each grid (workgroups of 256)."""
    import ctypes
    lib = _ceiling_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for g in grids:
        def f(g=g):
            if lib.ceil_empty(g, stream):
                raise RuntimeError("ceil_empty failed")
        out[f"grid_{g}"] = round(_time_launches(torch, [f], reps) * 1e6, 2)
    return out


def store_pattern_ceiling(torch, I, LA, slots, reps, out_buf, order=None):
    """The store's exact loads and stores (every layer's own K/V, the given
    slots, the layer's code rows and scale trailer) with no arithmetic,
    written to a scratch buffer laid out like the layout's cache; with an
    order (int32 permutation on the device), the tokens taken in it."""
    import ctypes
    lib = _ceiling_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rb = row_bytes(LA["mode"], I["hd"])
    sc = 8 if LA["dynamic"] else 0

    def mk(layer):
        base = out_buf.data_ptr() + LA["layer_base"][layer]
        k, v = I["keys"][layer], I["values"][layer]

        def f():
            if lib.ceil_store_pattern(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                      ctypes.c_void_p(slots.data_ptr()),
                                      ctypes.c_void_p(order.data_ptr() if order is not None else 0),
                                      ctypes.c_void_p(base), I["n"], I["hkv"],
                                      I["hd"], rb, sc, I["bs"], I["nblocks"], stream):
                raise RuntimeError("ceil_store_pattern failed")
        return f
    sec = _time_launches(torch, [mk(l) for l in range(I["L"])], reps)
    return _rate(LA["store_bytes"], sec)


def kernel_source_hash(sources=None):
    """Hash of the sources a kernel is built from (default: store and gather)."""
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


ATTN_SOURCES = [os.path.join(ROOT, "quantized_fp8_int4_amd", "csrc", f)
                for f in ("kvq_attention.hip", "kvq_device.h", "kvq_exact.h")]


def attention_profile_paths(mode_name, hd, tp=1):
    base = f"attention_decode_{mode_name}_hd{hd}.md" if tp == 1 else f"attention_decode_tp{tp}_{mode_name}_hd{hd}.md"
    return (os.path.join(ROOT, "profiles", "kernel_trace_" + base), os.path.join(ROOT, "profiles", "traffic_" + base))


def measured_attention_traffic(mode_name, hd, tp=1):
    """Per-launch HBM bytes of the attention kernel from the committed counter
    summary, if it was taken on the current kernel source."""
    path = attention_profile_paths(mode_name, hd, tp)[1]
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch\[attention\]:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash(ATTN_SOURCES):
        return None
    return float(m_val.group(1))


def measured_traffic(path=PROFILE_TRAFFIC):
    """Per-launch HBM bytes of each profiled kernel ("store/128/3": kind,
    head_dim, mode) from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return None
    vals = dict(re.findall(r"traffic_bytes_per_launch\[([\w/]+)\]:\s*([0-9.eE+]+)", text))
    return {k: float(v) for k, v in vals.items()}


def _kernel_key(name):
    """(kind/head_dim/mode, short name) of a library or ceiling kernel's
    demangled name, or None for other kernels."""
    m = re.search(r"\b(store_kernel|gather_kernel|attention_kernel|attention_quad_kernel|attention_tquad_kernel|"
                  r"combine_kernel|"
                  r"combine_wide_kernel|calib_kernel|"
                  r"store_pattern_kernel|gather_pattern_kernel|linear_copy_kernel)(?:<([^>]*)>)?", name)
    if not m:
        return None
    kind = m.group(1).replace("_kernel", "")
    short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
    targs = [t.strip() for t in (m.group(2) or "").split(",") if t.strip()]
    # library kernels by head_dim and mode; the ceiling kernels by all their arguments
    keep = targs[:2] if kind in ("store", "gather", "attention", "attention_quad", "attention_tquad", "calib") else targs
    # the store that follows a token order (its last template argument) apart
    if kind == "store" and len(targs) >= 10 and targs[9] == "true":
        keep = keep + ["ordered"]
    return "/".join([kind] + keep), short


def _read_csv(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_per_kernel(rows, counter, names=None):
    """Mean counter value (KiB) per dispatch of the store kernel, the gather
    kernel, the attention and combine kernels and the calibration copy (the
    largest device-to-device copies); names, if given, receives each kind's
    kernel name."""
    acc = {}
    copies = []
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        if names is not None and "kvq" in name:
            short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
            for kind in ("store", "gather", "combine"):
                if kind + "_kernel" in name:
                    names.setdefault(kind, short)
            if "attention" in name:
                names.setdefault("attention", short)
        if "store_kernel" in name:
            acc.setdefault("store", []).append(val)
        elif "gather_kernel" in name:
            acc.setdefault("gather", []).append(val)
        elif "attention_kernel" in name or "attention_quad_kernel" in name or "attention_tquad_kernel" in name:
            acc.setdefault("attention", []).append(val)
        elif "combine_kernel" in name:
            acc.setdefault("combine", []).append(val)
        elif "copyBuffer" in name:
            copies.append(val)
    top = max(copies)
    acc["copy"] = [v for v in copies if v >= 0.5 * top]
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def attention_kernel_name(mode, hd, group, block_size, hkv, q_fp8):
    """The decode-attention kernel the library picks for a call (a label for
    the JSON line): quads of KV heads for per-token-head layers (FP8 at
    head_dim 64, INT4 at 64 and 128 with BF16 queries), groups of at most 4
    and blocks of at least 16 tokens, when a workgroup holds 4 or 8 KV heads;
    quads of tiles on the same layers when it holds 1 or 2, and on FP8 at
    head_dim 128 when it holds 2; else the one-head kernel."""
    import quantized_fp8_int4_amd as kvq
    quad_layer = ((mode == kvq.FP8_PER_TOKEN_HEAD and hd == 64) or
                  (mode == kvq.INT4_PER_TOKEN_HEAD and hd in (64, 128) and not q_fp8))
    tile_layer = quad_layer or (mode == kvq.FP8_PER_TOKEN_HEAD and hd == 128 and not q_fp8)
    if not tile_layer or block_size < 16 or group > 4:
        return "attention_kernel"
    hpw = 1
    while hpw < 8 and hkv % (2 * hpw) == 0:
        hpw *= 2
    if hpw % 4 == 0:
        return "attention_quad_kernel" if quad_layer else "attention_kernel"
    return "attention_tquad_kernel" if quad_layer or hpw == 2 else "attention_kernel"


def summarize_attention_profiles(kt_dir, fetch_dir, write_dir, mode_name, hd, layers=0, tp=1):
    """profiles/ summaries of the decode-attention workload from three
    rocprofv3 runs of bench.py --workload attention (kernel trace with
    --stats; --pmc FETCH_SIZE; --pmc WRITE_SIZE, the latter two with
    --calibrate-copy); layers > 0 when the runs took --layers (a cache of
    32 layers that would not fit in HBM); tp > 1 for a tensor-parallel
    shard's share of the heads (8/tp KV and 32/tp query heads)."""
    kt_path, tr_path = attention_profile_paths(mode_name, hd, tp)
    args_s = (f"--workload attention --mode {mode_name} --head-dim {hd}" + (f" --layers {layers}" if layers else "") +
              (f" --tp {tp}" if tp > 1 else ""))
    hkv, H = 8 // tp, 32 // tp
    stats = _read_csv(kt_dir, "kernel_stats.csv")
    lines = [f"# Kernel trace: decode attention, 256 x 8192 tokens, {H} query / {hkv} KV heads, {mode_name}, head_dim {hd}", "",
             "Command (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/{os.path.basename(os.path.normpath(kt_dir))} -o run -- python3 $R/bench.py {args_s} --steps 3 --warmup 1 --no-cpu-baseline",
             "", "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r.get("Name") or r.get("KernelName") or ""
        if "kvq" not in name:
            continue
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"kernel_source_sha256_16: {kernel_source_hash(ATTN_SOURCES)}"]
    with open(kt_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    knames = {}
    fetch = _counter_per_kernel(_read_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE", knames)
    write = _counter_per_kernel(_read_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch["copy"][0] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"][0] * 1024.0)
    mode = {"bf16": 0, "fp8_per_tensor": 1, "fp8_per_head": 2, "fp8_per_token_head": 3,
            "int4_per_token_head": 4}[mode_name]
    S, ctx, bs = 256, 8192, 16
    # the profiled launches: 4 fused steps (lengths ctx + 1 .. ctx + 4) and 4
    # attention-only passes at ctx + 4, 32 layers each: mean length ctx + 3.25
    algo = attention_bytes(mode, hd, hkv, bs, H, S, int(S * (ctx + 3.25)))
    flt = "--kernel-include-regex 'attention_kernel|attention_quad_kernel|attention_tquad_kernel|combine_kernel|copyBuffer'"
    out = [f"# HBM traffic per launch: decode attention, {mode_name}, head_dim {hd} (256 x ~8195 cached tokens, {hkv} KV heads)", "",
           "Two counter runs of the same bench command (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "",
           f"    rocprofv3 --pmc FETCH_SIZE {flt} --output-format csv -d $OUT/{os.path.basename(os.path.normpath(fetch_dir))} -o run -- python3 $R/bench.py {args_s} --steps 3 --warmup 1 --no-cpu-baseline --calibrate-copy",
           f"    rocprofv3 --pmc WRITE_SIZE {flt} --output-format csv -d $OUT/{os.path.basename(os.path.normpath(write_dir))} -o run -- python3 $R/bench.py {args_s} --steps 3 --warmup 1 --no-cpu-baseline --calibrate-copy",
           "",
           f"Calibration: a {COPY_BYTES >> 20} MiB device-to-device copy reads FETCH_SIZE {fetch['copy'][0]:.0f} KiB and "
           f"WRITE_SIZE {write['copy'][0]:.0f} KiB per dispatch; scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
           "Algorithmic bytes per launch: every cached token's K and V codes and per-token scales once, the block-table "
           "entries, the BF16 queries and outputs (the split partials the combine kernel reads are not counted).", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) | traffic | algorithmic | traffic / algorithmic |",
           "|---|---|---|---|---|---|---|---|---|"]
    tot = 0.0
    for k in ("attention", "combine"):
        if k not in fetch:
            continue
        fb = fetch[k][0] * 1024.0 * f_scale
        wb = write[k][0] * 1024.0 * w_scale
        tot += fb + wb
        a_s = f"{algo:.4g}" if k == "attention" else "-"
        r_s = f"{(fb + wb) / algo:.3f}" if k == "attention" else "-"
        out.append(f"| {knames.get(k, k + '_kernel')} | {fetch[k][1]} | {fetch[k][0]:.0f} | {write[k][0]:.0f} | {fb:.4g} | {wb:.4g} | "
                   f"{fb + wb:.4g} | {a_s} | {r_s} |")
    out += ["", f"kernel_source_sha256_16: {kernel_source_hash(ATTN_SOURCES)}",
            f"traffic_bytes_per_launch[attention]: {tot:.6g}"]
    with open(tr_path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + [""] + out))


def summarize_itl_trace(kt_dir):
    """profiles/kernel_trace_itl_gptoss_batch1.md from a rocprofv3 kernel
    trace of `bench.py --workload itl`: every attention and merge dispatch
    grouped by kernel and grid (the grid names the layer type and the
    context: one workgroup for a sliding layer, one per split range for a
    full layer), with the median and minimum duration."""
    import csv
    import glob
    import statistics
    files = sorted(glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *kernel_trace.csv under {kt_dir}")
    groups = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            key = _kernel_key(r["Kernel_Name"])
            if key is None or not (key[0].startswith("attention") or key[0].startswith("combine")):
                continue
            grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
            wg = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)
            groups.setdefault((key[1], grid // max(wg, 1)), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel trace: batch-1 decode attention, gpt-oss-20b shape (24 layers, 64 query / 8 KV heads, "
             "head_dim 64, one sequence of 8K / 16K / 32K tokens)", "",
             "Command (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "",
             f"    rocprofv3 --kernel-trace --output-format csv -d $OUT/{os.path.basename(os.path.normpath(kt_dir))} "
             "-o run -- python3 $R/bench.py --workload itl --steps 20 --warmup 5 --no-cpu-baseline", "",
             "Every dispatch of the three cache variants (eager and graph-replayed steps alike), grouped by kernel "
             "and workgroup count: one workgroup is a sliding layer (128 cached tokens, one split), more are the "
             "split ranges of a full layer, whose merge (combine) runs one workgroup per query head.", "",
             "| kernel | workgroups | dispatches | median (us) | min (us) |", "|---|---|---|---|---|"]
    for (name, wgs), ds in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        lines.append(f"| {name} | {wgs} | {len(ds)} | {statistics.median(ds):.2f} | {min(ds):.2f} |")
    lines += ["", f"kernel_source_sha256_16: {kernel_source_hash(ATTN_SOURCES)}"]
    with open(os.path.join(ROOT, "profiles", "kernel_trace_itl_gptoss_batch1.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kernels(kt_dir, fetch_dir, write_dir, tag, bytes_json, bench_args, pmc_filter=""):
    """profiles/kernel_trace_<tag>.md and profiles/traffic_<tag>.md from three
    rocprofv3 runs of `bench.py <bench_args>` (kernel trace with --stats;
    --pmc FETCH_SIZE; --pmc WRITE_SIZE, the counter runs with
    --calibrate-copy and, when pmc_filter is given, that
    --kernel-include-regex), with each kernel's algorithmic bytes per launch
    from the JSON the bench wrote with --launch-bytes-out.  Counter KiB are
    scaled by what the same counters read for a 256 MiB device-to-device
    copy."""
    import json as _json
    stats = _read_csv(kt_dir, "kernel_stats.csv")
    kt_cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/{os.path.basename(os.path.normpath(kt_dir))} "
              f"-o run -- python3 $R/bench.py {bench_args} --launch-bytes-out $OUT/{os.path.basename(bytes_json)}")
    lines = [f"# Kernel trace: {tag}", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "",
             f"    {kt_cmd}", "", "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        name = r.get("Name") or r.get("KernelName") or ""
        if _kernel_key(name) is None:
            continue
        lines.append(f"| {_kernel_key(name)[1]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"kernel_source_sha256_16: {kernel_source_hash()}"]
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(rows, counter):
        acc, names, copies = {}, {}, []
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            val = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(val)
                continue
            kk = _kernel_key(r["Kernel_Name"])
            if kk is None:
                continue
            acc.setdefault(kk[0], []).append(val)
            names[kk[0]] = kk[1]
        top = max(copies)
        copy = [v for v in copies if v >= 0.5 * top]
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}, names, sum(copy) / len(copy)

    fetch, names, fcopy = per_kernel(_read_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write, _, wcopy = per_kernel(_read_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / (fcopy * 1024.0), COPY_BYTES / (wcopy * 1024.0)
    algo = _json.load(open(bytes_json))
    flt = f"--kernel-include-regex '{pmc_filter}' " if pmc_filter else ""
    cmd = lambda c, d: (f"rocprofv3 --pmc {c} {flt}--output-format csv -d $OUT/{os.path.basename(os.path.normpath(d))} "
                        f"-o run -- python3 $R/bench.py {bench_args} --calibrate-copy")
    out = [f"# HBM traffic per launch: {tag}", "",
           "Two counter runs of the same bench command (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "",
           f"    {cmd('FETCH_SIZE', fetch_dir)}", f"    {cmd('WRITE_SIZE', write_dir)}", "",
           f"Calibration: a {COPY_BYTES >> 20} MiB device-to-device copy reads FETCH_SIZE {fcopy:.0f} KiB and "
           f"WRITE_SIZE {wcopy:.0f} KiB per dispatch; scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).",
           "", "Algorithmic bytes per launch are the bench's own (what each launch must move: no re-reads, no padding).",
           "", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) "
               "| traffic | algorithmic | traffic / algorithmic |", "|---|---|---|---|---|---|---|---|---|"]
    tail = ["", f"kernel_source_sha256_16: {kernel_source_hash()}"]
    for k in sorted(fetch):
        if k not in write:
            continue
        fb, wb = fetch[k][0] * 1024.0 * f_scale, write[k][0] * 1024.0 * w_scale
        a = algo.get(k)
        out.append(f"| {names[k]} | {fetch[k][1]} | {fetch[k][0]:.0f} | {write[k][0]:.0f} | {fb:.4g} | {wb:.4g} | "
                   f"{fb + wb:.4g} | {'-' if a is None else f'{a:.4g}'} | {'-' if not a else f'{(fb + wb) / a:.3f}'} |")
        tail.append(f"traffic_bytes_per_launch[{k}]: {fb + wb:.6g}")
    with open(os.path.join(ROOT, "profiles", f"traffic_{tag}.md"), "w") as f:
        f.write("\n".join(out + tail) + "\n")
    print("\n".join(lines + [""] + out + tail))


SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU "
               "SQ_BUSY_CYCLES SQ_WAIT_INST_ANY")


def summarize_instructions(tag, dirs):
    """profiles/instructions_<tag>.md: the SQ instruction counters of the
    decode-attention kernels from rocprofv3 runs of
    `bench.py --workload attention --mode M --head-dim D --steps 1 --warmup 0 --layers 4 [--tp T]`
    (one directory per run, named pmc_attn_<mode>_<hd>[_tp<T>]), per dispatch
    and per head-tile (16 cached tokens of one KV head for its whole query
    group)."""
    rows_out = []
    cmds = []
    for d in dirs:
        rows = _read_csv(d, "counter_collection.csv")
        acc, info = {}, {}
        for r in rows:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            info = r
        mean = {k: sum(v) / len(v) for k, v in acc.items()}
        dispatches = len(acc["SQ_WAVES"])
        m = re.search(r"pmc_attn_([a-z0-9_]+?)_(\d+)(?:_tp(\d+))?$", os.path.basename(os.path.normpath(d)))
        mode_name, hd, tp = m.group(1), int(m.group(2)), int(m.group(3) or 1)
        # the profiled step appends one token to 8192 cached ones: 513 tiles per (sequence, KV head)
        tiles = 256 * (8 // tp) * 513
        kname = info["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
        shape = f"{mode_name} / {hd}" + (f" (TP {tp}: {8 // tp} KV heads)" if tp > 1 else "")
        rows_out.append(f"| {shape} | {kname} | {dispatches} | {info['Workgroup_Size']} | "
                        f"{mean['SQ_WAVES']:.0f} | "
                        f"{mean['SQ_INSTS_VALU'] / tiles:.1f} | {mean['SQ_INSTS_SALU'] / tiles:.1f} | "
                        f"{mean['SQ_INSTS_LDS'] / tiles:.2f} | "
                        f"{100 * mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_WAVE_CYCLES']:.1f}% | "
                        f"{100 * mean['SQ_WAIT_INST_ANY'] / mean['SQ_WAVE_CYCLES']:.1f}% |")
        cmds.append(f"    rocprofv3 --pmc {SQ_COUNTERS} --kernel-include-regex 'attention_kernel|attention_quad_kernel|attention_tquad_kernel' "
                    f"--output-format csv -d $OUT/{os.path.basename(os.path.normpath(d))} -o run -- python3 "
                    f"$R/bench.py --workload attention --mode {mode_name} --head-dim {hd} --steps 1 --warmup 0 "
                    f"--layers 4 --no-cpu-baseline" + (f" --tp {tp}" if tp > 1 else ""))
    out = ["# Instruction counters: decode attention, 256 sequences x 8193 cached tokens, 8 KV heads, 32 query heads "
           "(a TP-T shard: 8/T and 32/T)", "",
           "Commands (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = an output directory):", "", *cmds, "",
           "Means over the dispatches of the attention kernel (4 layers x 3 passes).  A head-tile is 16 cached "
           "tokens of one KV head for its whole query group: 256 x 8 x 513 = 1.05 M per dispatch (divided by T "
           "on a TP-T shard).  "
           "VALU-active and waiting are SQ_ACTIVE_INST_VALU and SQ_WAIT_INST_ANY as shares of SQ_WAVE_CYCLES.", "",
           "| mode / head_dim | kernel | dispatches | workgroup | waves | VALU per head-tile "
           "| SALU per head-tile | LDS per head-tile | VALU-active | waiting |",
           "|---|---|---|---|---|---|---|---|---|---|", *rows_out, "",
           f"kernel_source_sha256_16: {kernel_source_hash(ATTN_SOURCES)}"]
    with open(os.path.join(ROOT, "profiles", f"instructions_{tag}.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def write_launch_bytes(path, entries):
    """The algorithmic bytes per launch of each kernel a run launched
    ({"store/128/3": bytes, ...}), for summarize_kernels."""
    if path:
        with open(path, "w") as f:
            json.dump({k: float(v) for k, v in entries.items()}, f, indent=1)


GQA32_LAYOUTS = ("fp8_per_token_head", "fp8_per_tensor", "fp8_per_head", "int4_per_token_head")


def gqa32_inputs(args, torch, W):
    """The GQA-32 step's inputs, shared by every layout: each layer's own
    BF16 K/V (seed 1000 + layer), one permuted block table and its slots, and
    each layer's own BF16 output pair."""
    spec = W.WORKLOADS["gqa32"]
    L, hkv, hd, bs = spec["num_layers"], spec["hkv"], spec["hd"], spec["block_size"]
    # a tensor-parallel shard stores only its own KV heads for the same tokens
    hkv //= getattr(args, "tp", 1)
    # --block-size: the same block-level permutation with larger blocks (the
    # sensitivity of the random block order to the block size)
    bs = getattr(args, "block_size", 0) or bs
    nseq, slen = spec["num_seqs"], spec["seq_len"]
    n = nseq * slen
    nblocks = n // bs
    dev = torch.device("cuda", 0)
    bt = W.permuted_block_table(nseq, slen // bs, nblocks, seed=1000)
    slots_h = W.slots_from_block_table(bt, [slen] * nseq, bs)
    slots = slots_h.to(dev)
    # the tokens in slot order: made on the host with the slot mapping, as a
    # serving step's scheduler makes both, and shared by every layer's store
    import numpy as np
    slot_order = torch.from_numpy(np.argsort(slots_h.numpy(), kind="stable").astype(np.int32)).to(dev)
    keys, values, outs = [], [], []
    for layer in range(L):
        k, v = W.gqa_kv(n, hkv, hd, seed=1000 + layer, device=dev)
        keys.append(k)
        values.append(v)
        outs.append((torch.empty_like(k), torch.empty_like(v)))
    torch.cuda.synchronize()
    return dict(L=L, hkv=hkv, hd=hd, bs=bs, n=n, nseq=nseq, slen=slen, nblocks=nblocks, bt=bt, bt_d=bt.to(dev),
                slots=slots, slot_order=slot_order, identity_slots=torch.arange(n, dtype=torch.int64, device=dev),
                seq_lens=torch.full((nseq,), slen, dtype=torch.int32, device=dev), keys=keys, values=values, outs=outs)


def gqa32_layout(torch, kvq, W, I, mode_name):
    """One layout's cache over the shared inputs: per-tensor scale 1.0 (the
    uncalibrated case), per-head scales calibrated by the library
    (kvq_calibrate_amax + kvq_static_scales) on a separate draw (seed 2000 +
    layer), and the pre-marshalled store and gather calls of every layer."""
    import ctypes
    mode = {v: k for k, v in W.MODE_NAMES.items()}[mode_name]
    L, hkv, hd, bs, nblocks = I["L"], I["hkv"], I["hd"], I["bs"], I["nblocks"]
    dev = I["keys"][0].device
    cache = kvq.Cache(kvq.CacheConfig(bs, hkv, hd, [mode] * L, [nblocks] * L), device=dev)
    scales = []
    for layer in range(L):
        if mode == kvq.FP8_PER_TENSOR:
            scales.append([1.0, 1.0])
        elif mode == kvq.FP8_PER_HEAD:
            kc, vc = W.gqa_kv(4096, hkv, hd, seed=2000 + layer, device=dev)
            amax = torch.zeros(2 * hkv, dtype=torch.float32, device=dev)
            kvq.kvq_calibrate_amax(kc, vc, amax)
            scales.append(kvq.kvq_static_scales(amax, hkv, mode))
        else:
            scales.append(None)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    sa, sa_tok, ga = [], [], []
    for layer in range(L):
        sc = scales[layer]
        csc = None if sc is None else (ctypes.c_float * len(sc))(*[float(x) for x in sc])
        sa_tok.append((cache.handle, layer, P(I["keys"][layer].data_ptr()), P(I["values"][layer].data_ptr()),
                       P(I["slots"].data_ptr()), I["n"], mode, csc, stream))
        sa.append((cache.handle, layer, P(I["keys"][layer].data_ptr()), P(I["values"][layer].data_ptr()),
                   P(I["slots"].data_ptr()), P(I["slot_order"].data_ptr()), I["n"], mode, csc, stream))
        ga.append((cache.handle, layer, P(I["bt_d"].data_ptr()), I["bt_d"].shape[1], P(I["seq_lens"].data_ptr()),
                   I["nseq"], P(I["outs"][layer][0].data_ptr()), P(I["outs"][layer][1].data_ptr()),
                   int(I["outs"][layer][0].shape[0]), stream))
    return dict(layout_geometry(kvq, W, I, mode_name), cache=cache, scales=scales, ordered_store_args=sa,
                token_store_args=sa_tok, gather_args=ga)


def layout_geometry(kvq, W, I, mode_name):
    """A layout's mode, layer bases in the cache buffer (256-byte aligned
    layers of equal size) and algorithmic bytes per launch."""
    mode = {v: k for k, v in W.MODE_NAMES.items()}[mode_name]
    L, hkv, hd, bs, nblocks = I["L"], I["hkv"], I["hd"], I["bs"], I["nblocks"]
    dynamic = mode in (kvq.FP8_PER_TOKEN_HEAD, kvq.INT4_PER_TOKEN_HEAD)
    block_bytes = bs * hkv * (2 * row_bytes(mode, hd) + (8 if dynamic else 0))
    layer_bytes = (nblocks * block_bytes + 255) // 256 * 256
    store_b, gather_b = algorithmic_bytes(mode, hd, hkv, bs, I["n"] * hkv)
    return dict(mode=mode, name=mode_name, dynamic=dynamic, layer_base=[l * layer_bytes for l in range(L)],
                layers_bytes=L * layer_bytes, store_bytes=store_b, gather_bytes=gather_b)


def store_follows_order(mode, hd):
    """Whether kvq_store_ordered follows the token order for a layer (asked of
    the library); other layers take the tokens in their own order."""
    import quantized_fp8_int4_amd as kvq
    return bool(kvq._lib.kvq_store_follows_order(int(mode), int(hd)))


def time_layout(torch, kvq, LA, steps, warmup, ordered=True):
    """W untimed warmup steps, then exactly K timed steps of every layer's
    store followed by every layer's gather; HIP events on the launch stream
    bracket each step's stores and gathers.  The stores take the tokens in
    slot order (kvq_store_ordered), or in token order (kvq_store).  Returns
    seconds per store launch, per gather launch and per step (wall clock,
    synchronized on both sides)."""
    lib = kvq._lib
    ga = LA["gather_args"]
    sa, store = ((LA["ordered_store_args"], lib.kvq_store_ordered) if ordered
                 else (LA["token_store_args"], lib.kvq_store))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        for a in sa:
            st = store(*a)
            if st != 0:
                raise kvq.KVQError(st, "kvq_store")
        if ev is not None:
            ev[1].record()
        for a in ga:
            st = lib.kvq_gather_dequant(*a)
            if st != 0:
                raise kvq.KVQError(st, "kvq_gather_dequant")
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    n = steps * len(sa)
    store_s = sum(e[0].elapsed_time(e[1]) for e in evs) / n / 1e3
    gather_s = sum(e[1].elapsed_time(e[2]) for e in evs) / n / 1e3
    return store_s, gather_s, wall


def oracle_scales(torch, W, I, LA, layer):
    """The oracle side's static scales of one layer, by the oracle's own
    calibration of the same draw: calibrate_amax, then RN32(amax / 448) in
    numpy float32 (per-tensor: of the maximum over heads); the library's
    scales must equal them bit for bit."""
    import numpy as np
    import oracle
    import quantized_fp8_int4_amd as kvq
    if LA["mode"] == kvq.FP8_PER_TENSOR:
        return np.array([1.0, 1.0], np.float32)
    if LA["mode"] != kvq.FP8_PER_HEAD:
        return None
    hkv, hd = I["hkv"], I["hd"]
    # the same draw as the library's calibration (drawn on the device, as all
    # inputs are; the CPU generator's stream differs), copied to the host
    kc, vc = W.gqa_kv(4096, hkv, hd, seed=2000 + layer, device=I["keys"][0].device)
    a = oracle.calibrate_amax(_bits(torch, kc), _bits(torch, vc), hkv, hd)
    s = (a / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(np.finfo(np.float32).smallest_subnormal)
    return s


def oracle_leg(torch, W, I, LA, layers, single_core=False):
    """The oracle, as it stands, on the given layers of the same step (store
    then gather of each), on this host's cores; checks those layers' cache
    bytes and gathered values against the GPU's.  Returns (seconds, threads,
    parity, seconds of one layer on one core or None)."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    L, hkv, hd, bs, nb = I["L"], I["hkv"], I["hd"], I["bs"], I["nblocks"]
    g = oracle.Geometry(bs, hkv, hd, [LA["mode"]] * L, [nb] * L)
    host = oracle.new_cache(g)
    slots = I["slots"].cpu().numpy()
    bt = I["bt"].numpy()
    lens = np.full(I["nseq"], I["slen"], np.int32)
    ins = {l: (_bits(torch, I["keys"][l]), _bits(torch, I["values"][l])) for l in layers}
    osc = {l: oracle_scales(torch, W, I, LA, l) for l in layers}
    ok = True
    for l in layers:
        if osc[l] is not None:
            ok = ok and bool(np.array_equal(np.asarray(LA["scales"][l], np.float32).view(np.uint32),
                                            osc[l].view(np.uint32)))
    t0 = time.perf_counter()
    gathered = {}
    for l in layers:
        oracle.store(g, host, l, ins[l][0], ins[l][1], slots, osc[l])
    for l in layers:
        gathered[l] = oracle.gather(g, host, l, bt, lens)
    secs = time.perf_counter() - t0
    threads = oracle.num_threads()
    secs_one = None
    if single_core:
        l = layers[0]
        oracle.set_num_threads(1)
        t1 = time.perf_counter()
        oracle.store(g, host, l, ins[l][0], ins[l][1], slots, osc[l])
        oracle.gather(g, host, l, bt, lens)
        secs_one = time.perf_counter() - t1
        oracle.set_num_threads(threads)
    lb, _, _ = oracle.layer_offsets(g)
    lbytes = int(lb[1] - lb[0]) if L > 1 else host.size
    dev = LA["cache"].buffer
    for l in layers:
        lo = int(lb[l])
        ok = ok and bool(np.array_equal(dev[lo: lo + lbytes].cpu().numpy(), host[lo: lo + lbytes]))
        ok = ok and bool(np.array_equal(_bits(torch, I["outs"][l][0]), gathered[l][0]))
        ok = ok and bool(np.array_equal(_bits(torch, I["outs"][l][1]), gathered[l][1]))
    return secs, threads, ok, secs_one


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Launcher:
    """Pre-marshalled C-ABI calls on the current stream (the host stays far
    ahead of the GPU, so kernels run back to back)."""

    def __init__(self, torch, kvq, cache):
        import ctypes
        self.ct, self.kvq, self.lib, self.h = ctypes, kvq, kvq._lib, cache.handle
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def store_args(self, layer, k, v, slots, mode, scales=None):
        ct = self.ct
        sc = None if scales is None else (ct.c_float * len(scales))(*[float(x) for x in scales])
        return (self.h, layer, ct.c_void_p(k.data_ptr()), ct.c_void_p(v.data_ptr()), ct.c_void_p(slots.data_ptr()),
                int(slots.numel()), mode, sc, self.stream)

    def gather_args(self, layer, bt, sl, ok, ov):
        ct = self.ct
        return (self.h, layer, ct.c_void_p(bt.data_ptr()), int(bt.shape[1]), ct.c_void_p(sl.data_ptr()),
                int(sl.numel()), ct.c_void_p(ok.data_ptr()), ct.c_void_p(ov.data_ptr()), int(ok.shape[0]), self.stream)

    def store(self, a):
        st = self.lib.kvq_store(*a)
        if st != 0:
            raise self.kvq.KVQError(st, "kvq_store")

    def gather(self, a):
        st = self.lib.kvq_gather_dequant(*a)
        if st != 0:
            raise self.kvq.KVQError(st, "kvq_gather_dequant")


def _timed(torch, step, steps, warmup):
    """Run warmup steps, then time `steps` steps; step(ev) records ev[i] between
    its phases.  Returns (wall seconds per step, list of per-step events)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, evs


def _result(args, metric_cfg, value, ms_per_step, store_b, gather_b, store_s, gather_s, cpu, parity, extra):
    store_gbps = store_b / store_s / 1e9 if store_s > 0 else 0.0
    gather_gbps = gather_b / gather_s / 1e9 if gather_s > 0 else 0.0
    dominant = "store" if store_s >= gather_s else "gather"
    dom = store_gbps if dominant == "store" else gather_gbps
    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": metric_cfg,
           "store_GBps": round(store_gbps, 1), "gather_GBps": round(gather_gbps, 1),
           "store_frac_of_peak": round(store_gbps / HBM_PEAK_GBPS, 4),
           "gather_frac_of_peak": round(gather_gbps / HBM_PEAK_GBPS, 4),
           "store_us": round(store_s * 1e6, 2), "gather_us": round(gather_s * 1e6, 2),
           "roofline": {"bound": "hbm", "kernel": f"{dominant}_kernel", "achieved": round(dom, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom / HBM_PEAK_GBPS, 4), "traffic": None},
           "cpu_baseline": cpu, "parity_vs_oracle_sampled": parity}
    out.update(extra)
    return out


def _bits(torch, t):
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def attention_bytes(mode, hd, hkv, bs, H, num_seqs, total_tokens):
    """Algorithmic bytes of one decode-attention launch: every cached token's
    K and V codes (and per-token scales) once, the block-table entries, the
    BF16 queries and outputs."""
    rb = row_bytes(mode, hd)
    sigma = 8 if mode in (3, 4) else 0
    return (total_tokens * hkv * (2 * rb + sigma) + -(-total_tokens // bs) * 4
            + num_seqs * H * hd * 2 * 2)


def _decode_setup(args, torch, kvq, W, dev):
    """The decode workload: a 32-layer cache of 256 sequences prefilled with
    8192 seeded N(0,1) tokens each, plus the slots, lengths and new K/V of
    every decode step the run will take."""
    spec = W.WORKLOADS["decode"]
    L, hkv, bs, S, ctx = spec["num_layers"], spec["hkv"], spec["block_size"], spec["num_seqs"], spec["context"]
    # a tensor-parallel shard holds only its own KV heads (and their query heads)
    hkv //= args.tp
    hd = args.head_dim
    mode = {v: k for k, v in W.MODE_NAMES.items()}[args.mode]
    if args.workload == "decode" and mode not in (kvq.FP8_PER_TOKEN_HEAD, kvq.INT4_PER_TOKEN_HEAD):
        raise SystemExit("decode workload: --mode fp8_per_token_head or int4_per_token_head")
    if args.layers:
        L = int(args.layers)
    # static layers: uncalibrated scale 1.0 (the pages' per-tensor default)
    scales = {kvq.FP8_PER_TENSOR: [1.0, 1.0], kvq.FP8_PER_HEAD: [1.0] * (2 * hkv)}.get(mode)
    # the workload's 513 blocks per sequence hold 8192 + 16 tokens; room is
    # added for every appended step this run takes
    maxb = ctx // bs + 1 + (args.warmup + args.steps) // bs
    nb = S * maxb
    cfg = kvq.CacheConfig(bs, hkv, hd, [mode] * L, [nb] * L)
    cache = kvq.Cache(cfg, device=dev)
    log(f"[bench] decode: cache {cache.bytes['total'] / 2**30:.2f} GiB; prefilling {L} layers x {S} x {ctx} tokens")
    st = W.DecodeState(S, bs, nb, maxb, seed=5000)
    slots = []
    for b in range(S):
        slots += st.append(b, ctx)
    slots = torch.tensor(slots, dtype=torch.int64, device=dev)
    Lc = Launcher(torch, kvq, cache)
    chunk = 32768
    for l in range(L):
        for c0 in range(0, S * ctx, chunk):
            k, v = W.normal_kv(chunk, hkv, hd, seed=5000 + 1000 * l + c0 // chunk, device=dev)
            Lc.store(Lc.store_args(l, k, v, slots[c0: c0 + chunk], mode, scales if c0 == 0 else None))
        torch.cuda.synchronize()
    steps_slots = []
    for _ in range(args.warmup + args.steps):
        steps_slots.append(torch.tensor([st.append(b, 1)[0] for b in range(S)], dtype=torch.int64, device=dev))
    kdec, vdec = W.normal_kv(S, hkv, hd, seed=6000, device=dev)
    lens_at = [torch.tensor([ctx + s_ + 1] * S, dtype=torch.int32, device=dev)
               for s_ in range(args.warmup + args.steps)]
    return {"L": L, "S": S, "hkv": hkv, "hd": hd, "bs": bs, "ctx": ctx, "mode": mode, "nb": nb, "cache": cache,
            "scales": scales,
            "st": st, "slots": slots, "chunk": chunk, "Lc": Lc, "steps_slots": steps_slots, "kdec": kdec,
            "vdec": vdec, "lens_at": lens_at, "bt": st.block_table.to(dev),
            "desc": spec["desc"] + f", head_dim {hd}, {args.mode}"
                    + (f"; tensor-parallel shard (TP {args.tp}): {hkv} of 8 KV heads per GPU" if args.tp > 1 else "")}


def _decode_oracle_layer(D, torch, W, oracle):
    """The oracle's own image of the last layer after every step: its store
    of the same seeded prefill chunks and appended tokens."""
    import numpy as np
    l = D["L"] - 1
    g = oracle.Geometry(D["bs"], D["hkv"], D["hd"], [D["mode"]], [D["nb"]])
    host = oracle.new_cache(g)
    slots = D["slots"].cpu().numpy()
    dev = D["slots"].device
    sc = None if D["scales"] is None else np.array(D["scales"], np.float32)
    for c0 in range(0, D["S"] * D["ctx"], D["chunk"]):
        k, v = W.normal_kv(D["chunk"], D["hkv"], D["hd"], seed=5000 + 1000 * l + c0 // D["chunk"], device=dev)
        oracle.store(g, host, 0, _bits(torch, k), _bits(torch, v), slots[c0: c0 + D["chunk"]], sc)
    kb, vb = _bits(torch, D["kdec"]), _bits(torch, D["vdec"])
    for ss in D["steps_slots"]:
        oracle.store(g, host, 0, kb, vb, ss.cpu().numpy(), sc)
    return g, host


def run_other_workload(args, torch, kvq, W):
    """long80, gptoss and decode: the remaining shapes, each with its own
    timing, oracle sample and parity cross-check.  Printed as one JSON line."""
    import numpy as np
    import oracle

    dev = torch.device("cuda", 0)
    oracle.build(force=False)
    name = args.workload
    launch_bytes = {}
    if name == "long80":
        spec = W.WORKLOADS["long80"]
        L, hkv, hd, bs, T = spec["num_layers"], spec["hkv"], spec["hd"], spec["block_size"], spec["seq_len"]
        mode = kvq.FP8_PER_TOKEN_HEAD
        nb = T // bs
        cfg = kvq.CacheConfig(bs, hkv, hd, [mode] * L, [nb] * L)
        cache = kvq.Cache(cfg, device=dev)
        log(f"[bench] long80: cache {cache.bytes['total'] / 2**30:.3f} GiB; generating {L} layers of inputs")
        slots = torch.arange(T, dtype=torch.int64, device=dev)
        bt = torch.arange(nb, dtype=torch.int32, device=dev).view(1, nb)
        sl = torch.tensor([T], dtype=torch.int32, device=dev)
        ins = [W.heavy_tail_kv(T, hkv, hd, seed=3000 + l, device=dev) for l in range(L)]
        outs = [(torch.empty_like(k), torch.empty_like(v)) for k, v in ins]
        Lc = Launcher(torch, kvq, cache)
        sa = [Lc.store_args(l, ins[l][0], ins[l][1], slots, mode) for l in range(L)]
        ga = [Lc.gather_args(l, bt, sl, outs[l][0], outs[l][1]) for l in range(L)]

        def step(ev):
            if ev: ev[0].record()
            for a in sa: Lc.store(a)
            if ev: ev[1].record()
            for a in ga: Lc.gather(a)
            if ev: ev[2].record()
        sec, evs = _timed(torch, step, args.steps, args.warmup)
        store_s = sum(e[0].elapsed_time(e[1]) for e in evs) / (args.steps * L) / 1e3
        gather_s = sum(e[1].elapsed_time(e[2]) for e in evs) / (args.steps * L) / 1e3
        sb, gb = algorithmic_bytes(mode, hd, hkv, bs, T * hkv)
        launch_bytes.update({f"store/{hd}/{mode}": sb, f"gather/{hd}/{mode}": gb})
        # oracle: one layer, store + gather
        g = oracle.Geometry(bs, hkv, hd, [mode], [nb])
        host = oracle.new_cache(g)
        kb, vb = _bits(torch, ins[0][0]), _bits(torch, ins[0][1])
        t0 = time.perf_counter()
        oracle.store(g, host, 0, kb, vb, np.arange(T))
        ko, vo = oracle.gather(g, host, 0, np.arange(nb, dtype=np.int32)[None, :], np.array([T], np.int32))
        csec = time.perf_counter() - t0
        lb = int(oracle.layer_offsets(g)[2])          # bytes of one layer (layer 0 starts at 0)
        parity = bool(np.array_equal(cache.buffer[:lb].cpu().numpy(), host[:lb])
                      and np.array_equal(_bits(torch, outs[0][0]), ko)
                      and np.array_equal(_bits(torch, outs[0][1]), vo))
        cpu = {"value": round((sb + gb) / csec / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"1 of {L} layers (store + gather of {T} tokens), {csec:.2f} s wall"}
        res = _result(args, {"workload": spec["desc"] + "; per-token-head FP8 store of every layer, then full gather",
                             "layers": L, "tokens": T, "num_kv_heads": hkv, "head_dim": hd, "block_size": bs,
                             "mode": "fp8_per_token_head"},
                      L * (sb + gb) / sec / 1e9, sec * 1e3, sb, gb, store_s, gather_s, cpu, parity,
                      {"cached_tokens_per_s": round(T / (L * store_s), 1),
                       "cache_GiB": round(cache.bytes["total"] / 2**30, 4)})
    elif name == "gptoss":
        spec = W.WORKLOADS["gptoss"]
        L, hkv, hd, bs, T, Wn = spec["num_layers"], spec["hkv"], spec["hd"], spec["block_size"], spec["seq_len"], spec["window"]
        modes = [kvq.BF16 if W.gptoss_layer_is_sliding(l) else kvq.FP8_PER_TOKEN_HEAD for l in range(L)]
        nbs = [Wn // bs if m == kvq.BF16 else T // bs for m in modes]
        cfg = kvq.CacheConfig(bs, hkv, hd, modes, nbs)
        cache = kvq.Cache(cfg, device=dev)
        log(f"[bench] gptoss: cache {cache.bytes['total'] / 2**20:.1f} MiB")
        full_slots = torch.arange(T, dtype=torch.int64, device=dev)
        ring = (torch.arange(T - Wn, T, dtype=torch.int64, device=dev) % Wn)
        bt_full = torch.arange(T // bs, dtype=torch.int32, device=dev).view(1, -1)
        bt_ring = torch.arange(Wn // bs, dtype=torch.int32, device=dev).view(1, -1)
        sl_full = torch.tensor([T], dtype=torch.int32, device=dev)
        sl_ring = torch.tensor([Wn], dtype=torch.int32, device=dev)
        Lc = Launcher(torch, kvq, cache)
        ins, outs, sa, ga = [], [], [], []
        for l in range(L):
            k, v = W.normal_kv(T, hkv, hd, seed=4000 + l, device=dev)
            if modes[l] == kvq.BF16:
                # a sliding layer keeps only the last W tokens: only they are handed over
                k, v = k[T - Wn:].contiguous(), v[T - Wn:].contiguous()
                sa.append(Lc.store_args(l, k, v, ring, modes[l]))
                o = (torch.empty((Wn, hkv, hd), dtype=torch.bfloat16, device=dev),
                     torch.empty((Wn, hkv, hd), dtype=torch.bfloat16, device=dev))
                ga.append(Lc.gather_args(l, bt_ring, sl_ring, o[0], o[1]))
            else:
                sa.append(Lc.store_args(l, k, v, full_slots, modes[l]))
                o = (torch.empty_like(k), torch.empty_like(v))
                ga.append(Lc.gather_args(l, bt_full, sl_full, o[0], o[1]))
            ins.append((k, v))
            outs.append(o)
        full = [l for l in range(L) if modes[l] != kvq.BF16]
        slide = [l for l in range(L) if modes[l] == kvq.BF16]

        def step(ev):
            if ev: ev[0].record()
            for l in full: Lc.store(sa[l])
            for l in slide: Lc.store(sa[l])
            if ev: ev[1].record()
            for l in full: Lc.gather(ga[l])
            for l in slide: Lc.gather(ga[l])
            if ev: ev[2].record()
        sec, evs = _timed(torch, step, args.steps, args.warmup)
        # per-kernel times of the full layers alone
        def phase(seq_calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                for f, a in seq_calls: f(a)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / (args.steps * len(seq_calls))
        store_s = phase([(Lc.store, sa[l]) for l in full])
        gather_s = phase([(Lc.gather, ga[l]) for l in full])
        slide_store_s = phase([(Lc.store, sa[l]) for l in slide])
        slide_gather_s = phase([(Lc.gather, ga[l]) for l in slide])
        sb, gb = algorithmic_bytes(kvq.FP8_PER_TOKEN_HEAD, hd, hkv, bs, T * hkv)
        ssb, sgb = algorithmic_bytes(kvq.BF16, hd, hkv, bs, Wn * hkv)
        launch_bytes.update({f"store/{hd}/{kvq.FP8_PER_TOKEN_HEAD}": sb, f"gather/{hd}/{kvq.FP8_PER_TOKEN_HEAD}": gb,
                             f"store/{hd}/{kvq.BF16}": ssb, f"gather/{hd}/{kvq.BF16}": sgb})
        step_bytes = len(full) * (sb + gb) + len(slide) * (ssb + sgb)
        g = oracle.Geometry(bs, hkv, hd, modes, nbs)
        host = oracle.new_cache(g)
        t0 = time.perf_counter()
        got = {}
        for l in (slide[0], full[0]):
            k, v = ins[l]
            sm = (ring if modes[l] == kvq.BF16 else full_slots).cpu().numpy()
            oracle.store(g, host, l, _bits(torch, k), _bits(torch, v), sm)
            btn = (bt_ring if modes[l] == kvq.BF16 else bt_full).cpu().numpy()
            sln = (sl_ring if modes[l] == kvq.BF16 else sl_full).cpu().numpy()
            got[l] = oracle.gather(g, host, l, btn, sln)
        csec = time.perf_counter() - t0
        lb, _, _ = oracle.layer_offsets(g)
        dev_buf = cache.buffer.cpu().numpy()
        parity = True
        for l in (slide[0], full[0]):
            end = int(lb[l + 1]) if l + 1 < L else int(oracle.layer_offsets(g)[1][0])
            parity &= bool(np.array_equal(dev_buf[int(lb[l]): end], host[int(lb[l]): end]))
            parity &= bool(np.array_equal(_bits(torch, outs[l][0]), got[l][0]) and
                           np.array_equal(_bits(torch, outs[l][1]), got[l][1]))
        cpu = {"value": round((sb + gb + ssb + sgb) / csec / 1e9, 3), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"one full and one sliding layer of the {L} (store + gather), {csec:.2f} s wall"}
        extra = {"sliding_store_us": round(slide_store_s * 1e6, 2), "sliding_gather_us": round(slide_gather_s * 1e6, 2),
                 "cache_MiB": round(cache.bytes["total"] / 2**20, 3)}
        if not args.no_ceiling:
            # the full layers' own access patterns without arithmetic, at the
            # same launch size (32768 tokens x 8 KV heads x head_dim 64)
            nbf = T // bs
            lbytes = (nbf * bs * hkv * (2 * hd + 8) + 255) // 256 * 256
            Ifull = dict(L=len(full), hkv=hkv, hd=hd, bs=bs, n=T, nblocks=nbf, nseq=1, seq_lens=sl_full,
                         keys=[ins[l][0] for l in full], values=[ins[l][1] for l in full],
                         outs=[outs[l] for l in full])
            geo = dict(mode=kvq.FP8_PER_TOKEN_HEAD, dynamic=True, layer_base=[i * lbytes for i in range(len(full))],
                       store_bytes=sb, gather_bytes=gb)
            sbuf = torch.zeros(len(full) * lbytes, dtype=torch.uint8, device=dev)
            reps = max(3, args.steps)
            spc = store_pattern_ceiling(torch, Ifull, geo, full_slots, reps, sbuf)
            gpc = gather_pattern_ceiling(torch, Ifull, geo, bt_full, reps, sbuf)
            del sbuf
            extra["ceilings"] = {"store_pattern": spc, "gather_pattern": gpc,
                                 "store_vs_pattern_ceiling": round(sb / store_s / 1e9 / spc["GBps"], 4),
                                 "gather_vs_pattern_ceiling": round(gb / gather_s / 1e9 / gpc["GBps"], 4)}
            log(f"[bench] gptoss full-layer ceilings: store pattern {spc['GBps']:.0f} GB/s, "
                f"gather pattern {gpc['GBps']:.0f} GB/s")
        res = _result(args, {"workload": spec["desc"], "layers": L, "tokens": T, "window": Wn,
                             "num_kv_heads": hkv, "head_dim": hd, "block_size": bs,
                             "mode": "full: fp8_per_token_head, sliding: bf16 ring"},
                      step_bytes / sec / 1e9, sec * 1e3, sb, gb, store_s, gather_s, cpu, bool(parity), extra)
    elif name == "itl":
        # Attention-only inter-token latency against context, gpt-oss-20b shape
        # (24 layers alternating sliding W=128 and full, 64 query / 8 KV heads,
        # head_dim 64), batch 1: the three cache variants the pages' latency
        # study compares (all BF16, all FP8 with per-tensor scale 1.0, FP8 with
        # the sliding layers kept BF16); the slope is ms per context token.
        L, hkv, hd, bs, Wn, H = 24, 8, 64, 16, 128, 64
        ctxs = [8192, 16384, 32768]
        variants = {"bf16": (kvq.BF16, kvq.BF16), "fp8": (kvq.FP8_PER_TENSOR, kvq.FP8_PER_TENSOR),
                    "fp8_skip_sliding": (kvq.FP8_PER_TENSOR, kvq.BF16)}
        ct = __import__("ctypes")
        sm = 1.0 / math.sqrt(hd)
        slopes, times, intercepts = {}, {}, {}
        times_eager, slopes_eager = {}, {}
        graph_ok = True                   # every graph replay equal to the eager step, bit for bit
        itl_parity = None
        ocpu_s, ocpu_b = 0.0, 0           # oracle attention: seconds and algorithmic bytes
        for vname, (full_mode, slide_mode) in variants.items():
            ts, ts_eager = [], []
            for T in ctxs:
                sliding = [W.gptoss_layer_is_sliding(l) for l in range(L)]
                modes = [slide_mode if sl_ else full_mode for sl_ in sliding]
                nbs = [Wn // bs if sl_ else T // bs for sl_ in sliding]
                cache = kvq.Cache(kvq.CacheConfig(bs, hkv, hd, modes, nbs), device=dev)
                full_slots = torch.arange(T, dtype=torch.int64, device=dev)
                ring = W.ring_slots(T, Wn, device=dev)
                for l in range(L):
                    k, v = W.normal_kv(T, hkv, hd, seed=9000 + l, device=dev)
                    sc = [1.0, 1.0] if modes[l] == kvq.FP8_PER_TENSOR else None
                    cache.store(l, k, v, ring if sliding[l] else full_slots, sc)
                bt_full = torch.arange(T // bs, dtype=torch.int32, device=dev).view(1, -1)
                bt_ring = W.ring_block_table(Wn, bs, device=dev)
                sl_full = torch.tensor([T], dtype=torch.int32, device=dev)
                sl_ring = torch.tensor([Wn], dtype=torch.int32, device=dev)
                q = W.normal_kv(1, H, hd, seed=9999, device=dev)[0]
                outs = torch.zeros((L,) + tuple(q.shape), dtype=q.dtype, device=dev)   # one output per layer
                ws_n = max(kvq.kvq_decode_attention_workspace(cache.handle, H, T // bs, 1), 16)
                ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)

                def calls(stream_handle):
                    stream = ct.c_void_p(stream_handle)
                    aa = []
                    for l in range(L):
                        bt, sl_ = (bt_ring, sl_ring) if sliding[l] else (bt_full, sl_full)
                        aa.append((cache.handle, l, ct.c_void_p(q.data_ptr()), H, ct.c_void_p(bt.data_ptr()),
                                   int(bt.shape[1]), ct.c_void_p(sl_.data_ptr()), 1, ct.c_float(sm),
                                   ct.c_void_p(outs[l].data_ptr()), ct.c_void_p(ws.data_ptr()), ws_n, stream))
                    return aa

                def launch_all(aa):
                    for a in aa:
                        st_ = kvq._lib.kvq_decode_attention(*a)
                        if st_ != 0:
                            raise kvq.KVQError(st_, "kvq_decode_attention")

                aa = calls(torch.cuda.current_stream().cuda_stream)

                def step(ev):
                    if ev: ev[0].record()
                    launch_all(aa)
                    if ev: ev[1].record(); ev[2].record()
                _, evs = _timed(torch, step, args.steps, args.warmup)
                ts_eager.append(sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps)   # ms per decode step
                eager_outs = outs.clone()
                # the same 24 launches captured once in a HIP graph and replayed,
                # as a serving engine replays its decode step
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    launch_all(calls(side.cuda_stream))
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    launch_all(calls(torch.cuda.current_stream().cuda_stream))
                torch.cuda.synchronize()
                for _ in range(3):
                    # each checked replay follows eager work and a synchronization
                    outs.zero_()
                    torch.cuda.synchronize()
                    graph.replay()
                    torch.cuda.synchronize()
                    graph_ok = graph_ok and bool(torch.equal(outs, eager_outs))

                def gstep(ev):
                    if ev: ev[0].record()
                    graph.replay()
                    if ev: ev[1].record(); ev[2].record()
                _, gevs = _timed(torch, gstep, args.steps, args.warmup)
                ts.append(sum(e[0].elapsed_time(e[1]) for e in gevs) / args.steps)
                graph_ok = graph_ok and bool(torch.equal(outs, eager_outs))
                del graph
                if T == ctxs[0] and not args.no_cpu_baseline:
                    # oracle check of the first sliding and the first full layer
                    ok_layers = []
                    for l in (0, 1):
                        bt, sl_ = (bt_ring, sl_ring) if sliding[l] else (bt_full, sl_full)
                        o_l = eager_outs[l]
                        g1 = oracle.Geometry(bs, hkv, hd, [modes[l]], [nbs[l]])
                        img = oracle.new_cache(g1)
                        k, v = W.normal_kv(T, hkv, hd, seed=9000 + l, device=dev)
                        sc = np.array([1.0, 1.0], np.float32) if modes[l] == kvq.FP8_PER_TENSOR else None
                        oracle.store(g1, img, 0, _bits(torch, k), _bits(torch, v),
                                     (ring if sliding[l] else full_slots).cpu().numpy(), sc)
                        qb = _bits(torch, q.view(1, H, hd))
                        btn, sln = bt.cpu().numpy(), sl_.cpu().numpy()
                        c0 = time.perf_counter()
                        ref, absv = oracle.decode_attention(g1, img, 0, qb, btn, sln, sm, with_absv=True)
                        ocpu_s += time.perf_counter() - c0
                        ocpu_b += attention_bytes(modes[l], hd, hkv, bs, H, 1, int(sln[0]))
                        tol = oracle.attention_error_bound(g1, img, 0, qb, btn, sln, sm, ref, absv, 1.0)
                        got = o_l.float().cpu().numpy().reshape(ref.shape).astype(np.float64)
                        ok_layers.append(bool((np.abs(got - ref) <= tol).all()))
                    itl_parity = all(ok_layers) if itl_parity is None else (itl_parity and all(ok_layers))
                del cache
                torch.cuda.empty_cache()
            n = len(ctxs)
            mx = sum(ctxs) / n

            def fit(ys):
                my = sum(ys) / n
                sl = sum((x - mx) * (y - my) for x, y in zip(ctxs, ys)) / sum((x - mx) ** 2 for x in ctxs)
                return sl, my - sl * mx
            slopes[vname], intercepts[vname] = fit(ts)
            slopes_eager[vname] = fit(ts_eager)[0]
            times[vname] = [round(t, 5) for t in ts]
            times_eager[vname] = [round(t, 5) for t in ts_eager]
            log(f"[bench] itl {vname}: graph {times[vname]} ms, eager {times_eager[vname]} ms at {ctxs} tokens, "
                f"slope {slopes[vname]:.3e} ms/token (eager {slopes_eager[vname]:.3e})")
        # one decode step of the FP8 variant with BF16 sliding layers at the
        # longest context: 12 full layers of T tokens, 12 rings of W tokens
        T = ctxs[-1]
        step_b = 12 * attention_bytes(kvq.FP8_PER_TENSOR, hd, hkv, bs, H, 1, T) + \
            12 * attention_bytes(kvq.BF16, hd, hkv, bs, H, 1, Wn)
        ach = step_b / (times["fp8_skip_sliding"][-1] / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": f"attention_kernel + combine_wide_kernel, a step of {L} layers at {T} tokens "
                                          "(fp8_skip_sliding)",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None}
        cpu = None
        if ocpu_s > 0:
            cpu = {"value": round(ocpu_b / ocpu_s / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                   "kind": "oracle",
                   "sample": f"fp64 attention of the first sliding and the first full layer at {ctxs[0]} tokens, "
                             f"each variant, {ocpu_s:.2f} s wall"}
        res = {"metric": "attention-only inter-token latency slope (ms per context token), gpt-oss-20b shape, batch 1",
               "value": round(slopes["fp8_skip_sliding"], 12), "unit": "ms/token", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": times["fp8_skip_sliding"][-1], "higher_is_better": False,
               "scaling": "weak", "vs_baseline": None, "dtype": "fp8/bf16 codes, bf16 MFMA, f32 accumulate",
               "data": "synthetic",
               "config": {"workload": "gpt-oss-20b shape: 24 layers alternating sliding (W=128) and full, 64 query / "
                                      "8 KV heads, head_dim 64, one sequence; decode attention of all 24 layers",
                          "contexts": ctxs, "variants": list(variants)},
               "slopes_ms_per_token": {k: float(f"{v:.4g}") for k, v in slopes.items()},
               "step_ms": times,
               "timing": "HIP graph replay of the step's 24 launches (eager launches in step_ms_eager)",
               "graph_replays_equal_eager": graph_ok,
               "slopes_ms_per_token_eager": {k: float(f"{v:.4g}") for k, v in slopes_eager.items()},
               "step_ms_eager": times_eager,
               "pages_h100_full_model_slopes_ms_per_token": {"bf16": 8.94e-06, "fp8": 7.14e-06,
                                                              "fp8_skip_sliding": 6.34e-06},
               # the context where a variant's fitted line crosses BF16's (None
               # where it is not slower at short context, or not faster per token)
               "break_even_vs_bf16_tokens": {
                   k: (round((intercepts[k] - intercepts["bf16"]) / (slopes["bf16"] - slopes[k]))
                       if slopes["bf16"] > slopes[k] and intercepts[k] > intercepts["bf16"] else None)
                   for k in ("fp8", "fp8_skip_sliding")},
               "pages_h100_break_even_vs_bf16_tokens": {"fp8": 22109, "fp8_skip_sliding": 7659},
               "roofline": roof, "cpu_baseline": cpu, "parity_vs_oracle_sampled": itl_parity}
    elif name == "calib":
        # on-the-fly calibration over the GQA-32 prefill: one amax pass per layer
        spec = W.WORKLOADS["gqa32"]
        L, hkv, hd, n = spec["num_layers"], spec["hkv"], spec["hd"], spec["num_seqs"] * spec["seq_len"]
        ins = [W.gqa_kv(n, hkv, hd, seed=1000 + l, device=dev) for l in range(L)]
        amax = torch.zeros((L, 2 * hkv), dtype=torch.float32, device=dev)
        ct = __import__("ctypes")
        stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        args_c = [(ct.c_void_p(ins[l][0].data_ptr()), ct.c_void_p(ins[l][1].data_ptr()), n, hkv, hd,
                   ct.c_void_p(amax[l].data_ptr()), 0, stream) for l in range(L)]

        def step(ev):
            if ev: ev[0].record()
            for a in args_c:
                st_ = kvq._lib.kvq_calibrate_amax(*a)
                if st_ != 0:
                    raise kvq.KVQError(st_, "kvq_calibrate_amax")
            if ev: ev[1].record(); ev[2].record()
        sec, evs = _timed(torch, step, args.steps, args.warmup)
        cal_s = sum(e[0].elapsed_time(e[1]) for e in evs) / (args.steps * L) / 1e3
        # the later batches of a warmup loop accumulate into the running
        # maxima: the call is then calib_kernel alone, without the fill
        # kernel that clears amax for a first batch
        args_acc = [a[:6] + (1,) + a[7:] for a in args_c]

        def step_acc(ev):
            if ev: ev[0].record()
            for a in args_acc:
                st_ = kvq._lib.kvq_calibrate_amax(*a)
                if st_ != 0:
                    raise kvq.KVQError(st_, "kvq_calibrate_amax")
            if ev: ev[1].record(); ev[2].record()
        _, evs_acc = _timed(torch, step_acc, args.steps, args.warmup)
        acc_s = sum(e[0].elapsed_time(e[1]) for e in evs_acc) / (args.steps * L) / 1e3
        cal_b = n * hkv * 4 * hd
        t0 = time.perf_counter()
        ref = oracle.calibrate_amax(_bits(torch, ins[0][0]), _bits(torch, ins[0][1]), hkv, hd)
        csec = time.perf_counter() - t0
        parity = bool(np.array_equal(amax[0].cpu().numpy().view(np.uint32), ref.view(np.uint32)))
        gbps = cal_b / cal_s / 1e9
        res = {"metric": "kvq_calibrate_amax GB/s (on-the-fly static-scale calibration)", "value": round(gbps, 1),
               "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "bf16->f32 max", "data": "synthetic",
               "config": {"workload": "calibration amax of each GQA-32 layer's prefill K/V (32768 tokens x 8 KV heads x 128)",
                          "layers": L},
               "calib_us": round(cal_s * 1e6, 2),
               "calib_accumulate_us": round(acc_s * 1e6, 2),
               "calib_accumulate_GBps": round(cal_b / acc_s / 1e9, 1),
               "roofline": {"bound": "hbm", "kernel": "calib_kernel (accumulating calls: the kernel alone)",
                            "achieved": round(cal_b / acc_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(cal_b / acc_s / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None},
               "cpu_baseline": {"value": round(cal_b / csec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": f"one layer's amax (single-threaded loop), {csec:.2f} s wall"},
               "parity_vs_oracle_sampled": parity}
    elif name == "decode":
        D = _decode_setup(args, torch, kvq, W, dev)
        L, S, hkv, hd, bs, mode, Lc = D["L"], D["S"], D["hkv"], D["hd"], D["bs"], D["mode"], D["Lc"]
        tot_max = sum(D["st"].seq_lens)
        ok = torch.empty((tot_max, hkv, hd), dtype=torch.bfloat16, device=dev)
        ov = torch.empty_like(ok)
        counter = {"i": 0}

        def step(ev):
            i = counter["i"]
            counter["i"] += 1
            sa = [Lc.store_args(l, D["kdec"], D["vdec"], D["steps_slots"][i], mode) for l in range(L)]
            ga = [Lc.gather_args(l, D["bt"], D["lens_at"][i], ok, ov) for l in range(L)]
            if ev: ev[0].record()
            for a in sa: Lc.store(a)
            if ev: ev[1].record()
            for a in ga: Lc.gather(a)
            if ev: ev[2].record()
        sec, evs = _timed(torch, step, args.steps, args.warmup)
        store_s = sum(e[0].elapsed_time(e[1]) for e in evs) / (args.steps * L) / 1e3
        gather_s = sum(e[1].elapsed_time(e[2]) for e in evs) / (args.steps * L) / 1e3
        lens_last = D["lens_at"][-1].cpu().numpy()
        ntok = int(lens_last.sum())
        sb, _ = algorithmic_bytes(mode, hd, hkv, bs, S * hkv)
        _, gb = algorithmic_bytes(mode, hd, hkv, bs, ntok * hkv)
        # every gather launch of the run (warmup steps included) reads its step's
        # lengths; the store launches mix the prefill's 32768-token calls with
        # the 256-token appends, so no single figure is theirs
        mean_tok = sum(int(x.sum()) for x in D["lens_at"]) / len(D["lens_at"])
        launch_bytes.update({f"gather/{hd}/{mode}": algorithmic_bytes(mode, hd, hkv, bs, mean_tok * hkv)[1]})
        # oracle sample: the oracle's own image of layer L-1 (its store of the
        # same seeded inputs), then its gather of 8 sequences, timed
        g, host = _decode_oracle_layer(D, torch, W, oracle)
        pick = list(range(0, S, S // 8))[:8]
        bt_h = D["st"].block_table.numpy()
        t0 = time.perf_counter()
        ko, vo = oracle.gather(g, host, 0, bt_h[pick], lens_last[pick])
        csec = time.perf_counter() - t0
        offs = np.concatenate([[0], np.cumsum(lens_last)])
        dk = np.concatenate([_bits(torch, ok[offs[b]: offs[b + 1]]) for b in pick])
        dv = np.concatenate([_bits(torch, ov[offs[b]: offs[b + 1]]) for b in pick])
        parity = bool(np.array_equal(dk, ko) and np.array_equal(dv, vo))
        sample_tok = int(lens_last[pick].sum())
        _, cgb = algorithmic_bytes(mode, hd, hkv, bs, sample_tok * hkv)
        cpu = {"value": round(cgb / csec / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"gather of 8 of {S} sequences ({sample_tok} tokens) of one layer, {csec:.2f} s wall"}
        res = _result(args, {"workload": D["desc"], "layers": L, "num_seqs": S, "context": D["ctx"],
                             "num_kv_heads": hkv, "head_dim": hd, "block_size": bs, "mode": args.mode},
                      L * (sb + gb) / sec / 1e9, sec * 1e3, sb, gb, store_s, gather_s, cpu, parity,
                      {"decode_store_us": round(store_s * 1e6, 2),
                       "appended_tokens_per_s": round(S / (L * store_s), 1),
                       "cache_GiB": round(D["cache"].bytes["total"] / 2**30, 3)})
        res["roofline"]["kernel"] = "gather_kernel"
        gg = gb / gather_s / 1e9
        res["roofline"]["achieved"] = round(gg, 1)
        res["roofline"]["frac"] = round(gg / HBM_PEAK_GBPS, 4)
    else:  # attention: one decode step = per layer, append one token per sequence, then attend
        D = _decode_setup(args, torch, kvq, W, dev)
        L, S, hkv, hd, bs, mode, Lc = D["L"], D["S"], D["hkv"], D["hd"], D["bs"], D["mode"], D["Lc"]
        H = hkv * args.q_per_kv
        sm_scale = 1.0 / math.sqrt(hd)
        nsteps = args.warmup + args.steps
        qs = [W.normal_kv(S, H, hd, seed=7000 + i, device=dev)[0] for i in range(nsteps)]
        out = torch.empty((S, H, hd), dtype=torch.bfloat16, device=dev)
        maxb = int(D["bt"].shape[1])
        wsb = kvq.kvq_decode_attention_workspace(D["cache"].handle, H, maxb, S)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        ct = __import__("ctypes")

        q_scales, q_scales_h = None, None
        if args.q_fp8:
            # static per-query-head scales calibrated on the first step's queries
            amax = torch.zeros(2 * H, dtype=torch.float32, device=dev)
            kvq.kvq_calibrate_amax(qs[0], qs[0], amax)
            q_scales_h = kvq.kvq_static_scales(amax, H, kvq.FP8_PER_HEAD)[:H]
            q_scales = torch.tensor(q_scales_h, dtype=torch.float32, device=dev)
        attn_fn = kvq._lib.kvq_decode_attention_fp8q if args.q_fp8 else kvq._lib.kvq_decode_attention

        def attn_args(l, i):
            qpart = (ct.c_void_p(qs[i].data_ptr()),) + ((ct.c_void_p(q_scales.data_ptr()),) if args.q_fp8 else ())
            return (D["cache"].handle, l) + qpart + (H, ct.c_void_p(D["bt"].data_ptr()), maxb,
                                                     ct.c_void_p(D["lens_at"][i].data_ptr()), S, ct.c_float(sm_scale),
                                                     ct.c_void_p(out.data_ptr()), ct.c_void_p(ws.data_ptr()), wsb,
                                                     Lc.stream)
        counter = {"i": 0}

        # every timed attention launch between its own pair of events, with its
        # algorithmic bytes: the roofline's average launch (fused steps and
        # attention-only passes alike, as a kernel trace of this run averages)
        per_launch = []

        def launch_bytes_at(i):
            return attention_bytes(mode, hd, hkv, bs, H, S, int(S) * (D["ctx"] + i + 1))

        def attend(a, i, ev):
            if ev:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record()
            st_ = attn_fn(*a)
            if st_ != 0:
                raise kvq.KVQError(st_, "kvq_decode_attention")
            if ev:
                e[1].record()
                per_launch.append((e, launch_bytes_at(i)))

        def step(ev):
            i = counter["i"]
            counter["i"] += 1
            sa = [Lc.store_args(l, D["kdec"], D["vdec"], D["steps_slots"][i], mode) for l in range(L)]
            aa = [attn_args(l, i) for l in range(L)]
            if ev: ev[0].record()
            for l in range(L):
                Lc.store(sa[l])
                attend(aa[l], i, ev)
            if ev: ev[1].record(); ev[2].record()
        sec, evs = _timed(torch, step, args.steps, args.warmup)
        step_s = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps / 1e3
        # the attention launches of the last step alone, for their own time
        last = [attn_args(l, nsteps - 1) for l in range(L)]

        def attn_only(ev):
            if ev: ev[0].record()
            for a in last:
                attend(a, nsteps - 1, ev)
            if ev: ev[1].record(); ev[2].record()
        _, aevs = _timed(torch, attn_only, args.steps, 1)
        attn_s = sum(e[0].elapsed_time(e[1]) for e in aevs) / (args.steps * L) / 1e3
        launch_s = sum(e[0].elapsed_time(e[1]) for e, _ in per_launch) / 1e3
        launch_gbps = sum(b for _, b in per_launch) / launch_s / 1e9
        launch_us = launch_s / len(per_launch) * 1e6
        if args.calibrate_copy:
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        lens_last = D["lens_at"][-1].cpu().numpy()
        ntok = int(lens_last.sum())
        sb, _ = algorithmic_bytes(mode, hd, hkv, bs, S * hkv)
        ab = attention_bytes(mode, hd, hkv, bs, H, S, ntok)
        agbps = ab / attn_s / 1e9
        attn_kernel = attention_kernel_name(mode, hd, args.q_per_kv, bs, hkv, args.q_fp8)
        # oracle check: layer L-1 of the last step for 8 sequences, from the
        # oracle's own image of that layer, within the kernel's error bound
        parity, cpu = None, None
        if not args.no_cpu_baseline:
            g, host = _decode_oracle_layer(D, torch, W, oracle)
            pick = list(range(0, S, S // 8))[:8]
            bt_h = D["st"].block_table.numpy()
            qb = _bits(torch, qs[-1])[pick]
            t0 = time.perf_counter()
            ref, absv = oracle.decode_attention(g, host, 0, qb, bt_h[pick], lens_last[pick], sm_scale, with_absv=True,
                                                q_scales=q_scales_h)
            csec = time.perf_counter() - t0
            tol = oracle.attention_error_bound(g, host, 0, qb, bt_h[pick], lens_last[pick], sm_scale, ref, absv,
                                               q_scales=q_scales_h)
            got = (_bits(torch, out[pick]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            parity = bool((np.abs(got - ref) <= tol).all())
            sample_tok = int(lens_last[pick].sum())
            cab = attention_bytes(mode, hd, hkv, bs, H, len(pick), sample_tok)
            cpu = {"value": round(cab / csec / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                   "kind": "oracle",
                   "sample": f"fp64 attention of 8 of {S} sequences ({sample_tok} cached tokens) "
                             f"of one layer, {csec:.2f} s wall"}
        res = {"metric": "decode attention over the quantized cache: cache GB/s read and decode tokens/s "
                         "(per-token-head FP8)",
               "value": round(L * (sb + ab) / sec / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "fp8/int4 codes, bf16 MFMA, f32 accumulate",
               "data": "synthetic",
               "config": {"workload": D["desc"] + f", {H} query heads, fused append + attention per layer"
                                                  + (", FP8 queries (static per-head scales)" if args.q_fp8 else ""),
                          "layers": L, "num_seqs": S, "context": D["ctx"], "num_kv_heads": hkv,
                          "num_q_heads": H, "head_dim": hd, "block_size": bs, "mode": args.mode,
                          "queries": "fp8" if args.q_fp8 else "bf16"},
               "attention_us": round(attn_s * 1e6, 2), "attention_GBps": round(agbps, 1),
               "step_ms_events": round(step_s * 1e3, 4),
               "decode_tokens_per_s": round(S / sec, 1),
               "attention_launch_us": round(launch_us, 2),
               "roofline": {"bound": "hbm", "kernel": attn_kernel, "achieved": round(launch_gbps, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(launch_gbps / HBM_PEAK_GBPS, 4),
                            "traffic": None if args.q_fp8 else measured_attention_traffic(args.mode, hd, args.tp)},
               "cpu_baseline": cpu,
               "parity_vs_oracle_sampled": parity,
               "workspace_bytes": wsb, "cache_GiB": round(D["cache"].bytes["total"] / 2**30, 3)}
    if args.calibrate_copy and name != "attention":
        # the counter runs' reference: copies of a known size
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    write_launch_bytes(args.launch_bytes_out, launch_bytes)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa32",
                    choices=["gqa32", "long80", "gptoss", "decode", "attention", "itl", "calib"],
                    help="gqa32 is the headline line; the others measure the remaining shapes")
    ap.add_argument("--head-dim", type=int, default=128, choices=[64, 128, 256], help="decode and attention workloads")
    ap.add_argument("--tp", type=int, default=1, choices=[1, 2, 4, 8],
                    help="gqa32, decode and attention workloads: one tensor-parallel shard's share, "
                         "8/TP KV heads per GPU")
    ap.add_argument("--layers", type=int, default=0, help="attention workload: layers (default: the workload's 32)")
    ap.add_argument("--block-size", type=int, default=0, choices=[0, 16, 32, 64, 128, 256],
                    help="gqa32: block size of the permuted cache (default: the workload's 16)")
    ap.add_argument("--q-per-kv", type=int, default=4, help="attention workload: query heads per KV head")
    ap.add_argument("--q-fp8", action="store_true", help="attention workload: FP8 queries (kvq_decode_attention_fp8q)")
    ap.add_argument("--mode", default="fp8_per_token_head",
                    choices=["fp8_per_token_head", "fp8_per_tensor", "fp8_per_head", "int4_per_token_head", "bf16"])
    ap.add_argument("--cpu-layers", type=int, default=16, help="layers of one step timed on the CPU oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="gqa32: time only the --mode layout (default: also the other three layouts of the target)")
    ap.add_argument("--no-ceiling", action="store_true", help="gqa32: skip the bandwidth-ceiling kernels")
    ap.add_argument("--token-order", action="store_true",
                    help="gqa32: store the tokens in their own order (kvq_store) instead of slot order "
                         "(kvq_store_ordered with the slot mapping's argsort)")
    ap.add_argument("--launch-bytes-out", default="",
                    help="write the algorithmic bytes per launch of each kernel run (JSON) for --summarize-kernels")
    ap.add_argument("--summarize-kernels", nargs="+",
                    metavar="ARG",
                    help="KERNEL_TRACE_DIR FETCH_DIR WRITE_DIR TAG LAUNCH_BYTES_JSON BENCH_ARGS [PMC_REGEX]: write "
                         "profiles/kernel_trace_TAG.md and traffic_TAG.md from rocprofv3 csv output and exit")
    ap.add_argument("--summarize-instructions", nargs="+", metavar="ARG",
                    help="TAG PMC_DIR...: write profiles/instructions_TAG.md from SQ counter runs and exit")
    ap.add_argument("--summarize-itl-trace", metavar="KERNEL_TRACE_DIR",
                    help="write profiles/kernel_trace_itl_gptoss_batch1.md from a kernel trace of --workload itl and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, copy 256 MiB device-to-device 3 times (reference for counter scaling)")
    ap.add_argument("--summarize-attention-profiles", nargs=3, metavar=("KERNEL_TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the attention profiles/ summaries (for --mode and --head-dim) and exit")
    args = ap.parse_args()
    if args.summarize_kernels:
        if len(args.summarize_kernels) not in (6, 7):
            ap.error("--summarize-kernels takes 6 or 7 arguments")
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_instructions:
        summarize_instructions(args.summarize_instructions[0], args.summarize_instructions[1:])
        return
    if args.summarize_itl_trace:
        summarize_itl_trace(args.summarize_itl_trace)
        return
    if args.summarize_attention_profiles:
        summarize_attention_profiles(*args.summarize_attention_profiles, args.mode, args.head_dim, args.layers, args.tp)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the store/gather path needs no collective and this build "
              "runs on a single MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_fp8_int4_amd as kvq
    import workloads as W

    if args.workload != "gqa32":
        run_other_workload(args, torch, kvq, W)
        return

    run_gqa32(args, torch, kvq, W)


def run_gqa32(args, torch, kvq, W):
    """The headline line: the GQA-32 step in the --mode layout (default
    per-token-head FP8), and beside it every other layout of the target (FP8
    per-tensor, FP8 static per-head, INT4 per-token-head) on the same inputs,
    each with its oracle check; the store's bandwidth ceilings (a linear
    non-temporal copy, the store's own access pattern without arithmetic)."""
    log("[bench] setting up gqa32 inputs on the device")
    I = gqa32_inputs(args, torch, W)
    L = I["L"]
    order = [args.mode] + ([m for m in GQA32_LAYOUTS if m != args.mode] if not args.headline_only else [])
    layouts, head = {}, None
    cpu = cpu_one = None
    launch_bytes = {}
    for name in order:
        LA = gqa32_layout(torch, kvq, W, I, name)
        store_s, gather_s, wall = time_layout(torch, kvq, LA, args.steps, args.warmup, ordered=not args.token_order)
        sg, gg = LA["store_bytes"] / store_s / 1e9, LA["gather_bytes"] / gather_s / 1e9
        log(f"[bench] {name}: {wall * 1e3:.3f} ms/step; store {store_s * 1e6:.2f} us ({sg:.0f} GB/s), "
            f"gather {gather_s * 1e6:.2f} us ({gg:.0f} GB/s)")
        rec = {"store_us": round(store_s * 1e6, 2), "store_GBps": round(sg, 1),
               "store_frac_of_peak": round(sg / HBM_PEAK_GBPS, 4), "gather_us": round(gather_s * 1e6, 2),
               "gather_GBps": round(gg, 1), "gather_frac_of_peak": round(gg / HBM_PEAK_GBPS, 4),
               "store_bytes_per_launch": int(LA["store_bytes"]), "gather_bytes_per_launch": int(LA["gather_bytes"])}
        rec["store_order"] = "slot" if not args.token_order and store_follows_order(LA["mode"], I["hd"]) else "token"
        if rec["store_order"] == "slot":
            # the same stores in token order, for comparison (same cache contents)
            tok_s, _, _ = time_layout(torch, kvq, LA, args.steps, args.warmup, ordered=False)
            tg = LA["store_bytes"] / tok_s / 1e9
            rec.update({"store_us_token_order": round(tok_s * 1e6, 2), "store_GBps_token_order": round(tg, 1),
                        "store_frac_of_peak_token_order": round(tg / HBM_PEAK_GBPS, 4)})
            log(f"[bench] {name}: store in token order {tok_s * 1e6:.2f} us ({tg:.0f} GB/s)")
        if name == args.mode:
            head = dict(LA=LA, store_s=store_s, gather_s=gather_s, wall=wall)
        # the oracle's check of this layout, while the outputs hold its gather
        if args.no_cpu_baseline:
            rec["parity_vs_oracle_sampled"] = None
        elif name == args.mode:
            nl = max(1, min(args.cpu_layers, L))
            log(f"[bench] cpu baseline: oracle on {nl} layers (store + gather)")
            secs, cores, parity, secs_one = oracle_leg(torch, W, I, LA, list(range(nl)), single_core=True)
            cpu = {"value": round(nl * (LA["store_bytes"] + LA["gather_bytes"]) / secs / 1e9, 3), "unit": "GB/s",
                   "cores": cores, "kind": "oracle",
                   "sample": f"{nl} of {L} layers of one step (store then gather of {I['n']} tokens each), "
                             f"{secs:.2f} s wall"}
            cpu_one = {"value": round((LA["store_bytes"] + LA["gather_bytes"]) / secs_one / 1e9, 3), "unit": "GB/s",
                       "cores": 1, "sample": f"1 layer (store then gather), {secs_one:.2f} s wall",
                       "cpu_model": cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0))}
            rec["parity_vs_oracle_sampled"] = parity
            rec["parity_layers"] = nl
        else:
            sample = [0, L - 1]
            _, _, parity, _ = oracle_leg(torch, W, I, LA, sample)
            rec["parity_vs_oracle_sampled"] = parity
            rec["parity_layers"] = len(sample)
        layouts[name] = rec
        launch_bytes[f"store/{I['hd']}/{LA['mode']}"] = LA["store_bytes"]
        launch_bytes[f"store/{I['hd']}/{LA['mode']}/ordered"] = LA["store_bytes"]
        launch_bytes[f"gather/{I['hd']}/{LA['mode']}"] = LA["gather_bytes"]
        if name != args.mode:
            LA["cache"].close()
            del LA
            torch.cuda.empty_cache()

    # Ceilings: what the memory system gives the store's bytes with no
    # arithmetic, on the same inputs, rotating over all 32 layers.
    LA = head["LA"]
    ceilings = {}
    if not args.no_ceiling:
        geos = {name: layout_geometry(kvq, W, I, name) for name in layouts}
        dev = I["keys"][0].device
        out_buf = torch.zeros(max(g["layers_bytes"] for g in geos.values()), dtype=torch.uint8, device=dev)
        reps = max(3, args.steps)
        ident_bt = torch.arange(I["nblocks"], dtype=torch.int32, device=dev).view(I["nseq"], -1)
        hg = geos[args.mode]
        ceilings["store_pattern_permuted_slots"] = store_pattern_ceiling(torch, I, hg, I["slots"], reps, out_buf)
        ceilings["store_pattern_permuted_slots_slot_order"] = store_pattern_ceiling(
            torch, I, hg, I["slots"], reps, out_buf, order=I["slot_order"])
        ceilings["store_pattern_identity_slots"] = store_pattern_ceiling(torch, I, hg, I["identity_slots"], reps,
                                                                         out_buf)
        ceilings["gather_pattern_permuted_blocks"] = gather_pattern_ceiling(torch, I, hg, I["bt_d"], reps, out_buf)
        ceilings["gather_pattern_identity_blocks"] = gather_pattern_ceiling(torch, I, hg, ident_bt, reps, out_buf)
        ceilings["linear_nt_copy"] = linear_copy_ceiling(torch, LA["store_bytes"], 16, reps)
        # the store launches one workgroup per 32 rows: 8192 at this shape
        store_grid = (I["n"] * I["hkv"] + 31) // 32
        ceilings["empty_launch_us"] = empty_launch_us(torch, (1, 1024, store_grid))
        for name, g in geos.items():
            # each store against the pattern of the order it takes the tokens in
            ordered = not args.token_order and store_follows_order(g["mode"], I["hd"])
            if name == args.mode:
                pc = ceilings["store_pattern_permuted_slots_slot_order" if ordered else "store_pattern_permuted_slots"]
                gc = ceilings["gather_pattern_permuted_blocks"]
            else:
                pc = store_pattern_ceiling(torch, I, g, I["slots"], reps, out_buf,
                                           order=I["slot_order"] if ordered else None)
                gc = gather_pattern_ceiling(torch, I, g, I["bt_d"], reps, out_buf)
            layouts[name]["store_pattern_ceiling_GBps"] = pc["GBps"]
            layouts[name]["store_vs_pattern_ceiling"] = round(layouts[name]["store_GBps"] / pc["GBps"], 4)
            layouts[name]["gather_pattern_ceiling_GBps"] = gc["GBps"]
            layouts[name]["gather_vs_pattern_ceiling"] = round(layouts[name]["gather_GBps"] / gc["GBps"], 4)
        del out_buf
        torch.cuda.empty_cache()
        log("[bench] ceilings: store pattern {:.0f} GB/s (permuted slots), {:.0f} (the same in slot order), "
            "{:.0f} (identity); gather pattern {:.0f} (permuted blocks), {:.0f} (identity); linear copy {:.0f}".format(
                *(ceilings[k]["GBps"] for k in ("store_pattern_permuted_slots",
                                                "store_pattern_permuted_slots_slot_order",
                                                "store_pattern_identity_slots",
                                                "gather_pattern_permuted_blocks", "gather_pattern_identity_blocks",
                                                "linear_nt_copy"))))

    store_s, gather_s, wall = head["store_s"], head["gather_s"], head["wall"]
    store_bytes, gather_bytes = LA["store_bytes"], LA["gather_bytes"]
    step_bytes = L * (store_bytes + gather_bytes)
    value = step_bytes / wall / 1e9
    store_gbps, gather_gbps = store_bytes / store_s / 1e9, gather_bytes / gather_s / 1e9
    dominant = "store" if store_s >= gather_s else "gather"
    dom_gbps = store_gbps if dominant == "store" else gather_gbps
    if ceilings:
        ceilings["store_vs_pattern_ceiling"] = layouts[args.mode]["store_vs_pattern_ceiling"]
        ceilings["gather_vs_pattern_ceiling"] = round(
            gather_gbps / ceilings["gather_pattern_permuted_blocks"]["GBps"], 4)
        ceilings["store_vs_linear_copy"] = round(store_gbps / ceilings["linear_nt_copy"]["GBps"], 4)
        # the store's rate over its bytes once the fixed cost of an empty
        # launch of the same grid is taken out of its time
        empty_s = ceilings["empty_launch_us"][f"grid_{(I['n'] * I['hkv'] + 31) // 32}"] / 1e6
        ceilings["store_GBps_beyond_empty_launch"] = round(store_bytes / (store_s - empty_s) / 1e9, 1)

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    write_launch_bytes(args.launch_bytes_out, launch_bytes)
    # the committed counters were taken on the default shape only
    traffic = measured_traffic() if args.tp == 1 and I["bs"] == 16 else None
    dom_key = f"{dominant}/{I['hd']}/{LA['mode']}"
    if dominant == "store" and layouts[args.mode].get("store_order") == "slot":
        dom_key += "/ordered"
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (f"gqa32 tensor-parallel shard (TP {args.tp}): 32 layers, {I['hkv']} of 8 KV heads per GPU, "
                                if args.tp > 1 else "gqa32: 32 layers, 8 KV heads, ")
                               + f"head_dim 128, block {I['bs']}, prefill of 8 x 4096 "
                               f"tokens per layer call, store + gather_dequant of every layer, {args.mode}",
                   "mode": args.mode, "layers": L, "tokens_per_layer_call": I["n"], "num_kv_heads": I["hkv"],
                   "head_dim": I["hd"], "block_size": I["bs"], "tp": args.tp,
                   "store_order": ("token order (kvq_store)" if args.token_order else
                                   "slot order: kvq_store_ordered with the argsort of the slot mapping, made on the "
                                   "host with the slot mapping and shared by the 32 layers (followed by FP8 layers "
                                   "at head_dim >= 128; INT4 takes the tokens in their own order)")},
        "store_GBps": round(store_gbps, 1),
        "gather_GBps": round(gather_gbps, 1),
        "store_frac_of_peak": round(store_gbps / HBM_PEAK_GBPS, 4),
        "gather_frac_of_peak": round(gather_gbps / HBM_PEAK_GBPS, 4),
        "store_us": round(store_s * 1e6, 2),
        "gather_us": round(gather_s * 1e6, 2),
        "cached_tokens_per_s": round(I["n"] / (L * store_s), 1),
        "algorithmic_bytes_per_step": int(step_bytes),
        "roofline": {"bound": "hbm", "kernel": f"{dominant}_kernel", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else traffic.get(dom_key)},
        "cpu_baseline": cpu,
        "cpu_single_core": cpu_one,
        "parity_vs_oracle_sampled": layouts[args.mode]["parity_vs_oracle_sampled"],
        "layouts": layouts,
        "ceilings": ceilings,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
