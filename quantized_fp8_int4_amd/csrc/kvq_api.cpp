// kvq_api.cpp -- the C ABI declared in include/kvq.h: argument validation,
// static-scale bookkeeping and kernel dispatch.  Every check runs before the
// first HIP call, so a rejected call enqueues nothing and writes nothing.
#include <algorithm>
#include <cmath>
#include <limits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvq_internal.h"

struct kvq_cache {
    kvq::Layout layout;
    uint8_t* dev = nullptr;
    uint64_t dev_bytes = 0;
    // Static scales of each layer as first stored (empty until then).
    std::vector<std::vector<float>> static_values;
};

namespace {

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("KVQ_LOG");
        return v && v[0] && v[0] != '0';
    }();
    return on;
}

const char* mode_name(int32_t m) {
    switch (m) {
        case KVQ_BF16: return "bf16";
        case KVQ_FP8_PER_TENSOR: return "fp8_per_tensor";
        case KVQ_FP8_PER_HEAD: return "fp8_per_head";
        case KVQ_FP8_PER_TOKEN_HEAD: return "fp8_per_token_head";
        case KVQ_INT4_PER_TOKEN_HEAD: return "int4_per_token_head";
        default: return "?";
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_INVALID_ARG: return "invalid argument";
        case KVQ_ERR_MODE_MISMATCH: return "mode does not match the layer's mode";
        case KVQ_ERR_BUFFER_TOO_SMALL: return "cache buffer smaller than kvq_cache_bytes().total";
        case KVQ_ERR_UNSUPPORTED: return "unsupported geometry";
        case KVQ_ERR_HIP: return "HIP runtime error";
        case KVQ_ERR_NO_SPACE: return "no free block left";
        default: return "unknown status";
    }
}

kvq_status kvq_cache_bytes(const kvq_cache_config* cfg, kvq_bytes* out) {
    if (!out) return KVQ_ERR_INVALID_ARG;
    kvq::Layout L;
    const kvq_status st = kvq::build_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    *out = L.bytes;
    return KVQ_OK;
}

kvq_status kvq_create_cache(const kvq_cache_config* cfg, void* dev_mem, uint64_t dev_bytes,
                            kvq_cache** out) {
    if (!out || !dev_mem) return KVQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(dev_mem) & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    kvq::Layout L;
    const kvq_status st = kvq::build_layout(cfg, &L);
    if (st != KVQ_OK) return st;
    if (dev_bytes < L.bytes.total) return KVQ_ERR_BUFFER_TOO_SMALL;
    kvq_cache* c = new (std::nothrow) kvq_cache;
    if (!c) return KVQ_ERR_INVALID_ARG;
    c->layout = std::move(L);
    c->dev = static_cast<uint8_t*>(dev_mem);
    c->dev_bytes = dev_bytes;
    c->static_values.resize(c->layout.num_layers);
    *out = c;
    return KVQ_OK;
}

kvq_status kvq_destroy_cache(kvq_cache* c) {
    delete c;
    return KVQ_OK;
}

namespace {

kvq_status store_impl(kvq_cache* c, int32_t layer, const void* keys, const void* values,
                      const int64_t* slot_mapping, const int32_t* token_order, int64_t num_tokens, kvq_mode mode,
                      const float* scales, void* stream) {
    if (!c || layer < 0 || layer >= c->layout.num_layers || num_tokens < 0) return KVQ_ERR_INVALID_ARG;
    const kvq::Layout& L = c->layout;
    const int32_t lmode = L.mode[layer];
    if (static_cast<int32_t>(mode) != lmode) return KVQ_ERR_MODE_MISMATCH;
    const bool is_static = kvq::has_static_scales(lmode);
    const int n_static = lmode == KVQ_FP8_PER_TENSOR ? 2 : 2 * L.num_kv_heads;
    if (!is_static && scales) return KVQ_ERR_INVALID_ARG;
    std::vector<float>& known = c->static_values[layer];
    bool first_static = false;
    if (is_static) {
        if (known.empty()) {
            if (!scales) return KVQ_ERR_INVALID_ARG;
            for (int i = 0; i < n_static; ++i)
                if (!(std::isfinite(scales[i]) && scales[i] > 0.0f)) return KVQ_ERR_INVALID_ARG;
            first_static = true;
        } else if (scales && std::memcmp(scales, known.data(), sizeof(float) * n_static) != 0) {
            return KVQ_ERR_INVALID_ARG;
        }
    }
    if (num_tokens == 0 && !first_static) return KVQ_OK;
    if (num_tokens > 0) {
        if (!keys || !values || !slot_mapping) return KVQ_ERR_INVALID_ARG;
        if (!aligned16(keys) || !aligned16(values) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
            return KVQ_ERR_INVALID_ARG;
        if (token_order && (reinterpret_cast<uintptr_t>(token_order) & 3u)) return KVQ_ERR_INVALID_ARG;
        if (num_tokens * static_cast<int64_t>(L.num_kv_heads) >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    }
    if (L.block_bytes[layer] % 16 != 0) return KVQ_ERR_UNSUPPORTED;

    float* static_dev = reinterpret_cast<float*>(c->dev + L.static_base[layer]);
    if (first_static) {
        const int e = kvq::launch_write_static(static_dev, scales, n_static, stream);
        if (e != 0) return KVQ_ERR_HIP;
        known.assign(scales, scales + n_static);
    }
    if (num_tokens == 0 || L.num_blocks[layer] == 0) return KVQ_OK;

    kvq::StoreLaunch a;
    a.keys = keys;
    a.values = values;
    a.slots = slot_mapping;
    a.layer = c->dev + L.layer_base[layer];
    a.static_scales = static_dev;
    a.num_rows = num_tokens * L.num_kv_heads;
    a.num_slots = L.num_blocks[layer] * static_cast<int64_t>(L.block_size);
    a.block_bytes = L.block_bytes[layer];
    a.code_bytes = L.code_bytes[layer];
    a.num_kv_heads = L.num_kv_heads;
    a.bs_log2 = L.bs_log2;
    a.head_dim = L.head_dim;
    a.mode = lmode;
    a.order = token_order;
    if (log_enabled())
        std::fprintf(stderr, "[kvq] store layer=%d mode=%s hd=%d tokens=%lld rows=%lld%s\n", layer,
                     mode_name(lmode), L.head_dim, static_cast<long long>(num_tokens),
                     static_cast<long long>(a.num_rows), token_order ? " ordered" : "");
    return kvq::launch_store(a, stream) == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

kvq_status kvq_store(kvq_cache* c, int32_t layer, const void* keys, const void* values,
                     const int64_t* slot_mapping, int64_t num_tokens, kvq_mode mode,
                     const float* scales, void* stream) {
    return store_impl(c, layer, keys, values, slot_mapping, nullptr, num_tokens, mode, scales, stream);
}

kvq_status kvq_store_ordered(kvq_cache* c, int32_t layer, const void* keys, const void* values,
                             const int64_t* slot_mapping, const int32_t* token_order, int64_t num_tokens,
                             kvq_mode mode, const float* scales, void* stream) {
    if (num_tokens > 0 && !token_order) return KVQ_ERR_INVALID_ARG;
    return store_impl(c, layer, keys, values, slot_mapping, token_order, num_tokens, mode, scales, stream);
}

int32_t kvq_store_follows_order(kvq_mode mode, int32_t head_dim) {
    const bool known = (head_dim == 64 || head_dim == 128 || head_dim == 256) && mode >= KVQ_BF16 &&
                       mode <= KVQ_INT4_PER_TOKEN_HEAD;
    return known && kvq::store_follows_order(head_dim, static_cast<int32_t>(mode)) ? 1 : 0;
}

kvq_status kvq_gather_dequant(const kvq_cache* c, int32_t layer, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                              void* out_keys, void* out_values, int64_t out_rows, void* stream) {
    if (!c || layer < 0 || layer >= c->layout.num_layers || num_seqs < 0) return KVQ_ERR_INVALID_ARG;
    if (num_seqs == 0) return KVQ_OK;
    // out_rows beyond 2^46 rows (at least 8 PiB of output) cannot be a real buffer
    if (out_rows < 0 || out_rows > (int64_t{1} << 46)) return KVQ_ERR_INVALID_ARG;
    if (max_blocks_per_seq < 1 || !block_table || !seq_lens) return KVQ_ERR_INVALID_ARG;
    if (out_rows > 0 && (!out_keys || !out_values)) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(out_keys) || !aligned16(out_values)) return KVQ_ERR_INVALID_ARG;
    const kvq::Layout& L = c->layout;
    const int32_t lmode = L.mode[layer];
    if (kvq::has_static_scales(lmode) && c->static_values[layer].empty()) return KVQ_ERR_INVALID_ARG;
    if (L.block_bytes[layer] % 16 != 0) return KVQ_ERR_UNSUPPORTED;

    kvq::GatherLaunch a;
    a.layer = c->dev + L.layer_base[layer];
    a.static_scales = reinterpret_cast<const float*>(c->dev + L.static_base[layer]);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.out_keys = out_keys;
    a.out_values = out_values;
    a.out_rows = out_rows;
    a.num_blocks = L.num_blocks[layer];
    a.block_bytes = L.block_bytes[layer];
    a.code_bytes = L.code_bytes[layer];
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = L.num_kv_heads;
    a.block_size = L.block_size;
    a.head_dim = L.head_dim;
    a.mode = lmode;
    if (kvq::gather_grid(a) >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    if (L.num_blocks[layer] == 0 || out_rows == 0) return KVQ_OK;
    if (log_enabled())
        std::fprintf(stderr, "[kvq] gather layer=%d mode=%s hd=%d seqs=%d max_blocks=%d\n", layer,
                     mode_name(lmode), L.head_dim, num_seqs, max_blocks_per_seq);
    return kvq::launch_gather(a, stream) == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

namespace {

kvq_status attention_args(const kvq_cache* c, int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t num_seqs) {
    if (!c || num_seqs < 0 || max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
    const kvq::Layout& L = c->layout;
    if (num_q_heads < 1 || num_q_heads % L.num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
    if ((static_cast<int64_t>(max_blocks_per_seq) << L.bs_log2) >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(num_seqs) * num_q_heads >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

}  // namespace

kvq_status kvq_decode_attention_workspace(const kvq_cache* c, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                          int32_t num_seqs, uint64_t* bytes) {
    if (!bytes) return KVQ_ERR_INVALID_ARG;
    const kvq_status st = attention_args(c, num_q_heads, max_blocks_per_seq, num_seqs);
    if (st != KVQ_OK) return st;
    const kvq::Layout& L = c->layout;
    *bytes = num_seqs == 0 ? 0
                           : kvq::attention_plan(L.block_size, L.num_kv_heads, L.head_dim, num_q_heads,
                                                 max_blocks_per_seq, num_seqs).workspace_bytes;
    return KVQ_OK;
}

}  // extern "C"

namespace {

kvq_status decode_attention(const kvq_cache* c, int32_t layer, const void* q, const float* q_scales,
                            int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, float sm_scale, void* out, void* workspace,
                            uint64_t workspace_bytes, void* stream, bool fixed_scratch = false) {
    if (!c || layer < 0 || layer >= c->layout.num_layers || num_seqs < 0) return KVQ_ERR_INVALID_ARG;
    if (num_seqs == 0) return KVQ_OK;
    const kvq_status st = attention_args(c, num_q_heads, max_blocks_per_seq, num_seqs);
    if (st != KVQ_OK) return st;
    if (!q || !block_table || !seq_lens || !out || !std::isfinite(sm_scale)) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return KVQ_ERR_INVALID_ARG;
    const kvq::Layout& L = c->layout;
    const int32_t lmode = L.mode[layer];
    if (kvq::has_static_scales(lmode) && c->static_values[layer].empty()) return KVQ_ERR_INVALID_ARG;
    if (L.block_bytes[layer] % 16 != 0) return KVQ_ERR_UNSUPPORTED;
    if (L.block_bytes[layer] >= (uint64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    if (q_scales && (lmode == KVQ_BF16 || lmode == KVQ_INT4_PER_TOKEN_HEAD)) return KVQ_ERR_UNSUPPORTED;
    if (q_scales && (reinterpret_cast<uintptr_t>(q_scales) & 3u)) return KVQ_ERR_INVALID_ARG;
    const kvq::AttnPlan plan =
        kvq::attention_plan(L.block_size, L.num_kv_heads, L.head_dim, num_q_heads, max_blocks_per_seq, num_seqs,
                            lmode, q_scales != nullptr);
    if (plan.grid >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    if (fixed_scratch) {
        // The allocation-free variant: split partials go to this device's
        // fixed array, looked up (never allocated) after every other check.
        if (plan.workspace_bytes > KVQ_ATTENTION_SCRATCH_BYTES) {
            if (log_enabled())
                std::fprintf(stderr, "[kvq] attention_noalloc: %llu bytes of split partials exceed the fixed %llu\n",
                             static_cast<unsigned long long>(plan.workspace_bytes),
                             static_cast<unsigned long long>(KVQ_ATTENTION_SCRATCH_BYTES));
            return KVQ_ERR_UNSUPPORTED;
        }
        workspace = nullptr;
        if (plan.workspace_bytes > 0 && kvq::attention_scratch(&workspace) != 0) return KVQ_ERR_HIP;
    } else if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes)) {
        return KVQ_ERR_BUFFER_TOO_SMALL;
    }

    kvq::AttnLaunch a;
    a.layer = c->dev + L.layer_base[layer];
    a.static_scales = reinterpret_cast<const float*>(c->dev + L.static_base[layer]);
    a.q = q;
    a.q_scales = q_scales;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.out = out;
    a.workspace = workspace;
    a.num_blocks = L.num_blocks[layer];
    a.block_bytes = L.block_bytes[layer];
    a.code_bytes = L.code_bytes[layer];
    a.num_kv_heads = L.num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.bs_log2 = L.bs_log2;
    a.head_dim = L.head_dim;
    a.mode = lmode;
    a.sm_scale = sm_scale;
    if (log_enabled())
        std::fprintf(stderr, "[kvq] attention layer=%d mode=%s hd=%d seqs=%d H=%d q=%s splits=%d tiles/split=%d\n",
                     layer, mode_name(lmode), L.head_dim, num_seqs, num_q_heads, q_scales ? "fp8" : "bf16",
                     plan.splits, plan.tiles_per_split);
    return kvq::launch_attention(a, plan, stream) == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const kvq_cache* c, int32_t layer, const void* q, int32_t num_q_heads,
                                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                int32_t num_seqs, float sm_scale, void* out, void* workspace,
                                uint64_t workspace_bytes, void* stream) {
    return decode_attention(c, layer, q, nullptr, num_q_heads, block_table, max_blocks_per_seq, seq_lens, num_seqs,
                            sm_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* c, int32_t layer, const void* q, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t num_seqs, float sm_scale, void* out,
                                        void* stream) {
    return decode_attention(c, layer, q, nullptr, num_q_heads, block_table, max_blocks_per_seq, seq_lens, num_seqs,
                            sm_scale, out, nullptr, 0, stream, /*fixed_scratch=*/true);
}

kvq_status kvq_decode_attention_fp8q(const kvq_cache* c, int32_t layer, const void* q, const float* q_scales,
                                     int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t num_seqs, float sm_scale, void* out,
                                     void* workspace, uint64_t workspace_bytes, void* stream) {
    if (!q_scales) return KVQ_ERR_INVALID_ARG;
    return decode_attention(c, layer, q, q_scales, num_q_heads, block_table, max_blocks_per_seq, seq_lens, num_seqs,
                            sm_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_calibrate_amax(const void* keys, const void* values, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, float* amax, int32_t accumulate, void* stream) {
    if (num_tokens < 0 || num_kv_heads < 1 || !amax) return KVQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(amax) & 3u) != 0) return KVQ_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KVQ_ERR_UNSUPPORTED;
    if (num_kv_heads > KVQ_MAX_STATIC_KV_HEADS) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens * static_cast<int64_t>(num_kv_heads) >= (int64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens > 0) {
        if (!keys || !values) return KVQ_ERR_INVALID_ARG;
        if (!aligned16(keys) || !aligned16(values)) return KVQ_ERR_INVALID_ARG;
    }
    if (num_tokens == 0 && accumulate) return KVQ_OK;
    kvq::CalibLaunch a;
    a.keys = keys;
    a.values = values;
    a.num_rows = num_tokens * num_kv_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.amax = amax;
    a.accumulate = accumulate;
    return kvq::launch_calibrate(a, stream) == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_static_scales(const float* amax, int32_t num_kv_heads, kvq_mode mode, float* scales) {
    if (!amax || !scales || num_kv_heads < 1) return KVQ_ERR_INVALID_ARG;
    if (mode != KVQ_FP8_PER_TENSOR && mode != KVQ_FP8_PER_HEAD) return KVQ_ERR_INVALID_ARG;
    for (int32_t i = 0; i < 2 * num_kv_heads; ++i)
        if (!(std::isfinite(amax[i]) && amax[i] >= 0.0f)) return KVQ_ERR_INVALID_ARG;
    // RN32(a / 448); the smallest positive FP32 value stands in for a zero scale
    auto scale = [](float a) {
        const float s = a / 448.0f;
        return s > 0.0f ? s : std::numeric_limits<float>::denorm_min();
    };
    if (mode == KVQ_FP8_PER_HEAD) {
        for (int32_t i = 0; i < 2 * num_kv_heads; ++i) scales[i] = scale(amax[i]);
    } else {
        for (int kv = 0; kv < 2; ++kv) {
            float m = 0.0f;
            for (int32_t h = 0; h < num_kv_heads; ++h) m = std::max(m, amax[kv * num_kv_heads + h]);
            scales[kv] = scale(m);
        }
    }
    return KVQ_OK;
}

}  // extern "C"
