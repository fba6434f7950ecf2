// kvq_layout.cpp -- cache geometry and byte accounting (pure host code).
//
// Payload per retained token and KV head: 2 * head_dim * bytes_per_element
// ("Per-token-head KV cache scale overhead", "Per-token-head KV cache scale
// overhead"); dynamic layouts add one FP32 K and one FP32 V scale per slot,
// 8 bytes ("The FP8 scale tax is 4 divided by head size"; "INT4 makes the
// metadata fraction larger" for the packed half-width INT4 rows); storage is
// whole blocks of block_size tokens ("Convert bytes into block capacity").
// Static layouts store 2 FP32 values per layer (per-tensor) or per layer and
// KV head (per-head) ("Per-tensor vs per-head FP8 KV cache scales", "Static
// per-head metadata is almost free").  BF16 (skipped) layers cost 2 bytes per
// element and no scales ("FP8 KV cache layer skipping vs per-head scales",
// "Layer skipping follows retained-token footprint").
#include "kvq_internal.h"

namespace kvq {

namespace {
constexpr uint64_t kLayerAlign = 256;

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool valid_mode(int32_t m) { return m >= KVQ_BF16 && m <= KVQ_INT4_PER_TOKEN_HEAD; }
}  // namespace

uint64_t row_bytes(int32_t mode, int32_t head_dim) {
    const uint64_t hd = static_cast<uint64_t>(head_dim);
    switch (mode) {
        case KVQ_BF16: return 2 * hd;
        case KVQ_INT4_PER_TOKEN_HEAD: return hd / 2;
        default: return hd;
    }
}

bool has_token_scales(int32_t mode) {
    return mode == KVQ_FP8_PER_TOKEN_HEAD || mode == KVQ_INT4_PER_TOKEN_HEAD;
}

bool has_static_scales(int32_t mode) {
    return mode == KVQ_FP8_PER_TENSOR || mode == KVQ_FP8_PER_HEAD;
}

DivMagic div_magic(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;            // l = ceil(log2 d)
    const uint32_t p = 31 + l;
    const unsigned __int128 num = static_cast<unsigned __int128>(1) << p;
    const uint64_t m = static_cast<uint64_t>((num + d - 1) / d);   // < 2^32
    return DivMagic{static_cast<uint32_t>(m), p};
}

kvq_status build_layout(const kvq_cache_config* cfg, Layout* out) {
    if (!cfg || !out || !cfg->layer_mode || !cfg->layer_num_blocks) return KVQ_ERR_INVALID_ARG;
    if (cfg->num_layers < 1 || cfg->num_kv_heads < 1 || cfg->block_size < 1) return KVQ_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128 && cfg->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
    if (cfg->block_size > 1024 || (cfg->block_size & (cfg->block_size - 1)) != 0) return KVQ_ERR_UNSUPPORTED;
    if (cfg->num_kv_heads > (1 << 16)) return KVQ_ERR_UNSUPPORTED;

    Layout L;
    L.num_layers = cfg->num_layers;
    L.block_size = cfg->block_size;
    while ((1 << L.bs_log2) < cfg->block_size) ++L.bs_log2;
    L.num_kv_heads = cfg->num_kv_heads;
    L.head_dim = cfg->head_dim;
    const uint64_t bs = static_cast<uint64_t>(cfg->block_size);
    const uint64_t hkv = static_cast<uint64_t>(cfg->num_kv_heads);

    uint64_t off = 0, payload = 0, tok = 0, stat = 0;
    for (int32_t l = 0; l < cfg->num_layers; ++l) {
        const int32_t m = cfg->layer_mode[l];
        const int64_t nb = cfg->layer_num_blocks[l];
        if (!valid_mode(m) || nb < 0) return KVQ_ERR_INVALID_ARG;
        if (m == KVQ_FP8_PER_HEAD && hkv > KVQ_MAX_STATIC_KV_HEADS) return KVQ_ERR_UNSUPPORTED;
        if (static_cast<uint64_t>(nb) > (uint64_t{1} << 31) || bs * static_cast<uint64_t>(nb) > (uint64_t{1} << 40))
            return KVQ_ERR_UNSUPPORTED;
        const uint64_t code = bs * hkv * 2 * row_bytes(m, cfg->head_dim);
        const uint64_t trailer = has_token_scales(m) ? bs * hkv * 2 * 4 : 0;
        // the kernels address a block's bytes with 32-bit offsets
        if (code + trailer >= (uint64_t{1} << 31)) return KVQ_ERR_UNSUPPORTED;
        off = align_up(off, kLayerAlign);
        L.mode.push_back(m);
        L.num_blocks.push_back(nb);
        L.layer_base.push_back(off);
        L.code_bytes.push_back(code);
        L.block_bytes.push_back(code + trailer);
        off += static_cast<uint64_t>(nb) * (code + trailer);
        // (each term is below 2^62: nb <= 2^31 blocks of < 2^31 bytes)
        if (off > (uint64_t{1} << 62)) return KVQ_ERR_UNSUPPORTED;
        payload += static_cast<uint64_t>(nb) * code;
        tok += static_cast<uint64_t>(nb) * trailer;
    }
    off = align_up(off, kLayerAlign);
    for (int32_t l = 0; l < cfg->num_layers; ++l) {
        L.static_base.push_back(off);
        const int32_t m = L.mode[l];
        const uint64_t sb = (m == KVQ_FP8_PER_TENSOR) ? 8 : (m == KVQ_FP8_PER_HEAD ? 8 * hkv : 0);
        off += sb;
        stat += sb;
    }
    L.bytes.payload = payload;
    L.bytes.token_scales = tok;
    L.bytes.static_scales = stat;
    L.bytes.total = off;
    L.bytes.padding = off - payload - tok - stat;
    *out = std::move(L);
    return KVQ_OK;
}

}  // namespace kvq
