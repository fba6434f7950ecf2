// kvq_planner.cpp -- capacity planning and the decode-time block manager for
// mixed FP8 / INT4 / BF16 layers with full and sliding-window retention
// (pure host code).
//
// Planning follows "FP8 KV cache layer skipping vs per-head scales", section
// "Layer skipping follows retained-token footprint": a full-attention layer
// at context T retains T positions, a sliding layer with window W at most W;
// A is the sum over layers and S the sum over the BF16 (skipped) layers, and
// "Per-token-head KV cache scale overhead", section "Convert bytes into block
// capacity": bytes per token times the block size, rounded to whole blocks,
// then the usable pool divided by the rounded block bytes.  The byte prices
// of each layer are the cache layout's own (kvq_layout.cpp), so a plan's
// block counts give a kvq_create_cache buffer that fits the pool.
//
// The manager hands out blocks to sequences layer group by layer group
// (layers with the same window share block ids, each in its own layer's
// region): full layers grow a block list, sliding layers keep a ring of
// W / block_size blocks in which token t lands at position t mod W.
#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "kvq_internal.h"

namespace {

struct Group {
    int32_t window = 0;                  // 0: full attention
    int64_t num_blocks = 0;              // blocks per layer of the group
    std::vector<int32_t> free;           // free block ids, next allocation at the back
};

struct Seq {
    int64_t len = 0;                     // tokens appended so far
    std::vector<std::vector<int32_t>> blocks;   // per group: block ids in logical order
};

kvq_status check_model(const kvq_model_config* m) {
    if (!m || !m->layer_mode || !m->layer_window) return KVQ_ERR_INVALID_ARG;
    if (m->num_layers < 1 || m->num_kv_heads < 1 || m->block_size < 1) return KVQ_ERR_INVALID_ARG;
    for (int32_t l = 0; l < m->num_layers; ++l) {
        const int32_t w = m->layer_window[l];
        if (w < 0 || (w > 0 && w % m->block_size != 0)) return KVQ_ERR_INVALID_ARG;
        if (m->layer_mode[l] < KVQ_BF16 || m->layer_mode[l] > KVQ_INT4_PER_TOKEN_HEAD) return KVQ_ERR_INVALID_ARG;
    }
    return KVQ_OK;
}

int64_t retained(int32_t window, int64_t context) {
    return window > 0 ? std::min<int64_t>(window, context) : context;
}

// Layout of num_seqs sequences of the given context (whole blocks per layer).
kvq_status layout_for(const kvq_model_config* m, int64_t context, int64_t num_seqs, std::vector<int64_t>* blocks,
                      kvq::Layout* out) {
    blocks->assign(m->num_layers, 0);
    for (int32_t l = 0; l < m->num_layers; ++l) {
        const int64_t per_seq = (retained(m->layer_window[l], context) + m->block_size - 1) / m->block_size;
        if (num_seqs > 0 && per_seq > (int64_t{1} << 31) / num_seqs) return KVQ_ERR_UNSUPPORTED;
        (*blocks)[l] = per_seq * num_seqs;
    }
    kvq_cache_config c;
    c.num_layers = m->num_layers;
    c.block_size = m->block_size;
    c.num_kv_heads = m->num_kv_heads;
    c.head_dim = m->head_dim;
    c.layer_mode = m->layer_mode;
    c.layer_num_blocks = blocks->data();
    return kvq::build_layout(&c, out);
}

}  // namespace

struct kvq_seq_manager {
    int32_t block_size = 0;
    int32_t max_blocks_per_seq = 0;
    std::vector<int32_t> layer_group;    // group of each layer
    std::vector<Group> groups;
    std::unordered_map<int32_t, Seq> seqs;
};

extern "C" {

kvq_status kvq_plan_capacity(const kvq_model_config* model, int64_t context, uint64_t pool_bytes, kvq_plan* out,
                             int64_t* layer_num_blocks) {
    if (!out || context < 1) return KVQ_ERR_INVALID_ARG;
    kvq_status st = check_model(model);
    if (st != KVQ_OK) return st;
    kvq_plan p{};
    for (int32_t l = 0; l < model->num_layers; ++l) {
        const int64_t r = retained(model->layer_window[l], context);
        p.retained_positions += r;
        if (model->layer_mode[l] == KVQ_BF16) p.skipped_positions += r;
    }
    std::vector<int64_t> blocks;
    kvq::Layout one, best;
    st = layout_for(model, context, 1, &blocks, &one);
    if (st != KVQ_OK) return st;
    p.sequence_bytes = one.bytes.payload + one.bytes.token_scales;
    // The largest N whose whole buffer (blocks, layer alignment, static
    // table) fits the pool: the buffer grows with N, so bisect on it.
    int64_t lo = 0, hi = static_cast<int64_t>(std::min<uint64_t>(pool_bytes / p.sequence_bytes, uint64_t{1} << 40));
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        kvq::Layout L;
        if (layout_for(model, context, mid, &blocks, &L) == KVQ_OK && L.bytes.total <= pool_bytes) lo = mid;
        else hi = mid - 1;
    }
    p.max_sequences = lo;
    p.max_tokens = lo * context;
    st = layout_for(model, context, lo, &blocks, &best);
    if (st != KVQ_OK) return st;
    p.buffer_bytes = lo > 0 ? best.bytes.total : 0;
    if (layer_num_blocks)
        for (int32_t l = 0; l < model->num_layers; ++l) layer_num_blocks[l] = blocks[l];
    *out = p;
    return KVQ_OK;
}

kvq_status kvq_manager_create(const kvq_model_config* model, const int64_t* layer_num_blocks,
                              int32_t max_blocks_per_seq, kvq_seq_manager** out) {
    if (!out || !layer_num_blocks || max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
    const kvq_status st = check_model(model);
    if (st != KVQ_OK) return st;
    kvq_seq_manager* m = new (std::nothrow) kvq_seq_manager;
    if (!m) return KVQ_ERR_INVALID_ARG;
    m->block_size = model->block_size;
    m->max_blocks_per_seq = max_blocks_per_seq;
    for (int32_t l = 0; l < model->num_layers; ++l) {
        const int32_t w = model->layer_window[l];
        int32_t g = -1;
        for (size_t i = 0; i < m->groups.size(); ++i)
            if (m->groups[i].window == w) g = static_cast<int32_t>(i);
        if (g < 0) {
            Group gr;
            gr.window = w;
            gr.num_blocks = layer_num_blocks[l];
            if (gr.num_blocks < 0 || gr.num_blocks > (int64_t{1} << 31) ||
                (w > 0 && w / model->block_size > max_blocks_per_seq)) {
                delete m;
                return KVQ_ERR_INVALID_ARG;
            }
            gr.free.reserve(static_cast<size_t>(gr.num_blocks));
            for (int64_t b = gr.num_blocks - 1; b >= 0; --b) gr.free.push_back(static_cast<int32_t>(b));
            m->groups.push_back(std::move(gr));
            g = static_cast<int32_t>(m->groups.size()) - 1;
        } else if (m->groups[g].num_blocks != layer_num_blocks[l]) {
            delete m;                    // one block id must name a block in every layer of a group
            return KVQ_ERR_INVALID_ARG;
        }
        m->layer_group.push_back(g);
    }
    *out = m;
    return KVQ_OK;
}

kvq_status kvq_manager_destroy(kvq_seq_manager* m) {
    delete m;
    return KVQ_OK;
}

kvq_status kvq_manager_num_groups(const kvq_seq_manager* m, int32_t* num_groups) {
    if (!m || !num_groups) return KVQ_ERR_INVALID_ARG;
    *num_groups = static_cast<int32_t>(m->groups.size());
    return KVQ_OK;
}

kvq_status kvq_manager_layer_group(const kvq_seq_manager* m, int32_t layer, int32_t* group) {
    if (!m || !group || layer < 0 || layer >= static_cast<int32_t>(m->layer_group.size())) return KVQ_ERR_INVALID_ARG;
    *group = m->layer_group[layer];
    return KVQ_OK;
}

kvq_status kvq_manager_append(kvq_seq_manager* m, int32_t seq, int32_t n, int64_t* slots) {
    if (!m || seq < 0 || n < 0 || (n > 0 && !slots)) return KVQ_ERR_INVALID_ARG;
    const int32_t bs = m->block_size;
    const int32_t ng = static_cast<int32_t>(m->groups.size());
    auto it = m->seqs.find(seq);
    const int64_t len0 = it == m->seqs.end() ? 0 : it->second.len;
    const int64_t len1 = len0 + n;
    // blocks still to allocate per group; check everything before changing anything
    std::vector<int64_t> need(ng, 0);
    for (int32_t g = 0; g < ng; ++g) {
        const Group& gr = m->groups[g];
        const int64_t held = it == m->seqs.end() ? 0 : static_cast<int64_t>(it->second.blocks[g].size());
        const int64_t want_pos = gr.window > 0 ? std::min<int64_t>(len1, gr.window) : len1;
        const int64_t want = (want_pos + bs - 1) / bs;
        if (want > m->max_blocks_per_seq) return KVQ_ERR_INVALID_ARG;
        need[g] = std::max<int64_t>(0, want - held);
        if (need[g] > static_cast<int64_t>(gr.free.size())) return KVQ_ERR_NO_SPACE;
    }
    Seq& s = m->seqs[seq];
    if (s.blocks.empty()) s.blocks.resize(ng);
    for (int32_t g = 0; g < ng; ++g) {
        Group& gr = m->groups[g];
        for (int64_t k = 0; k < need[g]; ++k) {
            s.blocks[g].push_back(gr.free.back());
            gr.free.pop_back();
        }
        for (int32_t i = 0; i < n; ++i) {
            const int64_t t = len0 + i;
            int64_t slot = -1;
            // a sliding layer keeps position t mod W; a token that a later
            // token of this same call displaces is not stored at all (-1), so
            // no two slots of one call coincide
            if (gr.window == 0 || t >= len1 - gr.window) {
                const int64_t pos = gr.window > 0 ? t % gr.window : t;
                slot = static_cast<int64_t>(s.blocks[g][pos / bs]) * bs + pos % bs;
            }
            slots[static_cast<int64_t>(g) * n + i] = slot;
        }
    }
    s.len = len1;
    return KVQ_OK;
}

kvq_status kvq_manager_release(kvq_seq_manager* m, int32_t seq) {
    if (!m) return KVQ_ERR_INVALID_ARG;
    auto it = m->seqs.find(seq);
    if (it == m->seqs.end()) return KVQ_ERR_INVALID_ARG;
    for (size_t g = 0; g < it->second.blocks.size(); ++g)
        for (auto b = it->second.blocks[g].rbegin(); b != it->second.blocks[g].rend(); ++b)
            m->groups[g].free.push_back(*b);
    m->seqs.erase(it);
    return KVQ_OK;
}

kvq_status kvq_manager_tables(const kvq_seq_manager* m, int32_t group, const int32_t* seqs, int32_t num_seqs,
                              int32_t max_blocks, int32_t* block_table, int32_t* seq_lens) {
    if (!m || group < 0 || group >= static_cast<int32_t>(m->groups.size()) || num_seqs < 0) return KVQ_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!seqs || !block_table || !seq_lens || max_blocks < 1)) return KVQ_ERR_INVALID_ARG;
    const Group& gr = m->groups[group];
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = m->seqs.find(seqs[i]);
        if (it == m->seqs.end()) return KVQ_ERR_INVALID_ARG;
        if (static_cast<int64_t>(it->second.blocks[group].size()) > max_blocks) return KVQ_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const Seq& s = m->seqs.find(seqs[i])->second;
        const std::vector<int32_t>& bl = s.blocks[group];
        for (int32_t j = 0; j < max_blocks; ++j)
            block_table[static_cast<int64_t>(i) * max_blocks + j] = j < static_cast<int32_t>(bl.size()) ? bl[j] : -1;
        const int64_t n = gr.window > 0 ? std::min<int64_t>(s.len, gr.window) : s.len;
        seq_lens[i] = static_cast<int32_t>(std::min<int64_t>(n, INT32_MAX));
    }
    return KVQ_OK;
}

}  // extern "C"
