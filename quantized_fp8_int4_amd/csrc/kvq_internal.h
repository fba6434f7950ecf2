// kvq_internal.h -- host-side layout description and kernel launchers shared
// by the C API (kvq_api.cpp), the layout module (kvq_layout.cpp) and the HIP
// kernels (kvq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <vector>

#include "kvq.h"

namespace kvq {

// Geometry of a cache buffer: where each layer's blocks and static scales
// live.  Layout as documented for kvq_cache_bytes in kvq.h.
struct Layout {
    int32_t num_layers = 0;
    int32_t block_size = 0;
    int32_t bs_log2 = 0;
    int32_t num_kv_heads = 0;
    int32_t head_dim = 0;
    std::vector<int32_t> mode;           // kvq_mode per layer
    std::vector<int64_t> num_blocks;     // blocks per layer
    std::vector<uint64_t> layer_base;    // byte offset of the layer's first block
    std::vector<uint64_t> static_base;   // byte offset of the layer's static scales
    std::vector<uint64_t> block_bytes;   // bytes of one block (codes + scale trailer)
    std::vector<uint64_t> code_bytes;    // bytes of a block's codes = trailer offset
    kvq_bytes bytes{};
};

// Bytes of one K (or V) row of head_dim elements in a layer of this mode.
uint64_t row_bytes(int32_t mode, int32_t head_dim);
bool has_token_scales(int32_t mode);
bool has_static_scales(int32_t mode);

// Validate cfg and fill *out.  No device call.
kvq_status build_layout(const kvq_cache_config* cfg, Layout* out);

// Division of a row index n < 2^31 by d >= 1: n / d == (n * magic) >> shift
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, with the 31-bit dividend bound).
struct DivMagic {
    uint32_t magic;
    uint32_t shift;
};
DivMagic div_magic(uint32_t d);

// ---- kernel launchers (kvq_kernels.hip) --------------------------------
struct StoreLaunch {
    const void* keys;
    const void* values;
    const int64_t* slots;
    uint8_t* layer;                // device: layer base
    const float* static_scales;    // device: this layer's static table entry (static modes)
    int64_t num_rows;              // num_tokens * num_kv_heads (< 2^31)
    int64_t num_slots;             // num_blocks * block_size
    uint64_t block_bytes;
    uint64_t code_bytes;
    int32_t num_kv_heads;
    int32_t bs_log2;
    int32_t head_dim;
    int32_t mode;
    const int32_t* order;          // device: token order (nullptr: token order)
};

// Whether the store follows a caller's token order (else it takes the tokens
// in their own order, which for a permutation stores the same bytes): where
// slot order measured faster on a 32768-token prefill under a random order of
// 16-token blocks (MI355X, HIP events): FP8 and BF16 at head_dim 128 and 256
// +2 to +6%; every mode at head_dim 64 -2 to -10%; INT4 -0.8% (head_dim 128)
// and +0.9% (256).
constexpr bool store_follows_order(int hd, int mode) {
    return mode != KVQ_INT4_PER_TOKEN_HEAD && hd >= 128;
}

struct GatherLaunch {
    const uint8_t* layer;
    const float* static_scales;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* out_keys;
    void* out_values;
    int64_t out_rows;              // token rows each output holds; rows past it are not written
    int64_t num_blocks;
    uint64_t block_bytes;
    uint64_t code_bytes;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t mode;
};

// Each returns 0 on a successful enqueue, else the hipError_t value.
int launch_store(const StoreLaunch& a, void* stream);
int launch_gather(const GatherLaunch& a, void* stream);

// Gather tuning, chosen by measurement on MI355X (32768 tokens x 8 KV heads
// per call), shared by the kernel dispatch and the host's grid arithmetic:
// cb code bytes per thread chunk (8 FP8, 4 INT4, 16 BF16: every wave-wide
// 16-byte store writes 1 KiB of contiguous BF16), u chunks per thread, tpb
// threads per workgroup (INT4 from head_dim 128 on: 512 threads of 4 chunks,
// +1.4% at 128 and +3.4% at 256; 5.5% slower at 64, where 256 threads of 8
// chunks stay).
struct GatherTune {
    int cb;
    int u;
    int tpb;
};
constexpr GatherTune gather_tune(int hd, int mode) {
    return (mode == KVQ_INT4_PER_TOKEN_HEAD && hd >= 128)
               ? GatherTune{4, 4, 512}
               : GatherTune{mode == KVQ_BF16 ? 16 : (mode == KVQ_INT4_PER_TOKEN_HEAD ? 4 : 8),
                            (hd == 64 || mode == KVQ_INT4_PER_TOKEN_HEAD || mode == KVQ_BF16) ? 8 : 4, 256};
}
// Workgroups per logical block: parts of up to tpb * u chunks of cb bytes.
int64_t gather_parts(int64_t block_size, int64_t hkv, uint64_t hb, int cb, int u, int tpb);
// Workgroups launch_gather uses (to reject grids of 2^31 or more).
int64_t gather_grid(const GatherLaunch& a);
int launch_write_static(float* dst, const float* values, int n, void* stream);

struct CalibLaunch {
    const void* keys;
    const void* values;
    int64_t num_rows;              // num_tokens * num_kv_heads (< 2^31)
    int32_t num_kv_heads;
    int32_t head_dim;
    float* amax;                   // device [2 * num_kv_heads]
    int32_t accumulate;
};
int launch_calibrate(const CalibLaunch& a, void* stream);

// ---- decode attention (kvq_attention.hip; plan in kvq_launch_geometry.cpp)
constexpr int kAttnTile = 16;          // tokens per attention tile
constexpr int kAttnMaxHeadsPerWg = 8;  // waves (KV heads) per attention workgroup
// Splits per sequence never exceed the plan's target wave count, so the wide
// combine's LDS weight table holds them all.
constexpr int kAttnMaxSplits = 4096;
// The decode-attention kernel that serves a call.  Head quads: per-token-head
// FP8 at head_dim 64 (BF16 or FP8 queries) and INT4 at head_dim 64 and 128
// (BF16 queries), with blocks of at least 16 tokens, query groups of at most
// 4 and 4 or 8 KV heads per workgroup.  Tile quads: the same layers with 1
// or 2 KV heads per workgroup, and FP8 at head_dim 128 (BF16 queries) with
// 2.  Any other call takes the one-head kernel.
enum AttnKind : int32_t { kAttnOneHead = 0, kAttnHeadQuads = 1, kAttnTileQuads = 2 };
constexpr int32_t attention_kind(int32_t mode, int32_t head_dim, int32_t group, int32_t block_size,
                                 int32_t heads_per_wg, bool fp8_queries) {
    const bool quad_layer = (mode == KVQ_FP8_PER_TOKEN_HEAD && head_dim == 64) ||
                            (mode == KVQ_INT4_PER_TOKEN_HEAD && !fp8_queries && (head_dim == 64 || head_dim == 128));
    // FP8 at head_dim 128 takes the tile quads as head pairs only: its
    // 16 KiB head-quad tiles are not built (the one-head kernel is bound by
    // memory there), and on one KV head the one-head kernel measured 3-5%
    // faster than the tile quads, on two 5% slower than the pairs
    const bool tile_layer = quad_layer || (mode == KVQ_FP8_PER_TOKEN_HEAD && !fp8_queries && head_dim == 128);
    if (!tile_layer || block_size < 16 || group > 4) return kAttnOneHead;
    if (heads_per_wg % 4 == 0) return quad_layer ? kAttnHeadQuads : kAttnOneHead;
    if (!quad_layer && heads_per_wg != 2) return kAttnOneHead;
    return kAttnTileQuads;
}

// Waves per KV head of the tile-quad kernel: 4, or 8 for INT4 on one KV head
// per workgroup (the VALU-heavier rounds gain from the extra waves, which
// the planner counts, so such calls split less).  At most 8 waves per
// workgroup either way.
constexpr int32_t tquad_waves_per_head(int32_t mode, int32_t heads_per_wg) {
    return mode == KVQ_INT4_PER_TOKEN_HEAD && heads_per_wg == 1 ? 8 : 4;
}

// Tile quads on two KV heads per workgroup run as head pairs: each round
// takes two tiles of both heads, whose K|V rows are adjacent in a block, so
// a wave reads both heads' rows as one contiguous run (whole lines where one
// head's rows are half a 128-byte line, INT4 at head_dim 64).  The pair's 8
// waves are the heads' 4 + 4.
constexpr bool tquad_head_pairs(int32_t heads_per_wg) { return heads_per_wg == 2; }

struct AttnPlan {
    int32_t splits;                // tile ranges per sequence
    int32_t tiles_per_split;       // 16-token tiles per range
    int32_t heads_per_wg;          // KV heads per workgroup
    int32_t qgroups;               // 16-query-head groups per KV head
    int32_t kind;                  // AttnKind of the kernel
    int64_t grid;                  // workgroups of the attention kernel
    uint64_t workspace_bytes;      // partial results (0 with one split)
};
// mode < 0 plans for the one-head kernel, whose partials are never fewer
// than those of the quads (the workspace a cache's calls need at most).
AttnPlan attention_plan(int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t num_q_heads,
                        int32_t max_blocks, int32_t num_seqs, int32_t mode = -1, bool fp8_queries = false);

struct AttnLaunch {
    const uint8_t* layer;
    const float* static_scales;
    const void* q;
    const float* q_scales;         // device [H] static FP8 query scales, or null for BF16 queries
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* out;
    void* workspace;
    int64_t num_blocks;
    uint64_t block_bytes;
    uint64_t code_bytes;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t bs_log2;
    int32_t head_dim;
    int32_t mode;
    float sm_scale;
};
int launch_attention(const AttnLaunch& a, const AttnPlan& plan, void* stream);
// Device address of this device's fixed split-partial array
// (KVQ_ATTENTION_SCRATCH_BYTES), looked up on the device's first call; 0 on
// success, else the hipError_t value.
int attention_scratch(void** ptr);

}  // namespace kvq
