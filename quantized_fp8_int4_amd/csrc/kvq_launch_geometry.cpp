// kvq_launch_geometry.cpp -- host-side launch geometry of the kernels (pure
// host code): the gather's workgroups per call and the decode attention's
// plan (splits, tiles per split, workspace).  The kernel sources launch with
// these values; the C ABI checks them (grids below 2^31, workspace sizes)
// before any HIP call.
#include "kvq_internal.h"

namespace kvq {

int64_t gather_parts(int64_t block_size, int64_t hkv, uint64_t hb, int cb, int u, int tpb) {
    const int64_t chunks = block_size * hkv * 2 * static_cast<int64_t>(hb / cb);
    const int64_t per = static_cast<int64_t>(tpb) * u;
    return (chunks + per - 1) / per;
}

int64_t gather_grid(const GatherLaunch& a) {
    const GatherTune t = gather_tune(a.head_dim, a.mode);
    return static_cast<int64_t>(a.num_seqs) * a.max_blocks *
           gather_parts(a.block_size, a.num_kv_heads, row_bytes(a.mode, a.head_dim), t.cb, t.u, t.tpb);
}

// One wave per KV head of a run of up to kAttnMaxHeadsPerWg heads in a
// workgroup (4 or 8 per head on the tile quads), up to 16 query heads per
// wave, tile ranges of one sequence per workgroup.
AttnPlan attention_plan(int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t num_q_heads,
                        int32_t max_blocks, int32_t num_seqs, int32_t mode, bool fp8_queries) {
    AttnPlan pl{};
    int hpw = 1;
    while (hpw < kAttnMaxHeadsPerWg && num_kv_heads % (2 * hpw) == 0) hpw *= 2;
    pl.heads_per_wg = hpw;
    const int group = num_q_heads / num_kv_heads;
    pl.qgroups = (group + 15) / 16;
    pl.kind = mode < 0 ? kAttnOneHead : attention_kind(mode, head_dim, group, block_size, hpw, fp8_queries);
    // waves per workgroup: one per KV head, 4 or 8 per KV head on the tile
    // quads
    const int64_t wpw = static_cast<int64_t>(hpw) * (pl.kind == kAttnTileQuads ? tquad_waves_per_head(mode, hpw) : 1);
    const int64_t units = static_cast<int64_t>(num_seqs) * (num_kv_heads / hpw) * pl.qgroups;
    const int64_t max_tiles = (static_cast<int64_t>(max_blocks) * block_size + kAttnTile - 1) / kAttnTile;
    // About 1024 waves in all (measured best against 4096 and 2048: a wave
    // streams best over a long tile range, and fewer splits write fewer
    // partials); a split keeps at least 8 tiles.  A long single sequence gets
    // up to 1024 / (waves per workgroup) splits; a large batch gets one split,
    // and the kernel then writes the output itself.  (Tile quads counted one
    // wave per head, as the other kernels, measured 4-20% slower on one or two
    // KV heads.)
    constexpr int64_t kTargetWaves = 1024, kMinTilesPerSplit = 8;
    static_assert(kTargetWaves <= kAttnMaxSplits, "the wide combine holds every split's weight");
    const int64_t want = (kTargetWaves / wpw + units - 1) / units;
    const int64_t cap = (max_tiles + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
    int64_t splits = want < cap ? want : cap;
    if (splits < 1) splits = 1;
    int64_t tps = (max_tiles + splits - 1) / splits;
    if (tps < 1) tps = 1;
    splits = (max_tiles + tps - 1) / tps;
    if (splits < 1) splits = 1;
    pl.splits = static_cast<int32_t>(splits);
    pl.tiles_per_split = static_cast<int32_t>(tps);
    pl.grid = units * splits;
    pl.workspace_bytes =
        splits > 1 ? static_cast<uint64_t>(num_seqs) * num_q_heads * splits * (head_dim + 2) * 4 : 0;
    return pl;
}

}  // namespace kvq
