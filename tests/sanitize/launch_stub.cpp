// launch_stub.cpp -- host stand-ins for the library's kernel launchers, so
// that its host half (kvq_api.cpp, kvq_layout.cpp, kvq_planner.cpp,
// kvq_launch_geometry.cpp) builds and runs without HIP under the address and
// undefined-behaviour sanitizers.  Each stand-in enqueues nothing; it counts
// the call and checks the launch description it was handed against the
// bounds the real kernels rely on, aborting on a violation.
#include <cstdio>
#include <cstdlib>

#include "kvq_internal.h"

namespace kvq_stub {
long stores = 0, gathers = 0, statics = 0, calibrations = 0, attentions = 0, scratch_lookups = 0;
// the fake device buffer of the cache under test: [base, base + bytes)
uintptr_t cache_base = 0;
uint64_t cache_bytes = 0;
}  // namespace kvq_stub

namespace {

void require(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "launch stub: %s\n", what);
        std::abort();
    }
}

void inside_cache(const void* p, uint64_t n, const char* what) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    require(a >= kvq_stub::cache_base && a + n <= kvq_stub::cache_base + kvq_stub::cache_bytes, what);
}

}  // namespace

namespace kvq {

int launch_store(const StoreLaunch& a, void*) {
    ++kvq_stub::stores;
    require(a.num_rows > 0 && a.num_rows < (int64_t{1} << 31), "store rows");
    require(a.num_rows % a.num_kv_heads == 0, "store rows are whole tokens");
    require(a.keys && a.values && a.slots, "store inputs");
    require((reinterpret_cast<uintptr_t>(a.order) & 3u) == 0, "store order aligned");
    require(a.block_bytes % 16 == 0 && a.code_bytes <= a.block_bytes, "store block bytes");
    require(a.num_slots % (int64_t{1} << a.bs_log2) == 0, "store slots are whole blocks");
    inside_cache(a.layer, (a.num_slots >> a.bs_log2) * a.block_bytes, "store layer inside the cache");
    return 0;
}

int launch_gather(const GatherLaunch& a, void*) {
    ++kvq_stub::gathers;
    require(a.num_seqs > 0 && a.max_blocks > 0, "gather shape");
    require(a.out_rows > 0 && a.out_keys && a.out_values, "gather outputs");
    require(gather_grid(a) < (int64_t{1} << 31), "gather grid");
    inside_cache(a.layer, a.num_blocks * a.block_bytes, "gather layer inside the cache");
    return 0;
}

int launch_write_static(float* dst, const float* values, int n, void*) {
    ++kvq_stub::statics;
    require(n >= 2 && n <= 2 * KVQ_MAX_STATIC_KV_HEADS && values, "static table size");
    inside_cache(dst, sizeof(float) * n, "static table inside the cache");
    return 0;
}

int launch_calibrate(const CalibLaunch& a, void*) {
    ++kvq_stub::calibrations;
    require(a.amax && a.num_kv_heads >= 1 && a.num_rows >= 0, "calibration");
    return 0;
}

int launch_attention(const AttnLaunch& a, const AttnPlan& plan, void*) {
    ++kvq_stub::attentions;
    require(a.num_seqs > 0 && a.num_q_heads % a.num_kv_heads == 0, "attention shape");
    require(plan.grid > 0 && plan.grid < (int64_t{1} << 31), "attention grid");
    require(plan.splits >= 1 && static_cast<int64_t>(plan.splits) * plan.tiles_per_split * 16 >=
                                    static_cast<int64_t>(a.max_blocks) << a.bs_log2,
            "attention splits cover the table");
    require(plan.workspace_bytes == 0 || a.workspace, "attention workspace");
    inside_cache(a.layer, a.num_blocks * a.block_bytes, "attention layer inside the cache");
    return 0;
}

int attention_scratch(void** ptr) {
    ++kvq_stub::scratch_lookups;
    static unsigned char fake[256] __attribute__((aligned(256)));
    *ptr = fake;               // never dereferenced: the stub launches nothing
    return 0;
}

}  // namespace kvq
