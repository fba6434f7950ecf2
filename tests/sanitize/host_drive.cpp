// host_drive.cpp -- drives the library's host half and the CPU oracle under
// AddressSanitizer and UndefinedBehaviorSanitizer (built by
// tests/test_sanitizers.py with g++/gcc, the kernel launches replaced by the
// checking stubs of launch_stub.cpp).
//
// Random geometries and operation sequences exercise:
//  A. byte accounting (kvq_cache_bytes) of valid and invalid geometries,
//     equal to the oracle's accounting wherever the library accepts one;
//  B. the C-ABI argument checks of store, gather, calibration and the decode
//     attention entry points: every result is a defined status, a refused
//     call enqueues nothing, an accepted one enqueues a launch whose
//     description the stub checks against the cache buffer;
//  C. the capacity planner (the plan fits the pool, one more sequence does
//     not) and the block manager (properties of the slots and block tables
//     it hands out over random appends and releases);
//  D. the oracle's store, gather, calibration and decode attention on tiny
//     random inputs with skipped and out-of-range slots, bad block-table
//     entries and clamped lengths.
// Exits 1 on a failed property; a sanitizer report aborts the run.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

extern "C" {
void orc_cache_bytes(int, int64_t, int64_t, int64_t, const int32_t*, const int64_t*, int64_t*);
void orc_store(int, int64_t, int64_t, int64_t, const int32_t*, const int64_t*, uint8_t*, int, const uint16_t*,
               const uint16_t*, const int64_t*, int64_t, const float*);
void orc_gather(int, int64_t, int64_t, int64_t, const int32_t*, const int64_t*, const uint8_t*, int, const int32_t*,
                int64_t, const int32_t*, int64_t, uint16_t*, uint16_t*);
void orc_calibrate_amax(const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, float*, int);
void orc_decode_attention(int, int64_t, int64_t, int64_t, const int32_t*, const int64_t*, const uint8_t*, int,
                          const uint16_t*, int64_t, const int32_t*, int64_t, const int32_t*, int64_t, double,
                          const float*, double*, double*);
void orc_set_num_threads(int);
}

namespace kvq_stub {
extern long stores, gathers, statics, calibrations, attentions, scratch_lookups;
extern uintptr_t cache_base;
extern uint64_t cache_bytes;
}  // namespace kvq_stub

#define CHECK(c, ...)                                                       \
    do {                                                                    \
        if (!(c)) {                                                         \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);       \
            std::fprintf(stderr, __VA_ARGS__);                              \
            std::fputc('\n', stderr);                                       \
            std::exit(1);                                                   \
        }                                                                   \
    } while (0)

namespace {

// splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014)
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    int64_t in(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next() % static_cast<uint64_t>(hi - lo + 1)); }
    bool p(double prob) { return (next() >> 11) * (1.0 / 9007199254740992.0) < prob; }
    template <class T>
    T pick(const std::vector<T>& v) { return v[next() % v.size()]; }
};

constexpr uintptr_t kFake = 0x7F0000000000ull;     // 256-byte aligned; never dereferenced

bool status_ok(int st) { return st <= 0 && st >= -6; }

long launches() {
    return kvq_stub::stores + kvq_stub::gathers + kvq_stub::statics + kvq_stub::calibrations + kvq_stub::attentions +
           kvq_stub::scratch_lookups;
}

// ------------------------------------------------------------------ A
void drive_accounting(Rng& r) {
    const std::vector<int32_t> bss = {1, 2, 4, 16, 64, 1024, 3, 2048, 0, -4};
    const std::vector<int32_t> hkvs = {1, 2, 3, 8, 16, 1024, 4096, 65536, 65537, 0, -1};
    const std::vector<int32_t> hds = {64, 128, 256, 32, 512, 0};
    const std::vector<int64_t> nbs = {0, 1, 7, 100, 4096, int64_t{1} << 20, (int64_t{1} << 31) + 1, -3};
    long accepted = 0;
    for (int i = 0; i < 4000; ++i) {
        const int nl = static_cast<int>(r.in(1, 6));
        std::vector<int32_t> modes(nl);
        std::vector<int64_t> nb(nl);
        for (int l = 0; l < nl; ++l) {
            modes[l] = static_cast<int32_t>(r.p(0.05) ? r.in(-2, 7) : r.in(0, 4));
            nb[l] = r.p(0.7) ? r.in(0, 300) : r.pick(nbs);
        }
        kvq_cache_config cfg{nl, r.pick(bss), r.pick(hkvs), r.pick(hds), modes.data(), nb.data()};
        kvq_bytes b{};
        const int st = kvq_cache_bytes(&cfg, &b);
        CHECK(st == KVQ_OK || st == KVQ_ERR_INVALID_ARG || st == KVQ_ERR_UNSUPPORTED, "cache_bytes status %d", st);
        if (st != KVQ_OK) continue;
        ++accepted;
        CHECK(b.total == b.payload + b.token_scales + b.static_scales + b.padding, "total is the sum of its parts");
        CHECK(b.total < (uint64_t{1} << 62), "accepted totals stay far from overflow");
        if (b.total < (uint64_t{1} << 50)) {
            int64_t o[5];
            orc_cache_bytes(nl, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, modes.data(), nb.data(), o);
            CHECK(static_cast<uint64_t>(o[0]) == b.payload && static_cast<uint64_t>(o[1]) == b.token_scales &&
                      static_cast<uint64_t>(o[2]) == b.static_scales && static_cast<uint64_t>(o[4]) == b.total,
                  "library and oracle accounting differ");
        }
    }
    CHECK(accepted > 300, "too few accepted geometries (%ld)", accepted);
    kvq_bytes b{};
    CHECK(kvq_cache_bytes(nullptr, &b) == KVQ_ERR_INVALID_ARG, "null config");
    int32_t m = KVQ_BF16;
    int64_t n = 1;
    kvq_cache_config cfg{1, 16, 2, 64, &m, &n};
    CHECK(kvq_cache_bytes(&cfg, nullptr) == KVQ_ERR_INVALID_ARG, "null output");
    cfg.layer_mode = nullptr;
    CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_ERR_INVALID_ARG, "null modes");
    // many layers of the largest blocks: refused, not wrapped around
    std::vector<int32_t> big_m(1 << 13, KVQ_BF16);
    std::vector<int64_t> big_n(1 << 13, int64_t{1} << 30);
    kvq_cache_config big{1 << 13, 1, 1024, 256, big_m.data(), big_n.data()};
    CHECK(kvq_cache_bytes(&big, &b) == KVQ_ERR_UNSUPPORTED, "a buffer beyond 2^62 bytes is refused");
    std::printf("A accounting: %ld accepted geometries\n", accepted);
}

// ------------------------------------------------------------------ B
void* fake_ptr(Rng& r) {
    switch (r.in(0, 9)) {
        case 0: return nullptr;
        case 1: return reinterpret_cast<void*>(kFake + 2);
        case 2: return reinterpret_cast<void*>(kFake + 8);
        default: return reinterpret_cast<void*>(kFake + 16 * r.in(0, 1 << 20));
    }
}

void drive_abi(Rng& r) {
    long ok_calls = 0, refused = 0;
    for (int trial = 0; trial < 150; ++trial) {
        const int nl = static_cast<int>(r.in(1, 4));
        std::vector<int32_t> modes(nl);
        std::vector<int64_t> nb(nl);
        for (int l = 0; l < nl; ++l) {
            modes[l] = static_cast<int32_t>(r.in(0, 4));
            nb[l] = r.in(0, 40);
        }
        const int32_t bs = static_cast<int32_t>(int64_t{1} << r.in(0, 6));
        const int32_t hkv = static_cast<int32_t>(r.in(1, 8));
        const int32_t hd = r.pick(std::vector<int32_t>{64, 128, 256});
        kvq_cache_config cfg{nl, bs, hkv, hd, modes.data(), nb.data()};
        kvq_bytes b{};
        CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_OK, "valid geometry refused");
        kvq_stub::cache_base = kFake;
        kvq_stub::cache_bytes = b.total;
        kvq_cache* c = nullptr;
        CHECK(kvq_create_cache(&cfg, reinterpret_cast<void*>(kFake), b.total - 1, &c) ==
                  (b.total > 0 ? KVQ_ERR_BUFFER_TOO_SMALL : KVQ_OK),
              "short buffer");
        if (c) kvq_destroy_cache(c);
        CHECK(kvq_create_cache(&cfg, reinterpret_cast<void*>(kFake + 64), b.total, &c) == KVQ_ERR_INVALID_ARG,
              "unaligned buffer");
        CHECK(kvq_create_cache(&cfg, reinterpret_cast<void*>(kFake), b.total, &c) == KVQ_OK, "create");
        for (int call = 0; call < 300; ++call) {
            const long before = launches();
            const int32_t layer = static_cast<int32_t>(r.in(-1, nl));
            int st = 0;
            const int op = static_cast<int>(r.in(0, 6));
            if (op == 0) {
                const int64_t n = r.pick(std::vector<int64_t>{-1, 0, 1, 5, 33, int64_t{1} << 30});
                float sc[2 * 8 + 2];
                for (float& x : sc) x = r.pick(std::vector<float>{1.0f, 0.02f, 0.0f, -1.0f, NAN, INFINITY, 3e38f});
                const bool with = r.p(0.5);
                // mostly the layer's own mode, so that the launch path is reached often
                const int mode = (layer >= 0 && layer < nl && r.p(0.8)) ? modes[layer] : static_cast<int>(r.in(0, 5));
                if (r.p(0.5)) {
                    st = kvq_store(c, layer, fake_ptr(r), fake_ptr(r), static_cast<const int64_t*>(fake_ptr(r)), n,
                                   static_cast<kvq_mode>(mode), with ? sc : nullptr, nullptr);
                } else {
                    const int32_t* order = static_cast<const int32_t*>(fake_ptr(r));
                    st = kvq_store_ordered(c, layer, fake_ptr(r), fake_ptr(r),
                                           static_cast<const int64_t*>(fake_ptr(r)), order, n,
                                           static_cast<kvq_mode>(mode), with ? sc : nullptr, nullptr);
                    CHECK(!(n > 0 && order == nullptr && st == KVQ_OK), "ordered store without an order refused");
                }
            } else if (op == 1) {
                st = kvq_gather_dequant(c, layer, static_cast<const int32_t*>(fake_ptr(r)),
                                        static_cast<int32_t>(r.in(-1, 70)), static_cast<const int32_t*>(fake_ptr(r)),
                                        static_cast<int32_t>(r.pick(std::vector<int64_t>{-1, 0, 1, 3, 300, 1 << 20})),
                                        fake_ptr(r), fake_ptr(r), r.pick(std::vector<int64_t>{-1, 0, 1, 100, int64_t{1} << 47}),
                                        nullptr);
            } else if (op == 2 || op == 3) {
                const int32_t H = static_cast<int32_t>(hkv * r.in(0, 5) + (r.p(0.1) ? 1 : 0));
                const int32_t maxb = static_cast<int32_t>(r.pick(std::vector<int64_t>{-1, 0, 1, 8, 100, 1 << 27}));
                const int32_t ns = static_cast<int32_t>(r.pick(std::vector<int64_t>{-1, 0, 1, 4, 1000}));
                const float sm = r.pick(std::vector<float>{0.125f, NAN, 0.0f});
                if (op == 2) {
                    uint64_t need = 0;
                    const int ws_st = kvq_decode_attention_workspace(c, H, maxb, ns, &need);
                    CHECK(status_ok(ws_st), "workspace status");
                    const uint64_t have = r.p(0.5) ? need : (need ? need - 1 : 0);
                    void* const ws = r.p(0.8) ? reinterpret_cast<void*>(kFake) : nullptr;
                    st = kvq_decode_attention(c, layer, fake_ptr(r), H, static_cast<const int32_t*>(fake_ptr(r)), maxb,
                                              static_cast<const int32_t*>(fake_ptr(r)), ns, sm, fake_ptr(r), ws, have,
                                              nullptr);
                    // the query covers every layer of the cache; a layer whose
                    // kernel splits less (the tile quads) needs no more
                    if (st == KVQ_OK && ns > 0) {
                        const kvq::AttnPlan pl =
                            kvq::attention_plan(bs, hkv, hd, H, maxb, ns, modes[layer], false);
                        CHECK(ws_st == KVQ_OK && have >= pl.workspace_bytes && pl.workspace_bytes <= need,
                              "workspace honoured");
                    }
                    CHECK(!(ws_st == KVQ_OK && ws && have >= need && st == KVQ_ERR_BUFFER_TOO_SMALL), "query sufficient");
                } else {
                    st = kvq_decode_attention_noalloc(c, layer, fake_ptr(r), H, static_cast<const int32_t*>(fake_ptr(r)),
                                                      maxb, static_cast<const int32_t*>(fake_ptr(r)), ns, sm,
                                                      fake_ptr(r), nullptr);
                }
            } else if (op == 4) {
                st = kvq_decode_attention_fp8q(c, layer, fake_ptr(r), static_cast<const float*>(fake_ptr(r)),
                                               static_cast<int32_t>(hkv * r.in(0, 3)),
                                               static_cast<const int32_t*>(fake_ptr(r)), static_cast<int32_t>(r.in(0, 9)),
                                               static_cast<const int32_t*>(fake_ptr(r)), static_cast<int32_t>(r.in(-1, 3)),
                                               0.1f, fake_ptr(r), reinterpret_cast<void*>(kFake), 1 << 20, nullptr);
            } else if (op == 5) {
                st = kvq_calibrate_amax(fake_ptr(r), fake_ptr(r), r.in(-1, 100), static_cast<int32_t>(r.in(0, 300)),
                                        r.pick(std::vector<int32_t>{64, 96, 128, 256}), static_cast<float*>(fake_ptr(r)),
                                        static_cast<int32_t>(r.in(0, 1)), nullptr);
            } else {
                float amax[2 * 9], out[2 * 9];
                for (float& x : amax) x = r.pick(std::vector<float>{0.0f, 1.0f, 448.0f, -1.0f, NAN, 1e-40f});
                st = kvq_static_scales(r.p(0.9) ? amax : nullptr, static_cast<int32_t>(r.in(0, 9)),
                                       static_cast<kvq_mode>(r.in(0, 4)), out);
                CHECK(launches() == before, "static scales are host arithmetic");
            }
            CHECK(status_ok(st), "op %d status %d", op, st);
            if (st != KVQ_OK) {
                ++refused;
                CHECK(launches() == before, "op %d refused with %d but enqueued work", op, st);
            } else {
                ++ok_calls;
            }
        }
        CHECK(kvq_destroy_cache(c) == KVQ_OK, "destroy");
    }
    CHECK(kvq_destroy_cache(nullptr) == KVQ_OK, "destroy null");
    std::printf("B c-abi: %ld accepted, %ld refused calls; stub launches: store %ld gather %ld static %ld calib %ld "
                "attention %ld scratch %ld\n",
                ok_calls, refused, kvq_stub::stores, kvq_stub::gathers, kvq_stub::statics, kvq_stub::calibrations,
                kvq_stub::attentions, kvq_stub::scratch_lookups);
    CHECK(kvq_stub::stores > 100 && kvq_stub::statics > 10 && kvq_stub::gathers > 100 && kvq_stub::attentions > 100 &&
              kvq_stub::scratch_lookups > 10,
          "launch paths reached");
}

// ------------------------------------------------------------------ C
void drive_planner(Rng& r) {
    long plans = 0;
    for (int i = 0; i < 300; ++i) {
        const int nl = static_cast<int>(r.in(1, 6));
        const int32_t bs = static_cast<int32_t>(int64_t{1} << r.in(0, 5));
        std::vector<int32_t> modes(nl), wins(nl);
        for (int l = 0; l < nl; ++l) {
            modes[l] = static_cast<int32_t>(r.in(0, 4));
            wins[l] = r.p(0.4) ? static_cast<int32_t>(bs * r.in(1, 8)) : 0;
        }
        kvq_model_config m{nl, bs, static_cast<int32_t>(r.in(1, 8)), r.pick(std::vector<int32_t>{64, 128, 256}),
                           modes.data(), wins.data()};
        const int64_t ctx = r.in(1, 5000);
        const uint64_t pool = static_cast<uint64_t>(r.in(0, int64_t{1} << 32));
        kvq_plan p{};
        std::vector<int64_t> blocks(nl);
        const int st = kvq_plan_capacity(&m, ctx, pool, &p, blocks.data());
        CHECK(status_ok(st), "plan status");
        if (st != KVQ_OK) continue;
        ++plans;
        CHECK(p.buffer_bytes <= pool, "the plan fits the pool");
        CHECK(p.max_tokens == p.max_sequences * ctx, "tokens of the plan");
        // one more sequence would not fit
        std::vector<int64_t> more(nl);
        for (int l = 0; l < nl; ++l) {
            const int64_t ret = wins[l] ? std::min<int64_t>(wins[l], ctx) : ctx;
            more[l] = (p.max_sequences + 1) * ((ret + bs - 1) / bs);
            CHECK(blocks[l] == p.max_sequences * ((ret + bs - 1) / bs), "planned blocks");
        }
        kvq_cache_config cfg{nl, bs, m.num_kv_heads, m.head_dim, modes.data(), more.data()};
        kvq_bytes b{};
        if (kvq_cache_bytes(&cfg, &b) == KVQ_OK) CHECK(b.total > pool, "one more sequence would fit");
    }
    CHECK(plans > 50, "too few plans (%ld)", plans);

    // block manager: random appends and releases, properties of what it hands out
    long appends = 0;
    for (int trial = 0; trial < 30; ++trial) {
        const int32_t bs = static_cast<int32_t>(int64_t{1} << r.in(0, 4));
        const std::vector<int32_t> wins = {0, 2 * bs, 0, 2 * bs, 4 * bs};
        const std::vector<int32_t> modes = {KVQ_FP8_PER_TOKEN_HEAD, KVQ_BF16, KVQ_INT4_PER_TOKEN_HEAD, KVQ_BF16,
                                            KVQ_BF16};
        kvq_model_config m{5, bs, 2, 64, modes.data(), wins.data()};
        const std::vector<int32_t> gw = {0, 2 * bs, 4 * bs};            // groups in order of first layer
        const std::vector<int64_t> gblocks = {r.in(1, 40), r.in(2, 14), r.in(4, 18)};
        const std::vector<int64_t> per_layer = {gblocks[0], gblocks[1], gblocks[0], gblocks[1], gblocks[2]};
        const int32_t maxb = static_cast<int32_t>(r.in(4, 24));
        kvq_seq_manager* mg = nullptr;
        CHECK(kvq_manager_create(&m, per_layer.data(), maxb, &mg) == KVQ_OK, "manager create");
        int32_t ng = 0;
        CHECK(kvq_manager_num_groups(mg, &ng) == KVQ_OK && ng == 3, "groups");
        std::map<int32_t, std::vector<std::vector<int64_t>>> hist;     // seq -> group -> slots of tokens
        for (int step = 0; step < 300; ++step) {
            if (!hist.empty() && r.p(0.08)) {
                auto it = hist.begin();
                std::advance(it, r.in(0, static_cast<int64_t>(hist.size()) - 1));
                CHECK(kvq_manager_release(mg, it->first) == KVQ_OK, "release");
                hist.erase(it);
            } else {
                const int32_t seq = static_cast<int32_t>(r.in(0, 5));
                const int32_t n = r.pick(std::vector<int32_t>{0, 1, 1, 1, 3, 17, 40});
                std::vector<int64_t> slots(3 * static_cast<size_t>(n) + 1, -99);
                const int st = kvq_manager_append(mg, seq, n, slots.data());
                CHECK(st == KVQ_OK || st == KVQ_ERR_NO_SPACE || st == KVQ_ERR_INVALID_ARG, "append status");
                if (st != KVQ_OK) continue;
                ++appends;
                auto& h = hist[seq];
                h.resize(3);
                for (int g = 0; g < 3; ++g) {
                    std::set<int64_t> seen;
                    int skipped = 0;
                    for (int i = 0; i < n; ++i) {
                        const int64_t s = slots[static_cast<size_t>(g) * n + i];
                        if (s < 0) {
                            ++skipped;
                        } else {
                            CHECK(seen.insert(s).second, "one call repeats a slot");
                        }
                        h[g].push_back(s);
                    }
                    CHECK(skipped == (gw[g] ? std::max(0, n - gw[g]) : 0), "displaced tokens of one call");
                }
            }
            for (int g = 0; g < 3; ++g) {
                std::set<int64_t> live;
                size_t live_n = 0;
                for (auto& kv : hist) {
                    const std::vector<int64_t>& sl = kv.second[g];
                    const size_t w = static_cast<size_t>(gw[g]);
                    const size_t first = (w && sl.size() > w) ? sl.size() - w : 0;
                    for (size_t t = first; t < sl.size(); ++t) {
                        CHECK(sl[t] >= 0 && sl[t] < gblocks[g] * bs, "live slot inside the layer");
                        live.insert(sl[t]);
                        ++live_n;
                    }
                    if (w)
                        for (size_t t = 0; t + w < sl.size(); ++t)
                            CHECK(sl[t] == sl[t + w] || sl[t] < 0 || sl[t + w] < 0, "ring position reuse");
                    int32_t seqid = kv.first, len = -1;
                    std::vector<int32_t> bt(static_cast<size_t>(maxb), -7);
                    CHECK(kvq_manager_tables(mg, g, &seqid, 1, maxb, bt.data(), &len) == KVQ_OK, "tables");
                    CHECK(len == static_cast<int32_t>(sl.size() - first), "retained length");
                    std::set<int64_t> view;
                    for (int32_t j = 0; j < len; ++j) view.insert(int64_t{bt[j / bs]} * bs + j % bs);
                    std::set<int64_t> keep(sl.begin() + static_cast<long>(first), sl.end());
                    CHECK(view == keep, "block table reads back the retained slots");
                }
                CHECK(live.size() == live_n, "two live tokens share a slot");
            }
        }
        CHECK(kvq_manager_release(mg, 1000) == KVQ_ERR_INVALID_ARG, "unknown sequence");
        CHECK(kvq_manager_destroy(mg) == KVQ_OK, "manager destroy");
    }
    CHECK(appends > 1000, "too few appends (%ld)", appends);
    std::printf("C planner: %ld plans; manager: %ld appends\n", plans, appends);
}

// ------------------------------------------------------------------ D
uint16_t bf16_bits(Rng& r) {
    // finite BF16 values of every magnitude, both signs, zeros and subnormals
    uint16_t b = static_cast<uint16_t>(r.next());
    if ((b & 0x7F80) == 0x7F80) b &= 0xBFFF;
    return b;
}

void drive_oracle(Rng& r) {
    orc_set_num_threads(2);
    long cases = 0;
    for (int trial = 0; trial < 120; ++trial) {
        const int nl = static_cast<int>(r.in(1, 3));
        const int64_t bs = int64_t{1} << r.in(0, 5), hkv = r.in(1, 4);
        const int64_t hd = r.pick(std::vector<int64_t>{64, 128, 256});
        std::vector<int32_t> modes(nl);
        std::vector<int64_t> nb(nl);
        for (int l = 0; l < nl; ++l) {
            modes[l] = static_cast<int32_t>(r.in(0, 4));
            nb[l] = r.in(0, 6);
        }
        int64_t o[5];
        orc_cache_bytes(nl, bs, hkv, hd, modes.data(), nb.data(), o);
        std::vector<uint8_t> buf(static_cast<size_t>(o[4]) + 1, 0);
        const int layer = static_cast<int>(r.in(0, nl - 1));
        const int64_t nslots = nb[layer] * bs;
        const int64_t n = r.in(0, 40);
        std::vector<uint16_t> k(static_cast<size_t>(n * hkv * hd) + 1), v(k.size());
        for (auto& x : k) x = bf16_bits(r);
        for (auto& x : v) x = bf16_bits(r);
        std::vector<int64_t> slots(static_cast<size_t>(n) + 1);
        std::vector<int64_t> perm(static_cast<size_t>(std::max<int64_t>(nslots, 1)));
        for (int64_t i = 0; i < nslots; ++i) perm[i] = i;
        for (int64_t i = nslots - 1; i > 0; --i) std::swap(perm[i], perm[r.in(0, i)]);
        for (int64_t t = 0; t < n; ++t)
            slots[t] = (t < nslots && r.p(0.9)) ? perm[t] : r.pick(std::vector<int64_t>{-1, -5, nslots, nslots + 9});
        std::vector<float> sc(2 * static_cast<size_t>(hkv));
        for (auto& x : sc) x = r.pick(std::vector<float>{1.0f, 0.013f, 3e38f, 1e-40f, 0.5f});
        const bool stat = modes[layer] == KVQ_FP8_PER_TENSOR || modes[layer] == KVQ_FP8_PER_HEAD;
        orc_store(nl, bs, hkv, hd, modes.data(), nb.data(), buf.data(), layer, k.data(), v.data(), slots.data(), n,
                  stat ? sc.data() : nullptr);
        CHECK(buf.back() == 0, "store wrote past the buffer");
        // gather through a table with bad entries and clamped lengths
        const int64_t ns = r.in(1, 4), maxb = r.in(1, 4);
        std::vector<int32_t> bt(static_cast<size_t>(ns * maxb)), lens(static_cast<size_t>(ns));
        for (auto& e : bt) e = static_cast<int32_t>(r.p(0.85) ? r.in(0, std::max<int64_t>(nb[layer] - 1, 0))
                                                               : r.pick(std::vector<int64_t>{-1, nb[layer], 99}));
        int64_t total = 0;
        for (auto& e : lens) {
            e = static_cast<int32_t>(r.in(-3, maxb * bs + 5));
            total += std::max<int64_t>(0, std::min<int64_t>(e, maxb * bs));
        }
        // the oracle writes sum(max(len, 0)) rows; lengths past the table keep rows unwritten
        int64_t rows = 0;
        for (auto e : lens) rows += std::max<int32_t>(e, 0);
        const size_t row_elems = static_cast<size_t>(hkv * hd);
        std::vector<uint16_t> ok(static_cast<size_t>(rows) * row_elems + 1, 0xABCD), ov(ok.size(), 0xABCD);
        orc_gather(nl, bs, hkv, hd, modes.data(), nb.data(), buf.data(), layer, bt.data(), maxb, lens.data(), ns,
                   ok.data(), ov.data());
        CHECK(ok.back() == 0xABCD && ov.back() == 0xABCD, "gather wrote past its output");
        if (modes[layer] == KVQ_BF16 && n > 0 && nslots > 0) {
            // a BF16 layer returns the stored bits: token t at its slot
            for (int64_t t = 0; t < n; ++t) {
                if (slots[t] < 0 || slots[t] >= nslots) continue;
                std::vector<int32_t> one = {static_cast<int32_t>(slots[t] / bs)};
                int32_t len = static_cast<int32_t>(slots[t] % bs + 1);
                std::vector<uint16_t> rk(static_cast<size_t>(len) * row_elems), rv(rk.size());
                orc_gather(nl, bs, hkv, hd, modes.data(), nb.data(), buf.data(), layer, one.data(), 1, &len, 1,
                           rk.data(), rv.data());
                CHECK(std::memcmp(&rk[(len - 1) * row_elems], &k[t * row_elems], row_elems * 2) == 0 &&
                          std::memcmp(&rv[(len - 1) * row_elems], &v[t * row_elems], row_elems * 2) == 0,
                      "BF16 round trip");
            }
        }
        // calibration and decode attention over the same layer
        std::vector<float> amax(2 * static_cast<size_t>(hkv));
        orc_calibrate_amax(k.data(), v.data(), n, hkv, hd, amax.data(), 0);
        const int64_t H = hkv * r.in(1, 3);
        std::vector<uint16_t> q(static_cast<size_t>(ns * H * hd));
        for (auto& x : q) x = static_cast<uint16_t>(0x3F80 ^ (r.next() & 0x807F));   // values near +-1
        std::vector<double> out(q.size() + 1, -7.0), absv(q.size() + 1, -7.0);
        orc_decode_attention(nl, bs, hkv, hd, modes.data(), nb.data(), buf.data(), layer, q.data(), H, bt.data(), maxb,
                             lens.data(), ns, 0.125, nullptr, out.data(), absv.data());
        CHECK(out.back() == -7.0 && absv.back() == -7.0, "attention wrote past its output");
        for (size_t i = 0; i + 1 < out.size(); ++i)
            CHECK(std::fabs(out[i]) <= absv[i] * (1 + 1e-12) + 1e-300 || std::isnan(out[i]),
                  "|o| <= sum p |V|");
        ++cases;
        (void)total;
    }
    std::printf("D oracle: %ld store/gather/calibration/attention cases\n", cases);
}

}  // namespace

int main() {
    Rng r{0x5EED};
    drive_accounting(r);
    drive_abi(r);
    drive_planner(r);
    drive_oracle(r);
    std::printf("sanitized host drive ok\n");
    return 0;
}
