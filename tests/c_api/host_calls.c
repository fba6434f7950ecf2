/* A plain C99 caller of the library's host-only entry points: it includes
 * include/kvq.h, links libkvq.so and checks byte counts the pages print,
 * the static-scale arithmetic and argument errors.  No call here touches a
 * device, so it runs without a GPU.  Prints "c-abi ok" on success. */
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int failures = 0;

#define CHECK(cond, msg)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAILED: %s\n", msg);          \
            ++failures;                                    \
        }                                                  \
    } while (0)

static kvq_cache_config geometry(int32_t layers, int32_t mode, int64_t blocks, int32_t* modes,
                                 int64_t* nblocks) {
    kvq_cache_config c;
    int32_t l;
    for (l = 0; l < layers; ++l) {
        modes[l] = mode;
        nblocks[l] = blocks;
    }
    c.num_layers = layers;
    c.block_size = 16;
    c.num_kv_heads = 8;
    c.head_dim = 128;
    c.layer_mode = modes;
    c.layer_num_blocks = nblocks;
    return c;
}

int main(void) {
    int32_t modes[80];
    int64_t nblocks[80];
    kvq_bytes b;
    kvq_cache_config cfg;
    kvq_cache* c = NULL;
    float amax[16], scales[16];
    uint32_t bits;
    int i;

    /* 80 layers x 8 KV heads x head_dim 128 at 131072 tokens ("Per-tensor vs
     * per-head FP8 KV cache scales"): 20 GiB of FP8 codes, 640 MiB of
     * per-token-head scales, 20.625 GiB in all. */
    cfg = geometry(80, KVQ_FP8_PER_TOKEN_HEAD, 8192, modes, nblocks);
    CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_OK, "cache_bytes 80 layers");
    CHECK(b.payload == 21474836480ull, "20 GiB payload");
    CHECK(b.token_scales == 671088640ull, "640 MiB of scales");
    CHECK(b.static_scales == 0 && b.padding == 0, "no static scales, no padding");
    CHECK(b.total == 22145925120ull, "20.625 GiB total");

    /* the same model with static scales: 640 B per-tensor, 5120 B per-head */
    cfg = geometry(80, KVQ_FP8_PER_TENSOR, 8192, modes, nblocks);
    CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_OK && b.static_scales == 640, "per-tensor 640 B");
    cfg = geometry(80, KVQ_FP8_PER_HEAD, 8192, modes, nblocks);
    CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_OK && b.static_scales == 5120, "per-head 5120 B");

    /* 32 layers x 8 x 128 ("Per-token-head KV cache scale overhead"): 66 KiB per
     * token, 1056 KiB per 16-token block */
    cfg = geometry(32, KVQ_FP8_PER_TOKEN_HEAD, 1, modes, nblocks);
    CHECK(kvq_cache_bytes(&cfg, &b) == KVQ_OK, "cache_bytes 32 layers");
    CHECK(b.payload + b.token_scales == 1056ull * 1024, "1056 KiB per block");

    /* argument errors, found before any device call */
    cfg = geometry(32, KVQ_FP8_PER_TOKEN_HEAD, 2048, modes, nblocks);
    CHECK(kvq_cache_bytes(&cfg, NULL) == KVQ_ERR_INVALID_ARG, "null out");
    cfg.head_dim = 96;
    CHECK(kvq_cache_bytes(&cfg, &b) != KVQ_OK, "head_dim 96 rejected");
    cfg.head_dim = 128;
    CHECK(kvq_create_cache(&cfg, NULL, 1ull << 30, &c) == KVQ_ERR_INVALID_ARG, "null device buffer");
    CHECK(kvq_create_cache(&cfg, (void*)(uintptr_t)0x100000, 1024, &c) == KVQ_ERR_BUFFER_TOO_SMALL,
          "buffer too small");
    CHECK(kvq_store(NULL, 0, NULL, NULL, NULL, 1, KVQ_FP8_PER_TOKEN_HEAD, NULL, NULL) == KVQ_ERR_INVALID_ARG,
          "store without a cache");
    CHECK(kvq_store_ordered(NULL, 0, NULL, NULL, NULL, NULL, 1, KVQ_FP8_PER_TOKEN_HEAD, NULL, NULL) ==
              KVQ_ERR_INVALID_ARG,
          "ordered store without a cache");
    CHECK(kvq_status_string(KVQ_ERR_HIP) != NULL && strlen(kvq_status_string(KVQ_ERR_HIP)) > 0, "status string");

    /* static scales: RN32(amax / 448); a zero maximum gives the smallest
     * positive FP32 value */
    for (i = 0; i < 16; ++i) amax[i] = 0.0f;
    amax[0] = 896.0f;
    amax[8] = 44.8f;
    CHECK(kvq_static_scales(amax, 8, KVQ_FP8_PER_HEAD, scales) == KVQ_OK, "static scales");
    CHECK(scales[0] == 2.0f, "896 / 448 = 2");
    CHECK(scales[8] == 44.8f / 448.0f, "44.8 / 448 in FP32");
    memcpy(&bits, &scales[1], sizeof bits);
    CHECK(bits == 1u, "zero maximum -> smallest positive FP32");
    CHECK(kvq_static_scales(amax, 8, KVQ_FP8_PER_TENSOR, scales) == KVQ_OK && scales[0] == 2.0f &&
              scales[1] == 44.8f / 448.0f,
          "per-tensor scales take the maximum over heads");

    if (failures) return 1;
    printf("c-abi ok\n");
    return 0;
}
