/* A plain C99 program on the GPU path: HIP runtime C API for memory, the
 * library's C ABI for the work.  It stores 100 tokens (2 KV heads, head_dim
 * 64) into a per-token-head FP8 layer and a per-token-head INT4 layer
 * through a permuted block table, gathers them back and checks the BF16
 * output bit for bit against the input.  The inputs are chosen so that the
 * round trip is exact by construction: every row is an E4M3 value (or an
 * integer in [-7, 7]) times 2^e with its absmax at 448 * 2^e (7 * 2^e), so
 * its scale is exactly 2^e, every quotient is exactly representable and
 * decoding gives the input back (INT4 zeros are +0: a zero nibble carries
 * no sign).  Prints "c-abi device ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvq.h"

#define HKV 2
#define HD 64
#define BS 16
#define NBLK 8
#define NTOK 100
#define NELEM (NTOK * HKV * HD)

static uint16_t bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16); /* every input here is exactly a BF16 value */
}

static float pow2(int e) {
    float r = 1.0f;
    while (e > 0) { r *= 2.0f; --e; }
    while (e < 0) { r *= 0.5f; ++e; }
    return r;
}

/* E4M3 magnitudes: zero, subnormal (2^-9), normal, the top code */
static const float kFp8[] = {0.0f, 0.001953125f, 0.015625f, 0.25f, 1.0f, 1.5f, 3.5f, 2.0f, 240.0f, 448.0f};

static void make_rows(int int4, uint16_t* k, uint16_t* v) {
    int t, h, d, kv;
    for (kv = 0; kv < 2; ++kv) {
        uint16_t* out = kv ? v : k;
        for (t = 0; t < NTOK; ++t)
            for (h = 0; h < HKV; ++h) {
                const int e = (t + 3 * h + 5 * kv) % 9 - 4;
                const float s = pow2(e);
                for (d = 0; d < HD; ++d) {
                    float x;
                    const float sign = ((t + d + kv) % 3 == 0) ? -1.0f : 1.0f;
                    if (d == 0)
                        x = int4 ? 7.0f : 448.0f;
                    else if (int4)
                        x = (float)((t * 7 + d * 3 + h + kv) % 8); /* 0..7 */
                    else
                        x = kFp8[(t * 7 + d * 3 + h + kv) % 10];
                    /* INT4 keeps no sign on a zero code, so its zeros are +0 */
                    out[(t * HKV + h) * HD + d] = bf16_bits((int4 && x == 0.0f) ? 0.0f : sign * x * s);
                }
            }
    }
}

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));  \
            return 1;                                                           \
        }                                                                       \
    } while (0)

int main(void) {
    static uint16_t hk[NELEM], hv[NELEM], ok[NELEM], ov[NELEM];
    const int32_t modes[2] = {KVQ_FP8_PER_TOKEN_HEAD, KVQ_INT4_PER_TOKEN_HEAD};
    const int64_t nblocks[2] = {NBLK, NBLK};
    const int32_t table[NBLK] = {5, 2, 7, 0, 3, 6, 1, 4};
    const int32_t len = NTOK;
    int64_t slots[NTOK];
    int32_t order[NTOK];
    kvq_cache_config cfg;
    kvq_bytes bytes;
    kvq_cache* cache = NULL;
    void *dcache, *dk, *dv, *dok, *dov, *dslots, *dorder, *dtable, *dlen;
    int layer, t, bad = 0;

    cfg.num_layers = 2;
    cfg.block_size = BS;
    cfg.num_kv_heads = HKV;
    cfg.head_dim = HD;
    cfg.layer_mode = modes;
    cfg.layer_num_blocks = nblocks;
    if (kvq_cache_bytes(&cfg, &bytes) != KVQ_OK) { fprintf(stderr, "cache_bytes\n"); return 1; }
    for (t = 0; t < NTOK; ++t) slots[t] = (int64_t)table[t / BS] * BS + t % BS; /* t / BS <= 6 */

    HIP_OK(hipSetDevice(0));
    HIP_OK(hipMalloc(&dcache, bytes.total));
    HIP_OK(hipMalloc(&dk, sizeof hk));
    HIP_OK(hipMalloc(&dv, sizeof hv));
    HIP_OK(hipMalloc(&dok, sizeof ok));
    HIP_OK(hipMalloc(&dov, sizeof ov));
    HIP_OK(hipMalloc(&dslots, sizeof slots));
    HIP_OK(hipMalloc(&dorder, sizeof order));
    /* layer 1 goes through kvq_store_ordered (last token first; head_dim 64 keeps
     * token order, with the same contents) */
    for (t = 0; t < NTOK; ++t) order[t] = NTOK - 1 - t;
    HIP_OK(hipMemcpy(dorder, order, sizeof order, hipMemcpyHostToDevice));
    HIP_OK(hipMalloc(&dtable, sizeof table));
    HIP_OK(hipMalloc(&dlen, sizeof len));
    HIP_OK(hipMemcpy(dslots, slots, sizeof slots, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dtable, table, sizeof table, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dlen, &len, sizeof len, hipMemcpyHostToDevice));
    if (kvq_create_cache(&cfg, dcache, bytes.total, &cache) != KVQ_OK) { fprintf(stderr, "create\n"); return 1; }

    for (layer = 0; layer < 2; ++layer) {
        int i;
        make_rows(layer == 1, hk, hv);
        HIP_OK(hipMemcpy(dk, hk, sizeof hk, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dv, hv, sizeof hv, hipMemcpyHostToDevice));
        const kvq_status sst =
            layer == 0 ? kvq_store(cache, layer, dk, dv, (const int64_t*)dslots, NTOK, (kvq_mode)modes[layer], NULL,
                                   NULL)
                       : kvq_store_ordered(cache, layer, dk, dv, (const int64_t*)dslots, (const int32_t*)dorder, NTOK,
                                           (kvq_mode)modes[layer], NULL, NULL);
        if (sst != KVQ_OK ||
            kvq_gather_dequant(cache, layer, (const int32_t*)dtable, NBLK, (const int32_t*)dlen, 1, dok, dov,
                               NTOK, NULL) != KVQ_OK) {
            fprintf(stderr, "store/gather of layer %d\n", layer);
            return 1;
        }
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(ok, dok, sizeof ok, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ov, dov, sizeof ov, hipMemcpyDeviceToHost));
        for (i = 0; i < NELEM; ++i)
            if (ok[i] != hk[i] || ov[i] != hv[i]) {
                if (bad < 5)
                    fprintf(stderr, "layer %d element %d: K %04x/%04x V %04x/%04x\n", layer, i, ok[i], hk[i],
                            ov[i], hv[i]);
                ++bad;
            }
    }
    kvq_destroy_cache(cache);
    HIP_OK(hipFree(dcache));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dok));
    HIP_OK(hipFree(dov));
    HIP_OK(hipFree(dslots));
    HIP_OK(hipFree(dorder));
    HIP_OK(hipFree(dtable));
    HIP_OK(hipFree(dlen));
    if (bad) {
        fprintf(stderr, "%d elements differ\n", bad);
        return 1;
    }
    printf("c-abi device ok\n");
    return 0;
}
