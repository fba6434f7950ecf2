/*
 * kvq_oracle.c -- plain CPU oracle for the quantized paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, call or
 * link this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library; the two agree only because both follow the same pages.
 *
 * Style: scalar C, one element at a time, in the order the method states.
 * Floating point is evaluated in double and rounded to float exactly where
 * the method stores or defines a float (scales are FP32; the quotient x/s is
 * an FP32 quantity).  Rounding a double quotient or product of two floats to
 * float gives the correctly rounded float result, because a 53-bit
 * intermediate is wide enough for double rounding to be harmless for one
 * division or multiplication of 24-bit operands (Figueroa, "When is double
 * rounding innocuous?", SIGNUM 1995).
 *
 * Sources (the pages' titles and sections):
 *  [P1] "Per-tensor vs per-head FP8 KV cache scales"
 *       - "Per-tensor vs per-head FP8 KV cache scales": the three scale
 *         layouts (one K and one V scale per layer; one per layer and KV head;
 *         one per new K or V vector measured over head_dim).
 *       - "Range sharing explains the accuracy trade": values are mapped
 *         through a scale into E4M3; values beyond the range clip.
 *       - "Static per-head metadata is almost free": static scales are FP32,
 *         2 per layer (per-tensor) or 2 per layer and KV head (per-head).
 *       - "Dynamic per-token-head scales add 3.125 percent": one FP32 K and
 *         one FP32 V scale beside each token-head pair; the store reduces over
 *         each new head vector and writes the scales; attention reads them.
 *  [P2] "Per-token-head KV cache scale overhead"
 *       - "Per-token-head KV cache scale overhead": payload and metadata
 *         formulas per retained token.
 *       - "The FP8 scale tax is 4 divided by head size": a slot holds K data,
 *         a K scale, V data and a V scale, indexed by block, token position
 *         and KV head.
 *       - "INT4 makes the metadata fraction larger": packed INT4 halves the
 *         K and V widths and keeps the two FP32 scales.
 *       - "Convert bytes into block capacity": fixed-size token blocks.
 *  [P3] "FP8 KV cache layer skipping vs per-head scales"
 *       - "Layer skipping follows retained-token footprint": skipped layers
 *         keep BF16 (2 bytes per element); sliding layers retain at most W
 *         positions.
 *
 * Readings where the pages leave a step open (each is a choice, listed with
 * its reason in the design notes):
 *  - FP8 is OCP E4M3FN (bias 7, largest finite 448, no infinities), rounding
 *    to nearest with ties to even, saturating to +-448 instead of NaN.
 *  - Dynamic FP8 scale s = RN32(a / 448), a = max |x| over head_dim.
 *    Dynamic INT4 scale s = RN32(a / 7); codes clamp(rint_even(v), -8, 7),
 *    two's-complement nibbles, even element in the low nibble.
 *  - Quotient v = RN32(x / s), correctly rounded division.
 *  - s == 0 (only when a == 0): FP8 codes are zeros carrying the sign of x,
 *    INT4 nibbles are 0.
 *  - Dequantized value = BF16_RNE(RN32(decode(code) * s)).
 *  - Layout: per layer, block-major; block = codes[bs][Hkv][K,V][row_bytes]
 *    followed (per-token-head modes only) by scales[bs][Hkv][K,V] FP32.
 *    Layer bases are rounded up to 256 bytes; a table of static scales
 *    follows the last layer (per-tensor: [sK, sV]; per-head: [sK[h]..., sV[h]...]).
 *  - slot < 0 or beyond the layer's slots: token not stored.  Gather: tokens
 *    whose block-table entry is out of range, or beyond max_blocks*bs, are
 *    not written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Modes, in the numbering the tests pass in. */
enum {
    ORC_BF16 = 0,                 /* layer skipped: native BF16 [P3] */
    ORC_FP8_PER_TENSOR = 1,       /* one K and one V scale per layer [P1] */
    ORC_FP8_PER_HEAD = 2,         /* one K and one V scale per layer and KV head [P1] */
    ORC_FP8_PER_TOKEN_HEAD = 3,   /* dynamic, per token and KV head [P1][P2] */
    ORC_INT4_PER_TOKEN_HEAD = 4   /* packed INT4, dynamic per token-head [P2] */
};

/* ------------------------------------------------------------------ */
/* Scalar number formats                                               */
/* ------------------------------------------------------------------ */

/* BF16 -> float: the BF16 bits are the high half of the float's bits. */
static float orc_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> BF16, round to nearest, ties to even (finite inputs). */
static uint16_t orc_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* E4M3FN encode of a finite float: nearest representable magnitude, ties to
 * the even code, saturating at 448.  Values are represented as k * quantum,
 * where quantum is the spacing of E4M3 values in m's binade (2^-9 below the
 * smallest normal 2^-6, else 2^(floor(log2 m) - 3)). */
static uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double m = fabs((double)v);
    if (m >= 448.0)
        return sign | 0x7E;                 /* largest finite: E=15, f=6 */
    double quantum;
    if (m < 0x1p-6) {
        quantum = 0x1p-9;                   /* subnormal spacing */
    } else {
        int e;
        frexp(m, &e);                       /* m = fr * 2^e, fr in [0.5, 1) */
        quantum = ldexp(1.0, (e - 1) - 3);  /* 3 fraction bits */
    }
    double k = nearbyint(m / quantum);      /* default mode: ties to even */
    double r = k * quantum;                 /* rounded magnitude, exact */
    if (r == 0.0)
        return sign;
    if (r < 0x1p-6)
        return sign | (uint8_t)k;           /* subnormal: E=0, f=k */
    int e;
    frexp(r, &e);
    int E = (e - 1) + 7;                    /* biased exponent */
    double frac = r / ldexp(1.0, e - 1) - 1.0;
    int f = (int)(frac * 8.0);
    return sign | (uint8_t)((E << 3) | f);
}

/* E4M3FN decode: (-1)^S * (E == 0 ? f * 2^-9 : (1 + f/8) * 2^(E-7)).
 * The NaN codes (S.1111.111) are never produced by the encoder. */
static float orc_e4m3_decode(uint8_t c)
{
    int S = c >> 7, E = (c >> 3) & 0xF, f = c & 7;
    double mag = (E == 0) ? ldexp((double)f, -9)
                          : ldexp(1.0 + f / 8.0, E - 7);
    return (float)(S ? -mag : mag);
}

/* INT4 encode: clamp(rint_even(v), -8, 7). */
static int orc_int4_encode(float v)
{
    double r = nearbyint((double)v);
    if (r < -8.0) r = -8.0;
    if (r > 7.0) r = 7.0;
    return (int)r;
}

/* INT4 decode of a nibble: two's complement sign extension. */
static int orc_int4_decode(unsigned nib)
{
    nib &= 0xF;
    return (nib & 0x8) ? (int)nib - 16 : (int)nib;
}

/* RN32(x / s). */
static float orc_quotient(float x, float s)
{
    return (float)((double)x / (double)s);
}

/* RN32(a / qmax): the dynamic scale. */
static float orc_dynamic_scale(float a, double qmax)
{
    return (float)((double)a / qmax);
}

/* BF16_RNE(RN32(decoded * s)). */
static uint16_t orc_dequant(double decoded, float s)
{
    float p = (float)(decoded * (double)s);
    return orc_float_to_bf16(p);
}

/* ------------------------------------------------------------------ */
/* Layout                                                              */
/* ------------------------------------------------------------------ */

/* Bytes of one K (or V) row of head_dim elements in a layer of this mode. */
static int64_t orc_row_bytes(int mode, int64_t hd)
{
    switch (mode) {
    case ORC_BF16: return 2 * hd;
    case ORC_INT4_PER_TOKEN_HEAD: return hd / 2;
    default: return hd;                     /* FP8: one byte per element */
    }
}

static int orc_has_token_scales(int mode)
{
    return mode == ORC_FP8_PER_TOKEN_HEAD || mode == ORC_INT4_PER_TOKEN_HEAD;
}

static int64_t orc_block_code_bytes(int mode, int64_t bs, int64_t hkv, int64_t hd)
{
    return bs * hkv * 2 * orc_row_bytes(mode, hd);
}

static int64_t orc_block_bytes(int mode, int64_t bs, int64_t hkv, int64_t hd)
{
    int64_t b = orc_block_code_bytes(mode, bs, hkv, hd);
    if (orc_has_token_scales(mode))
        b += bs * hkv * 2 * 4;
    return b;
}

static int64_t orc_static_bytes(int mode, int64_t hkv)
{
    if (mode == ORC_FP8_PER_TENSOR) return 2 * 4;
    if (mode == ORC_FP8_PER_HEAD) return 2 * hkv * 4;
    return 0;
}

static int64_t orc_round_up_256(int64_t x)
{
    return (x + 255) / 256 * 256;
}

/* Byte offsets of each layer's block region and static-scale entry.
 * layer_base and static_base may be NULL.  Returns the total size. */
static int64_t orc_layout(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
                          const int32_t* modes, const int64_t* nblocks,
                          int64_t* layer_base, int64_t* static_base)
{
    int64_t off = 0;
    for (int l = 0; l < num_layers; ++l) {
        off = orc_round_up_256(off);
        if (layer_base) layer_base[l] = off;
        off += nblocks[l] * orc_block_bytes(modes[l], bs, hkv, hd);
    }
    off = orc_round_up_256(off);
    for (int l = 0; l < num_layers; ++l) {
        if (static_base) static_base[l] = off;
        off += orc_static_bytes(modes[l], hkv);
    }
    return off;
}

/* out[0..4] = payload, token_scales, static_scales, padding, total. */
void orc_cache_bytes(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
                     const int32_t* modes, const int64_t* nblocks, int64_t* out)
{
    int64_t payload = 0, tok = 0, stat = 0;
    for (int l = 0; l < num_layers; ++l) {
        payload += nblocks[l] * orc_block_code_bytes(modes[l], bs, hkv, hd);
        if (orc_has_token_scales(modes[l]))
            tok += nblocks[l] * bs * hkv * 2 * 4;
        stat += orc_static_bytes(modes[l], hkv);
    }
    int64_t total = orc_layout(num_layers, bs, hkv, hd, modes, nblocks, NULL, NULL);
    out[0] = payload;
    out[1] = tok;
    out[2] = stat;
    out[3] = total - payload - tok - stat;
    out[4] = total;
}

/* Offsets exposed for tests (layer_base[num_layers], static_base[num_layers]). */
int64_t orc_layer_offsets(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
                          const int32_t* modes, const int64_t* nblocks,
                          int64_t* layer_base, int64_t* static_base)
{
    return orc_layout(num_layers, bs, hkv, hd, modes, nblocks, layer_base, static_base);
}

/* ------------------------------------------------------------------ */
/* Quantize-and-store                                                  */
/* ------------------------------------------------------------------ */

/* Encode one row of head_dim BF16 values with scale s into dst. */
static void orc_encode_row(int mode, const uint16_t* x, int64_t hd, float s, uint8_t* dst)
{
    if (mode == ORC_BF16) {
        for (int64_t i = 0; i < hd; ++i) {      /* little-endian BF16 bits */
            dst[2 * i] = (uint8_t)(x[i] & 0xFF);
            dst[2 * i + 1] = (uint8_t)(x[i] >> 8);
        }
        return;
    }
    if (mode == ORC_INT4_PER_TOKEN_HEAD) {
        for (int64_t j = 0; j < hd / 2; ++j) {
            int n0 = 0, n1 = 0;
            if (s != 0.0f) {
                n0 = orc_int4_encode(orc_quotient(orc_bf16_to_float(x[2 * j]), s));
                n1 = orc_int4_encode(orc_quotient(orc_bf16_to_float(x[2 * j + 1]), s));
            }
            dst[j] = (uint8_t)((n0 & 0xF) | ((n1 & 0xF) << 4));
        }
        return;
    }
    for (int64_t i = 0; i < hd; ++i) {          /* FP8 E4M3 modes */
        float xi = orc_bf16_to_float(x[i]);
        if (s == 0.0f)
            dst[i] = signbit(xi) ? 0x80 : 0x00;
        else
            dst[i] = orc_e4m3_encode(orc_quotient(xi, s));
    }
}

static void orc_put_f32(uint8_t* dst, float v)
{
    memcpy(dst, &v, 4);                         /* little-endian host */
}

static float orc_get_f32(const uint8_t* src)
{
    float v;
    memcpy(&v, src, 4);
    return v;
}

/*
 * Store num_tokens new K/V vectors of one layer into the cache image `buf`.
 * keys, values: BF16 bits [num_tokens][hkv][hd].  slot_mapping[t]: slot of
 * token t (block = slot / bs, position = slot % bs).  scales: per-tensor
 * [sK, sV]; per-head [sK[0..hkv), sV[0..hkv)]; NULL otherwise.
 */
void orc_store(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
               const int32_t* modes, const int64_t* nblocks,
               uint8_t* buf, int layer,
               const uint16_t* keys, const uint16_t* values,
               const int64_t* slot_mapping, int64_t num_tokens,
               const float* scales)
{
    int64_t layer_base[num_layers > 0 ? num_layers : 1];
    int64_t static_base[num_layers > 0 ? num_layers : 1];
    orc_layout(num_layers, bs, hkv, hd, modes, nblocks, layer_base, static_base);
    const int mode = modes[layer];
    const int64_t rb = orc_row_bytes(mode, hd);
    const int64_t code_bytes = orc_block_code_bytes(mode, bs, hkv, hd);
    const int64_t blk_bytes = orc_block_bytes(mode, bs, hkv, hd);
    const int64_t nslots = nblocks[layer] * bs;
    uint8_t* base = buf + layer_base[layer];

    /* Static layouts keep their scales in the table after the layers. */
    if (mode == ORC_FP8_PER_TENSOR) {
        orc_put_f32(buf + static_base[layer], scales[0]);
        orc_put_f32(buf + static_base[layer] + 4, scales[1]);
    } else if (mode == ORC_FP8_PER_HEAD) {
        for (int64_t i = 0; i < 2 * hkv; ++i)
            orc_put_f32(buf + static_base[layer] + 4 * i, scales[i]);
    }

    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= nslots)
            continue;
        int64_t blk = slot / bs, pos = slot % bs;
        uint8_t* block = base + blk * blk_bytes;
        for (int64_t h = 0; h < hkv; ++h) {
            for (int kv = 0; kv < 2; ++kv) {
                const uint16_t* x = (kv == 0 ? keys : values) + (t * hkv + h) * hd;
                float s = 0.0f;
                if (mode == ORC_FP8_PER_TOKEN_HEAD || mode == ORC_INT4_PER_TOKEN_HEAD) {
                    float a = 0.0f;             /* absmax over head_dim */
                    for (int64_t i = 0; i < hd; ++i) {
                        float m = fabsf(orc_bf16_to_float(x[i]));
                        if (m > a) a = m;
                    }
                    s = orc_dynamic_scale(a, mode == ORC_FP8_PER_TOKEN_HEAD ? 448.0 : 7.0);
                    orc_put_f32(block + code_bytes + ((pos * hkv + h) * 2 + kv) * 4, s);
                } else if (mode == ORC_FP8_PER_TENSOR) {
                    s = scales[kv];
                } else if (mode == ORC_FP8_PER_HEAD) {
                    s = scales[kv * hkv + h];
                }
                uint8_t* dst = block + ((pos * hkv + h) * 2 + kv) * rb;
                orc_encode_row(mode, x, hd, s, dst);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Gather and dequantize                                               */
/* ------------------------------------------------------------------ */

/*
 * For each sequence b and t < seq_lens[b]: physical block
 * block_table[b][t / bs], position t % bs.  Output rows are packed in
 * sequence order: row (sum_{i<b} seq_lens[i]) + t of out_keys / out_values,
 * each [hkv][hd] BF16 bits.
 */
void orc_gather(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
                const int32_t* modes, const int64_t* nblocks,
                const uint8_t* buf, int layer,
                const int32_t* block_table, int64_t max_blocks,
                const int32_t* seq_lens, int64_t num_seqs,
                uint16_t* out_keys, uint16_t* out_values)
{
    int64_t layer_base[num_layers > 0 ? num_layers : 1];
    int64_t static_base[num_layers > 0 ? num_layers : 1];
    orc_layout(num_layers, bs, hkv, hd, modes, nblocks, layer_base, static_base);
    const int mode = modes[layer];
    const int64_t rb = orc_row_bytes(mode, hd);
    const int64_t code_bytes = orc_block_code_bytes(mode, bs, hkv, hd);
    const int64_t blk_bytes = orc_block_bytes(mode, bs, hkv, hd);
    const uint8_t* base = buf + layer_base[layer];

    int64_t offset = 0;
    for (int64_t b = 0; b < num_seqs; ++b) {
        int64_t len = seq_lens[b] > 0 ? seq_lens[b] : 0;
        #pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < len; ++t) {
            if (t / bs >= max_blocks)
                continue;
            int64_t blk = block_table[b * max_blocks + t / bs];
            if (blk < 0 || blk >= nblocks[layer])
                continue;
            int64_t pos = t % bs;
            const uint8_t* block = base + blk * blk_bytes;
            for (int64_t h = 0; h < hkv; ++h) {
                for (int kv = 0; kv < 2; ++kv) {
                    const uint8_t* src = block + ((pos * hkv + h) * 2 + kv) * rb;
                    uint16_t* out = (kv == 0 ? out_keys : out_values) + ((offset + t) * hkv + h) * hd;
                    float s = 0.0f;
                    if (orc_has_token_scales(mode))
                        s = orc_get_f32(block + code_bytes + ((pos * hkv + h) * 2 + kv) * 4);
                    else if (mode == ORC_FP8_PER_TENSOR)
                        s = orc_get_f32(buf + static_base[layer] + 4 * kv);
                    else if (mode == ORC_FP8_PER_HEAD)
                        s = orc_get_f32(buf + static_base[layer] + 4 * (kv * hkv + h));
                    for (int64_t i = 0; i < hd; ++i) {
                        if (mode == ORC_BF16) {
                            out[i] = (uint16_t)(src[2 * i] | (src[2 * i + 1] << 8));
                        } else if (mode == ORC_INT4_PER_TOKEN_HEAD) {
                            unsigned byte = src[i / 2];
                            unsigned nib = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                            out[i] = orc_dequant((double)orc_int4_decode(nib), s);
                        } else {
                            out[i] = orc_dequant((double)orc_e4m3_decode(src[i]), s);
                        }
                    }
                }
            }
        }
        offset += len;
    }
}

/* ------------------------------------------------------------------ */
/* Calibration                                                         */
/* ------------------------------------------------------------------ */

/*
 * On-the-fly calibration ("Per-tensor vs per-head FP8 KV cache scales",
 * "Calibration changes which scale layout exists": static scales estimated
 * during warmup; "Per-token-head KV cache scale overhead", "Static per-head
 * calibration pays once": they must cover every value seen).  out[kv * hkv + h]
 * = max(out[...], max |x| over the batch's tokens and head_dim) for K (kv = 0)
 * and V (kv = 1); out starts at 0 unless accumulate.
 */
void orc_calibrate_amax(const uint16_t* keys, const uint16_t* values, int64_t num_tokens,
                        int64_t hkv, int64_t hd, float* out, int accumulate)
{
    if (!accumulate)
        for (int64_t i = 0; i < 2 * hkv; ++i) out[i] = 0.0f;
    for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* x = kv == 0 ? keys : values;
        for (int64_t h = 0; h < hkv; ++h) {
            float m = out[kv * hkv + h];
            for (int64_t t = 0; t < num_tokens; ++t)
                for (int64_t i = 0; i < hd; ++i) {
                    float a = fabsf(orc_bf16_to_float(x[(t * hkv + h) * hd + i]));
                    if (a > m) m = a;
                }
            out[kv * hkv + h] = m;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Decode attention over the quantized cache                           */
/* ------------------------------------------------------------------ */

/* Dequantized value of element i of the K (kv = 0) or V (kv = 1) row of
 * (block, position, head), exact in double: decode(code) * s. */
static double orc_cached_value(int mode, const uint8_t* buf, int64_t layer_base, int64_t static_base,
                               int64_t bs, int64_t hkv, int64_t hd, int64_t blk, int64_t pos,
                               int64_t h, int kv, int64_t i)
{
    const int64_t rb = orc_row_bytes(mode, hd);
    const uint8_t* block = buf + layer_base + blk * orc_block_bytes(mode, bs, hkv, hd);
    const uint8_t* src = block + ((pos * hkv + h) * 2 + kv) * rb;
    if (mode == ORC_BF16)
        return (double)orc_bf16_to_float((uint16_t)(src[2 * i] | (src[2 * i + 1] << 8)));
    double s;
    if (orc_has_token_scales(mode))
        s = (double)orc_get_f32(block + orc_block_code_bytes(mode, bs, hkv, hd) + ((pos * hkv + h) * 2 + kv) * 4);
    else if (mode == ORC_FP8_PER_TENSOR)
        s = (double)orc_get_f32(buf + static_base + 4 * kv);
    else
        s = (double)orc_get_f32(buf + static_base + 4 * (kv * hkv + h));
    if (mode == ORC_INT4_PER_TOKEN_HEAD) {
        unsigned byte = src[i / 2];
        return (double)orc_int4_decode((i % 2 == 0) ? (byte & 0xF) : (byte >> 4)) * s;
    }
    return (double)orc_e4m3_decode(src[i]) * s;
}

/* A query element as attention uses it: the BF16 value itself, or, with a
 * static FP8 query scale sq > 0 (one per query head, "FP8 KV cache layer
 * skipping vs per-head scales", "Per-head scales have fixed overhead"), its
 * E4M3 code under that scale decoded back, exactly: decode(E4M3(RN32(q/sq)))
 * times sq, the same encoding the cache applies to K and V. */
static double orc_query_value(uint16_t qb, float sq)
{
    float x = orc_bf16_to_float(qb);
    if (sq == 0.0f)
        return (double)x;
    return (double)orc_e4m3_decode(orc_e4m3_encode(orc_quotient(x, sq))) * (double)sq;
}

/*
 * Attention of one new query token per sequence over the sequence's cached
 * tokens, read through the block table ("Per-tensor vs per-head FP8 KV cache
 * scales", "Dynamic per-token-head scales add 3.125 percent": the scales are
 * read during attention).  Query head qh attends with KV head qh / (H / hkv):
 *   score_t = sm_scale * sum_d q[b][qh][d] * K^[t][d],  p = softmax(score),
 *   out[b][qh][d] = sum_t p_t * V^[t][d],
 * with K^, V^ the dequantized cache values, all in double.  q: BF16 bits
 * [num_seqs][H][hd]; q_scales: NULL (BF16 queries) or [H] positive static
 * FP8 query scales; out: double [num_seqs][H][hd].  Lengths are clamped to
 * [0, max_blocks * bs]; a token whose block-table entry does not name a block
 * of the layer takes no part (no score, no weight), and a sequence with no
 * token left gives zeros.  Also returns sum_t p_t |V^[t][d]| in out_absv (for error
 * bounds), when out_absv is not NULL.
 */
void orc_decode_attention(int num_layers, int64_t bs, int64_t hkv, int64_t hd,
                          const int32_t* modes, const int64_t* nblocks,
                          const uint8_t* buf, int layer, const uint16_t* q, int64_t num_q_heads,
                          const int32_t* block_table, int64_t max_blocks,
                          const int32_t* seq_lens, int64_t num_seqs, double sm_scale,
                          const float* q_scales, double* out, double* out_absv)
{
    int64_t layer_base[num_layers > 0 ? num_layers : 1];
    int64_t static_base[num_layers > 0 ? num_layers : 1];
    orc_layout(num_layers, bs, hkv, hd, modes, nblocks, layer_base, static_base);
    const int mode = modes[layer];
    const int64_t group = num_q_heads / hkv;

    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t b = 0; b < num_seqs; ++b) {
        for (int64_t qh = 0; qh < num_q_heads; ++qh) {
            const int64_t h = qh / group;
            int64_t len = seq_lens[b] > 0 ? seq_lens[b] : 0;
            if (len > max_blocks * bs) len = max_blocks * bs;
            double* o = out + (b * num_q_heads + qh) * hd;
            double* oa = out_absv ? out_absv + (b * num_q_heads + qh) * hd : NULL;
            for (int64_t i = 0; i < hd; ++i) { o[i] = 0.0; if (oa) oa[i] = 0.0; }
            if (len == 0)
                continue;
            double* score = (double*)malloc(sizeof(double) * (size_t)len);
            double m = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                int64_t blk = block_table[b * max_blocks + t / bs], pos = t % bs;
                if (blk < 0 || blk >= nblocks[layer]) {
                    score[t] = -INFINITY;
                    continue;
                }
                double acc = 0.0;
                for (int64_t i = 0; i < hd; ++i)
                    acc += orc_query_value(q[(b * num_q_heads + qh) * hd + i], q_scales ? q_scales[qh] : 0.0f) *
                           orc_cached_value(mode, buf, layer_base[layer], static_base[layer], bs, hkv, hd,
                                            blk, pos, h, 0, i);
                score[t] = acc * sm_scale;
                if (score[t] > m) m = score[t];
            }
            if (m == -INFINITY) {           /* no token of this sequence is in the layer */
                free(score);
                continue;
            }
            double l = 0.0;
            for (int64_t t = 0; t < len; ++t) {
                score[t] = exp(score[t] - m);
                l += score[t];
            }
            for (int64_t t = 0; t < len; ++t) {
                int64_t blk = block_table[b * max_blocks + t / bs], pos = t % bs;
                if (blk < 0 || blk >= nblocks[layer])
                    continue;
                double p = score[t] / l;
                for (int64_t i = 0; i < hd; ++i) {
                    double v = orc_cached_value(mode, buf, layer_base[layer], static_base[layer], bs, hkv, hd,
                                                blk, pos, h, 1, i);
                    o[i] += p * v;
                    if (oa) oa[i] += p * fabs(v);
                }
            }
            free(score);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Element-wise entry points for the pins                              */
/* ------------------------------------------------------------------ */

void orc_e4m3_encode_n(const float* v, uint8_t* out, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_decode_n(const uint8_t* c, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

void orc_int4_encode_n(const float* v, int8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)orc_int4_encode(v[i]);
}

void orc_quotient_n(const float* x, const float* s, float* out, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_quotient(x[i], s[i]);
}

void orc_dynamic_scale_n(const float* a, double qmax, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dynamic_scale(a[i], qmax);
}

void orc_float_to_bf16_n(const float* v, uint16_t* out, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_bf16(v[i]);
}

void orc_dequant_fp8_n(const uint8_t* c, const float* s, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dequant((double)orc_e4m3_decode(c[i]), s[i]);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the oracle's parallel loops from here on (timing only). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}
