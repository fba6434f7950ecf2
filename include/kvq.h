/*
 * kvq.h -- C ABI of the MI355X (gfx950) quantized paged KV cache.
 *
 * The library quantizes new attention K/V vectors into a paged KV cache and
 * dequantizes them back on read, under the scale layouts described on the
 * pages "Per-tensor vs per-head FP8 KV cache scales" and "Per-token-head KV
 * cache scale overhead", with BF16 layers for layer skipping as on "FP8 KV
 * cache layer skipping vs per-head scales".
 *
 * Conventions for every entry point:
 *  - Plain pointers and sizes only.  "Device" pointers are HIP device memory
 *    of the current device; "host" pointers are ordinary CPU memory.
 *  - The caller allocates and owns all device memory (cache buffer, inputs,
 *    outputs).  The library allocates only the host-side handle and never
 *    synchronizes a stream.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and completes asynchronously.
 *  - Every argument check happens before the first HIP call; on a
 *    host-detected error nothing is enqueued and nothing is written.
 *  - Return value 0 is success; negative values are kvq_status errors.
 *
 * Numerics (identical, bit for bit, to the CPU oracle that the tests use):
 *  - FP8 is OCP E4M3FN (bias 7, largest finite 448), round to nearest even,
 *    saturating at +-448.  Quotients are correctly rounded FP32 x / s.
 *  - Dynamic FP8 scale s = RN32(absmax / 448); dynamic INT4 scale
 *    s = RN32(absmax / 7), codes clamp(rint_even(x / s), -8, 7) as
 *    two's-complement nibbles, even element in the low nibble.
 *  - An all-zero vector stores s = 0 and zero codes (FP8 zeros keep the sign
 *    of the input).
 *  - Dequantized value = BF16_RNE(RN32(decode(code) * s)); BF16 layers are
 *    copied bit for bit.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#if defined(__GNUC__)
#define KVQ_API __attribute__((visibility("default")))
#else
#define KVQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,      /* null pointer, out-of-range value, bad scale */
    KVQ_ERR_MODE_MISMATCH = -2,    /* kvq_store mode differs from the layer's mode */
    KVQ_ERR_BUFFER_TOO_SMALL = -3, /* cache buffer smaller than kvq_cache_bytes().total */
    KVQ_ERR_UNSUPPORTED = -4,      /* geometry outside what the kernels handle */
    KVQ_ERR_HIP = -5,              /* a HIP launch or runtime call failed */
    KVQ_ERR_NO_SPACE = -6          /* kvq_manager_append: no free block left */
} kvq_status;

/* Per-layer cache mode ("Per-tensor vs per-head FP8 KV cache scales",
 * section "Per-tensor vs per-head FP8 KV cache scales"; BF16 skip from "FP8
 * KV cache layer skipping vs per-head scales", "Layer skipping follows
 * retained-token footprint"; INT4 from "Per-token-head KV cache scale
 * overhead", "INT4 makes the metadata fraction larger"). */
typedef enum kvq_mode {
    KVQ_BF16 = 0,                /* layer kept in BF16 (skipped), 2 B per element */
    KVQ_FP8_PER_TENSOR = 1,      /* one K and one V FP32 scale per layer */
    KVQ_FP8_PER_HEAD = 2,        /* one K and one V FP32 scale per layer and KV head */
    KVQ_FP8_PER_TOKEN_HEAD = 3,  /* FP32 K and V scales beside every token-head slot */
    KVQ_INT4_PER_TOKEN_HEAD = 4  /* packed INT4 codes, same two FP32 scales per slot */
} kvq_mode;

/* Largest num_kv_heads a KVQ_FP8_PER_HEAD layer accepts. */
#define KVQ_MAX_STATIC_KV_HEADS 256

/* Cache geometry.  All pointers are host memory, read during the call only.
 *  num_layers       >= 1
 *  block_size       tokens per block; a power of two in [1, 1024]
 *  num_kv_heads     >= 1
 *  head_dim         64, 128 or 256
 *  layer_mode       [num_layers] kvq_mode values
 *  layer_num_blocks [num_layers] blocks of each layer, >= 0 (a sliding
 *                   layer may hold only window / block_size blocks) */
typedef struct kvq_cache_config {
    int32_t num_layers;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    const int32_t* layer_mode;
    const int64_t* layer_num_blocks;
} kvq_cache_config;

/* Byte accounting of a cache buffer.
 *  payload       K and V code bytes of all layers (1 B/element FP8,
 *                0.5 B INT4, 2 B BF16)
 *  token_scales  8 B per token-head slot of the per-token-head layers
 *  static_scales 8 B per per-tensor layer, 8 * num_kv_heads B per per-head layer
 *  padding       bytes added to start each layer on a 256-byte boundary
 *  total         payload + token_scales + static_scales + padding: the size
 *                of the device buffer kvq_create_cache needs */
typedef struct kvq_bytes {
    uint64_t payload;
    uint64_t token_scales;
    uint64_t static_scales;
    uint64_t padding;
    uint64_t total;
} kvq_bytes;

/* Opaque host handle describing a cache laid out in caller-owned memory. */
typedef struct kvq_cache kvq_cache;

/*
 * kvq_cache_bytes -- byte accounting of a geometry; pure host arithmetic, no
 * device call.  Payload and per-slot scale formulas: "Per-token-head KV cache
 * scale overhead", sections "Per-token-head KV cache scale overhead" (payload
 * and metadata per retained token), "The FP8 scale tax is 4 divided by head
 * size", "INT4 makes the metadata fraction larger" and "Convert bytes into
 * block capacity" (whole blocks of block_size tokens); static scale bytes:
 * "Per-tensor vs per-head FP8 KV cache scales", "Static per-head metadata is
 * almost free"; BF16 layers: "FP8 KV cache layer skipping vs per-head scales",
 * "Layer skipping follows retained-token footprint".
 *   cfg  host, read only.  out: host, written on success.
 *   Errors: KVQ_ERR_INVALID_ARG (null pointer, bad value),
 *           KVQ_ERR_UNSUPPORTED (head_dim or block_size not supported, a
 *           layer whose block, codes and scales, is 2 GiB or more, or a
 *           buffer beyond 2^62 bytes).
 *
 * Layout of the buffer: layers in order, each starting on a 256-byte
 * boundary; layer l is layer_num_blocks[l] blocks, each block
 *   codes [block_size][num_kv_heads][K, V][row_bytes]   then, per-token-head
 *   modes only, scales [block_size][num_kv_heads][K, V] FP32,
 * where row_bytes is head_dim (FP8), head_dim/2 (INT4) or 2*head_dim (BF16).
 * After the last layer (256-byte aligned) comes the static scale table:
 * per-tensor layers [sK, sV], per-head layers [sK[0..H), sV[0..H)], in layer
 * order.  The slot of (block, position, KV head) holds its K data, K scale,
 * V data and V scale as the pages describe, with the scales grouped at the
 * end of the block so that code rows stay 16-byte aligned.
 */
KVQ_API kvq_status kvq_cache_bytes(const kvq_cache_config* cfg, kvq_bytes* out);

/*
 * kvq_create_cache -- describe a cache that lives in dev_mem.  No device call
 * is made; the memory is not touched (zero it yourself if unwritten slots
 * must read as zero).
 *   cfg        host geometry (copied).
 *   dev_mem    device pointer, 256-byte aligned, dev_bytes >= total.
 *   out        receives the handle; free it with kvq_destroy_cache.
 *   Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_BUFFER_TOO_SMALL.
 * The buffer must outlive the handle.
 */
KVQ_API kvq_status kvq_create_cache(const kvq_cache_config* cfg, void* dev_mem,
                            uint64_t dev_bytes, kvq_cache** out);

/* kvq_destroy_cache -- free the host handle (not the device buffer).  NULL is
 * accepted. */
KVQ_API kvq_status kvq_destroy_cache(kvq_cache* c);

/*
 * kvq_store -- quantize num_tokens new K and V vectors of one layer and
 * scatter them into their cache slots.  "Per-tensor vs per-head FP8 KV cache
 * scales", sections "Per-tensor vs per-head FP8 KV cache scales" (the three
 * scale layouts; the dynamic one measures each new K or V vector over its
 * head dimension) and "Dynamic per-token-head scales add 3.125 percent" (a
 * reduction over each new head vector, then the scales are written beside
 * the data); "Per-token-head KV cache scale overhead", "The FP8 scale tax is 4
 * divided by head size" (slot = K data, K scale, V data, V scale, indexed by
 * block, token position and KV head) and "INT4 makes the metadata fraction
 * larger" (packed INT4 at half width with the same two FP32 scales).
 *   keys, values   device, BF16 [num_tokens][num_kv_heads][head_dim], contiguous,
 *                  16-byte aligned.
 *   slot_mapping   device, int64 [num_tokens]; token t goes to block
 *                  slot / block_size, position slot % block_size.  A negative
 *                  slot, or one >= the layer's blocks * block_size, is not
 *                  stored (ring buffers of sliding layers use -1 for tokens
 *                  outside the window).  A skipped token's K and V are still
 *                  read (all loads are issued before any slot is examined):
 *                  hand a sliding layer only the tokens of its window when
 *                  most of a call would be skipped.  Two tokens with the same slot in one
 *                  call race (undefined which one lands); the Python
 *                  binding's Cache.check_slots finds them, off this path.
 *   mode           must equal the layer's mode (else KVQ_ERR_MODE_MISMATCH).
 *   scales         host FP32.  KVQ_FP8_PER_TENSOR: [sK, sV].
 *                  KVQ_FP8_PER_HEAD: [sK[0..H), sV[0..H)].  Other modes: NULL.
 *                  Positive and finite.  The first call on a static layer
 *                  writes them into the cache's static table; later calls
 *                  pass NULL or the identical values (else KVQ_ERR_INVALID_ARG).
 *   num_tokens == 0 is a no-op returning KVQ_OK; num_tokens * num_kv_heads
 *   must stay below 2^31.
 *   Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_MODE_MISMATCH, KVQ_ERR_UNSUPPORTED
 *           (as for kvq_gather_dequant), KVQ_ERR_HIP.
 * Concurrent kvq_store calls on the same handle and layer are not allowed.
 */
KVQ_API kvq_status kvq_store(kvq_cache* c, int32_t layer, const void* keys, const void* values,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     kvq_mode mode, const float* scales, void* stream);

/*
 * kvq_store_ordered -- kvq_store with the tokens taken in a caller's order.
 * The cache contents are those of kvq_store: every token still lands in its
 * own slot with the same codes and scales; only the order in which the
 * kernel walks the tokens changes.  Blocks are handed out from a free list
 * ("Per-token-head KV cache scale overhead", "Convert bytes into block
 * capacity"), so consecutive tokens land in scattered blocks; walking the
 * tokens in slot order instead makes the writes run through the layer in
 * address order (the reads of the new K/V rows are then the scattered
 * side).  All layers of a model step share one slot mapping, so one order
 * serves every layer's call.
 *   token_order    device, int32 [num_tokens]: a permutation of
 *                  0 .. num_tokens-1, token_order[i] being the token taken
 *                  i-th; the slot order is argsort(slot_mapping).  4-byte
 *                  aligned; NULL only when num_tokens is 0.  Nothing checks
 *                  that it is a permutation.  A layer that follows the order
 *                  skips entries outside [0, num_tokens), so no access
 *                  leaves the arguments, and stores exactly the tokens the
 *                  order names (a repeated token is stored twice alike, an
 *                  omitted one not at all); a layer that does not follow it
 *                  stores every token.
 *   Every other argument, the errors and the no-op cases are kvq_store's.
 *   The order is followed for FP8 and BF16 layers at head_dim 128 and 256,
 *   where slot order measured faster; other layers (INT4, head_dim 64) take
 *   the tokens in their own order, which for a permutation gives the same
 *   contents.
 */
KVQ_API kvq_status kvq_store_ordered(kvq_cache* c, int32_t layer, const void* keys, const void* values,
                             const int64_t* slot_mapping, const int32_t* token_order, int64_t num_tokens,
                             kvq_mode mode, const float* scales, void* stream);

/* kvq_store_follows_order -- 1 if kvq_store_ordered follows the token order
 * on layers of this mode and head_dim, 0 if it takes the tokens in their own
 * order (also for an unknown mode or head_dim).  Host only. */
KVQ_API int32_t kvq_store_follows_order(kvq_mode mode, int32_t head_dim);

/*
 * kvq_gather_dequant -- read one layer's cached tokens of num_seqs sequences
 * through their block tables and write them back as BF16.  The scales are
 * read back when the cache is consumed ("Per-tensor vs per-head FP8 KV cache
 * scales", "Dynamic per-token-head scales add 3.125 percent"); blocks are the
 * fixed-size pages of "Per-token-head KV cache scale overhead", "Convert
 * bytes into block capacity".
 *   block_table         device, int32 [num_seqs][max_blocks_per_seq]: physical
 *                       block of each logical block.
 *   seq_lens            device, int32 [num_seqs]: tokens of each sequence
 *                       (negative counts as 0); must not exceed
 *                       max_blocks_per_seq * block_size.
 *   out_keys, out_values device, BF16 [out_rows][num_kv_heads][head_dim],
 *                       16-byte aligned; sequence b starts at row
 *                       sum(seq_lens[0..b)) (positive lengths only).  Token t
 *                       of sequence b comes from block
 *                       block_table[b][t / block_size], position
 *                       t % block_size.
 *   out_rows            rows (tokens) that out_keys and out_values each hold,
 *                       >= 0.  A token whose output row is out_rows or beyond
 *                       is not written, so an output shorter than
 *                       sum(seq_lens) is never overrun; size it to the sum
 *                       to receive every token.  out_keys and out_values may
 *                       be NULL only when out_rows is 0 (nothing is written
 *                       then).
 *   A block-table entry outside [0, layer blocks) leaves its tokens' output
 *   rows unwritten, as do tokens beyond max_blocks_per_seq * block_size.
 *   A static-scale layer must have been stored to at least once.
 *   num_seqs == 0 or out_rows == 0 is a no-op returning KVQ_OK (after the
 *   argument checks).
 *   Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED (block bytes not a
 *           multiple of 16, i.e. an odd block_size * num_kv_heads with a
 *           per-token-head mode), KVQ_ERR_HIP.
 */
KVQ_API kvq_status kvq_gather_dequant(const kvq_cache* c, int32_t layer, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t num_seqs, void* out_keys, void* out_values,
                              int64_t out_rows, void* stream);

/*
 * kvq_calibrate_amax -- on-the-fly calibration for the static layouts: the
 * running absolute maximum of K and of V per KV head over a batch of new
 * vectors.  "Per-tensor vs per-head FP8 KV cache scales", "Calibration
 * changes which scale layout exists" (static scales estimated during warmup);
 * "Per-token-head KV cache scale overhead", "Static per-head calibration pays
 * once" (the scales must cover every value expected at serving time).
 *   keys, values  device, BF16 [num_tokens][num_kv_heads][head_dim], contiguous,
 *                 16-byte aligned.
 *   amax          device, float [2 * num_kv_heads] (K heads, then V heads),
 *                 4-byte aligned.  amax[i] becomes max(prior, max |x|) where
 *                 prior is amax[i] when accumulate != 0, else 0.
 *   num_tokens == 0 with accumulate == 0 zeroes amax.
 *   Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED (head_dim not 64/128/256,
 *           num_kv_heads above KVQ_MAX_STATIC_KV_HEADS, num_tokens *
 *           num_kv_heads >= 2^31), KVQ_ERR_HIP.
 */
KVQ_API kvq_status kvq_calibrate_amax(const void* keys, const void* values, int64_t num_tokens,
                                      int32_t num_kv_heads, int32_t head_dim, float* amax,
                                      int32_t accumulate, void* stream);

/*
 * kvq_static_scales -- static scales from calibrated maxima (host arithmetic):
 * per-head: scales[i] = RN32(amax[i] / 448) for the 2 * num_kv_heads entries;
 * per-tensor: scales[0] = RN32(max_h amax[h] / 448) (K), scales[1] the same
 * over the V heads.  The absolute maximum maps to the largest E4M3 value, as
 * for the dynamic layout.  A zero maximum gives the smallest positive FP32
 * value instead of 0, so the scale stays valid for kvq_store.
 *   amax    host, float [2 * num_kv_heads], finite and >= 0.
 *   mode    KVQ_FP8_PER_TENSOR or KVQ_FP8_PER_HEAD.
 *   scales  host, float [2] or [2 * num_kv_heads], written on success.
 *   Errors: KVQ_ERR_INVALID_ARG.
 */
KVQ_API kvq_status kvq_static_scales(const float* amax, int32_t num_kv_heads, kvq_mode mode,
                                     float* scales);

/*
 * kvq_decode_attention_workspace -- device workspace bytes that are enough
 * for kvq_decode_attention and kvq_decode_attention_fp8q on any layer of
 * this cache with this call shape (0 when no call of the shape splits its
 * sequences); a call on a given layer may use less (kernels that serve
 * several heads or tiles per wave split less).  Host arithmetic only; no
 * device call.  Arguments as for kvq_decode_attention.
 *   Errors: KVQ_ERR_INVALID_ARG.
 */
KVQ_API kvq_status kvq_decode_attention_workspace(const kvq_cache* c, int32_t num_q_heads,
                                                  int32_t max_blocks_per_seq, int32_t num_seqs,
                                                  uint64_t* bytes);

/*
 * kvq_decode_attention -- attention of one new query token per sequence over
 * that sequence's cached tokens of one layer, reading the codes and their
 * scales straight from the paged blocks ("Per-tensor vs per-head FP8 KV cache
 * scales" and "Dynamic per-token-head scales add 3.125 percent": the scales
 * are read during attention; "FP8 KV cache layer skipping vs per-head
 * scales": BF16 layers are attended alike).  Query head g uses KV head
 * g / (num_q_heads / num_kv_heads):
 *   out[b][g] = sum_t softmax_t(sm_scale * q[b][g] . K^[t]) * V^[t]
 * over t < seq_lens[b], with K^, V^ the dequantized cache values.
 *   q             device, BF16 [num_seqs][num_q_heads][head_dim], 16-byte aligned.
 *   num_q_heads   a positive multiple of the cache's num_kv_heads.
 *   block_table, max_blocks_per_seq, seq_lens, num_seqs
 *                 as for kvq_gather_dequant; lengths are clamped to
 *                 [0, max_blocks_per_seq * block_size].  A token whose
 *                 block-table entry lies outside [0, layer blocks) takes no
 *                 part; a sequence left with no token gives zeros.
 *   sm_scale      finite softmax scale (1/sqrt(head_dim) for the usual model).
 *   out           device, BF16 [num_seqs][num_q_heads][head_dim], 16-byte aligned.
 *   workspace     device, 16-byte aligned, at least the bytes that
 *                 kvq_decode_attention_workspace reports (NULL when 0).  Owned
 *                 by the caller; it may be reused once the call's work on
 *                 the stream has finished.
 *   Results are FP32-accumulated: scores exactly of the widened codes, the
 *   softmax weights times per-token V scales rounded to BF16 before the value
 *   product, the output rounded to BF16.
 *   A static-scale layer must have been stored to at least once.
 *   num_seqs == 0 is a no-op returning KVQ_OK.
 *   Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_BUFFER_TOO_SMALL (workspace),
 *           KVQ_ERR_UNSUPPORTED (a block of 2 GiB or more,
 *           max_blocks_per_seq * block_size >= 2^31, block bytes not a
 *           multiple of 16), KVQ_ERR_HIP.
 */
KVQ_API kvq_status kvq_decode_attention(const kvq_cache* c, int32_t layer, const void* q, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t num_seqs, float sm_scale, void* out,
                                        void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * kvq_decode_attention_fp8q -- kvq_decode_attention with FP8 queries: each
 * query element is encoded to E4M3 under a static scale of its query head,
 * the way the cache encodes K and V (E4M3(RN32(q / s)), nearest even,
 * saturating at 448), and the Q K^T products run on the FP8 codes directly.
 * This is the per-attention-head calibration's one Q scale per query head
 * ("Per-tensor vs per-head FP8 KV cache scales", the section of the same
 * name; "FP8 KV cache layer skipping vs per-head scales", "Per-head scales
 * have fixed overhead": H query scales beside 2 * Hkv K and V scales);
 * a per-tensor Q scale is H equal values.  kvq_calibrate_amax over the
 * queries and kvq_static_scales give such scales.
 *   q_scales   device FP32 [num_q_heads], 4-byte aligned, positive and finite
 *              (not checked: other values give undefined results, never a
 *              memory fault).
 *   Other arguments, workspace and results as kvq_decode_attention, with the
 *   queries' decoded FP8 values in place of the BF16 ones.
 *   Errors: as kvq_decode_attention; KVQ_ERR_INVALID_ARG for a null
 *           q_scales; KVQ_ERR_UNSUPPORTED for a BF16 or INT4 layer.
 */
KVQ_API kvq_status kvq_decode_attention_fp8q(const kvq_cache* c, int32_t layer, const void* q, const float* q_scales,
                                             int32_t num_q_heads, const int32_t* block_table,
                                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                             float sm_scale, void* out, void* workspace, uint64_t workspace_bytes,
                                             void* stream);

/* Bytes of the fixed device array that holds kvq_decode_attention_noalloc's
 * split partials (one copy per GPU, kept until the process ends). */
#define KVQ_ATTENTION_SCRATCH_BYTES (32ull << 20)

/*
 * kvq_decode_attention_noalloc -- kvq_decode_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels, plan and
 * results, with the split partials kept in a fixed device array of
 * KVQ_ATTENTION_SCRATCH_BYTES instead of a caller workspace.  Nothing is
 * allocated by the call; the array's device address is looked up once per
 * GPU, on the first call made with that GPU current.
 *   Arguments, results and errors as kvq_decode_attention without
 *   workspace / workspace_bytes; KVQ_ERR_UNSUPPORTED also when the call
 *   shape needs more than KVQ_ATTENTION_SCRATCH_BYTES of partials
 *   (kvq_decode_attention_workspace reports the need; shapes with one split
 *   need none).
 *   All calls on one GPU share its array, and the partials of a call are
 *   live until that call's work on its stream has finished: calls that
 *   overlap on one GPU (other streams, other threads, other handles) race
 *   and give undefined results.  Calls on different GPUs do not interact.
 */
KVQ_API kvq_status kvq_decode_attention_noalloc(const kvq_cache* c, int32_t layer, const void* q,
                                                int32_t num_q_heads, const int32_t* block_table,
                                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                int32_t num_seqs, float sm_scale, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Capacity planning and the decode-time block manager (host code only)
 * ---------------------------------------------------------------------- */

/* Model geometry for planning: a cache geometry without block counts, plus
 * each layer's retention.  All pointers are host memory, read during the call.
 *  layer_mode    [num_layers] kvq_mode values
 *  layer_window  [num_layers] 0 = full attention (the layer retains the whole
 *                context); W > 0 = sliding window retaining at most the last
 *                W positions, a multiple of block_size ("FP8 KV cache layer
 *                skipping vs per-head scales", "Layer skipping follows
 *                retained-token footprint")
 * Other fields as in kvq_cache_config. */
typedef struct kvq_model_config {
    int32_t num_layers;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    const int32_t* layer_mode;
    const int32_t* layer_window;
} kvq_model_config;

/* A capacity plan for sequences of one context length.
 *  retained_positions  A: retained token-layer positions of one sequence,
 *                      min(context, W) for a sliding layer, context otherwise
 *  skipped_positions   S: the same sum over the BF16 (skipped) layers; the
 *                      payload compression against all-BF16 is 2A / (A + S)
 *                      when the quantized layers carry no per-token scales
 *  sequence_bytes      one sequence's cache bytes: whole blocks of every
 *                      layer, codes plus per-token scales
 *  max_sequences       the most sequences of this context whose whole cache
 *                      buffer (kvq_cache_bytes().total of the planned block
 *                      counts: blocks, layer alignment, static scales) fits
 *                      the pool
 *  max_tokens          max_sequences * context
 *  buffer_bytes        kvq_cache_bytes().total of the planned block counts */
typedef struct kvq_plan {
    int64_t retained_positions;
    int64_t skipped_positions;
    uint64_t sequence_bytes;
    int64_t max_sequences;
    int64_t max_tokens;
    uint64_t buffer_bytes;
} kvq_plan;

/*
 * kvq_plan_capacity -- how many sequences of `context` tokens fit a usable
 * pool of pool_bytes, and the block count of every layer that holds them.
 * "Per-token-head KV cache scale overhead", section "Convert bytes into block
 * capacity" (bytes per token times the block size, rounded to whole blocks;
 * the usable pool, after weights, activations and runtime reserves, divided
 * by the rounded bytes); "FP8 KV cache layer skipping vs per-head scales",
 * section "Layer skipping follows retained-token footprint" (a sliding layer
 * retains at most its window; A and S).  The byte prices are the cache
 * layout's own, so passing layer_num_blocks to kvq_create_cache with a
 * buffer of buffer_bytes always fits the pool.
 *   model             host, read only.
 *   context           >= 1 tokens per sequence.
 *   pool_bytes        the usable pool; the caller subtracts every reserve.
 *   out               host, written on success.
 *   layer_num_blocks  host [num_layers] or NULL: max_sequences times each
 *                     layer's blocks per sequence.
 *   Errors: KVQ_ERR_INVALID_ARG (null pointer, bad value, a window that is
 *           not a multiple of block_size), KVQ_ERR_UNSUPPORTED (as
 *           kvq_cache_bytes).
 */
KVQ_API kvq_status kvq_plan_capacity(const kvq_model_config* model, int64_t context, uint64_t pool_bytes,
                                     kvq_plan* out, int64_t* layer_num_blocks);

/* Opaque host handle: the blocks of a cache handed out to sequences. */
typedef struct kvq_seq_manager kvq_seq_manager;

/*
 * kvq_manager_create -- a block manager over a cache geometry.  Layers with
 * the same window form a group that shares block ids (each id names a block
 * in every layer of the group, in that layer's own region), so every layer
 * of a group must have the same block count.  A full-attention group gives
 * each sequence a growing list of blocks; a sliding group gives it a ring of
 * W / block_size blocks in which token t occupies position t mod W, so only
 * the last W tokens are retained ("FP8 KV cache layer skipping vs per-head
 * scales", "Layer skipping follows retained-token footprint").
 *   model               host, read only (the windows define the groups).
 *   layer_num_blocks    host [num_layers]: the cache's blocks per layer.
 *   max_blocks_per_seq  block-table width: the longest sequence is
 *                       max_blocks_per_seq * block_size tokens.
 *   out                 receives the handle; free it with kvq_manager_destroy.
 *   Errors: KVQ_ERR_INVALID_ARG.
 * Not thread safe: one caller at a time per handle.
 */
KVQ_API kvq_status kvq_manager_create(const kvq_model_config* model, const int64_t* layer_num_blocks,
                                      int32_t max_blocks_per_seq, kvq_seq_manager** out);
KVQ_API kvq_status kvq_manager_destroy(kvq_seq_manager* m);

/* kvq_manager_num_groups / kvq_manager_layer_group -- the number of layer
 * groups, and the group of a layer (groups are numbered in order of their
 * first layer).  Errors: KVQ_ERR_INVALID_ARG. */
KVQ_API kvq_status kvq_manager_num_groups(const kvq_seq_manager* m, int32_t* num_groups);
KVQ_API kvq_status kvq_manager_layer_group(const kvq_seq_manager* m, int32_t layer, int32_t* group);

/*
 * kvq_manager_append -- reserve n more tokens for sequence seq (an unknown
 * id starts a new, empty sequence) and write the slot of every new token in
 * every group: slots[g * n + i] is the kvq_store slot of token i for the
 * layers of group g.  In a sliding group, a token that a later token of the
 * same call displaces from the window gets slot -1 (kvq_store skips it), so
 * the slots of one call never coincide.  Blocks come from the group's free
 * list, lowest id first when none was released.
 *   seq    >= 0.  n >= 0.  slots: host [num_groups * n].
 *   Errors: KVQ_ERR_INVALID_ARG (bad argument, or the sequence would need
 *           more than max_blocks_per_seq blocks), KVQ_ERR_NO_SPACE (a group
 *           has no free block left).  On an error nothing changes.
 */
KVQ_API kvq_status kvq_manager_append(kvq_seq_manager* m, int32_t seq, int32_t n, int64_t* slots);

/* kvq_manager_release -- return a sequence's blocks to the free lists.
 * Errors: KVQ_ERR_INVALID_ARG (unknown sequence). */
KVQ_API kvq_status kvq_manager_release(kvq_seq_manager* m, int32_t seq);

/*
 * kvq_manager_tables -- the block table and lengths of group `group` for the
 * given sequences, ready for kvq_gather_dequant and kvq_decode_attention:
 * block_table[i][j] is the j-th block of seqs[i] (-1 past its last block),
 * seq_lens[i] its retained tokens (min(length, W) in a sliding group, whose
 * tokens are in ring order, which attention does not depend on).
 *   seqs        host [num_seqs] known sequence ids.
 *   block_table host [num_seqs][max_blocks].  seq_lens: host [num_seqs].
 *   Errors: KVQ_ERR_INVALID_ARG (unknown sequence, a table too narrow).
 */
KVQ_API kvq_status kvq_manager_tables(const kvq_seq_manager* m, int32_t group, const int32_t* seqs,
                                      int32_t num_seqs, int32_t max_blocks, int32_t* block_table,
                                      int32_t* seq_lens);

/* kvq_status_string -- static description of a status code. */
KVQ_API const char* kvq_status_string(kvq_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
