// kvq_attention.hip -- fused paged decode attention over the quantized cache
// (gfx950).  One new query token per sequence attends over the sequence's
// cached tokens; the kernel reads FP8 / INT4 codes and their scales (or BF16
// rows) straight from the paged blocks, so no dequantized copy of the cache
// is ever written.  Scales are read during attention, as "Per-tensor vs
// per-head FP8 KV cache scales" and "Dynamic per-token-head scales add 3.125
// percent" describe; the layer-skip BF16 layers ("FP8 KV cache layer
// skipping vs per-head scales") are attended by the same kernel.
//
// Arithmetic.  Codes widen exactly to BF16 (every E4M3 value and every INT4
// value / 16 is a BF16 number), so both products run on MFMA with exact
// operands and FP32 accumulation; the scales stay out of the products:
//   S[t][g]  = (sum_d code_K[t][d] * q[g][d]) * s_K[t] * sm_scale * log2(e)
//   P'[t][g] = BF16(exp2(S[t][g] - m[g]) * s_V[t])            (per-token-head)
//   O[g][d] += sum_t P'[t][g] * code_V[t][d]
// with an online (running-maximum) softmax over 16-token tiles; static
// scales are applied once, s_K folded into the score factor and s_V into the
// final output.  INT4 codes enter biased, as (n + 8) / 16 (a nibble XOR 8 is
// the E4M3 code of (n + 8) 2^-9); the bias leaves through the Q K^T
// product's initial accumulator and a separate value-bias accumulator.
//
// Work split.  A workgroup holds one wave per KV head of a run of heads and
// walks a range of tiles of one sequence; the waves of a workgroup read
// adjacent rows of the same blocks, and share the blocks' scale lines.  Each
// wave serves up to 16 query heads of its KV head (the MFMA N dimension).
// Long sequences are cut into splits whose partial (O, m, l) a second kernel
// combines; with one split the first kernel writes the output itself.
// Per-token-head layers with query groups of at most 4 (FP8 at head_dim 64,
// INT4 at 64 and 128) take attention_quad_kernel instead, whose waves each
// serve a quad of 4 KV heads on the same grid, plan and partials.  Where a
// workgroup holds only one or two KV heads (a tensor-parallel shard), those
// layers, and FP8 at head_dim 128 on two heads, take attention_tquad_kernel,
// whose waves each spread 4 consecutive tiles of one head (or 2 tiles of
// each head of a pair) over the 16 MFMA columns.
//
// MFMA operand layouts used here (gfx950, lane l, r = l % 16, q = l / 16):
//   mfma_f32_16x16x32_bf16:     A[m=r][k=8q+i], B[k=8q+i][n=r], D[m=4q+i][n=r]
//   mfma_f32_16x16x16_bf16_1k:  A[m=r][k=4q+i], B[k=4q+i][n=r], D[m=4q+i][n=r]
// Q K^T takes m = token, n = query head and its k slots permuted so that lane
// l holds the contiguous dims [q*hd/4, (q+1)*hd/4) of token r's K row; the
// result D[t=4q+i][g=r] is already the B operand of P V (k = token, n =
// head), which takes m = 16 dims spaced J = hd/16 apart, so that lane l
// loads J contiguous dims of 4 tokens' V rows and ends up holding hd/4
// contiguous output dims of query head r.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = kAttnTile;
constexpr int kMaxHeadsPerWg = kAttnMaxHeadsPerWg;
constexpr int kMaxAttnThreads = 64 * kMaxHeadsPerWg;
constexpr int kMaxSplits = kAttnMaxSplits;
constexpr int kWideCombineSplits = 16;       // from here on the combine spreads the splits
constexpr int kMaxStagedPieces = 16;         // 16-byte pieces per lane of a staged tile (16 KiB)
constexpr float kLog2e = 1.4426950408889634f;

template <int HD, int MODE>
struct Geo {
    static constexpr int J = HD / 16;                 // 16-dim output tiles of P V
    static constexpr int KSTEPS = HD / 32;            // 32-dim k steps of Q K^T
    static constexpr int BITS = MODE == KVQ_BF16 ? 16 : (MODE == KVQ_INT4_PER_TOKEN_HEAD ? 4 : 8);
    static constexpr int RB = HD * BITS / 8;          // bytes of one K or V row
    static constexpr int KB = RB / 4;                 // K bytes per lane (hd/4 dims)
    static constexpr int VB = J * BITS / 8;           // V bytes per lane and token (J dims)
    static constexpr int VL = VB < 4 ? 4 : VB;        // V bytes loaded (a 2-byte slice comes
                                                      // with its neighbour's, in one aligned dword)
    static constexpr int KW = (KB + 3) / 4;
    static constexpr int VW = VL / 4;
    static constexpr bool DYN = dynamic_mode<MODE>();
    // Staged reads: a tile's 16 K|V row pairs (2 * RB bytes each) read as
    // whole 16-byte pieces, NC wave-wide loads of 1 KiB, then regrouped in LDS.
    static constexpr int NC = 16 * 2 * RB / 1024;
    // A 1 KiB piece is exactly one token's row pair (BF16 at head_dim 256):
    // piece c of every lane lies one token further, a wave-uniform step.
    static constexpr bool PIECE_IS_ROW = 2 * RB == 1024;
    static constexpr int LDS_ROW = 2 * RB + 16;       // padded row pair: conflict-free K slices
    static constexpr int LDS_TILE = 16 * LDS_ROW;
    // INT4 codes widen to n / 16 (exact); the 16 goes back in with the scales.
    static constexpr float CODE_UNIT = MODE == KVQ_INT4_PER_TOKEN_HEAD ? 16.0f : 1.0f;
};

struct AttnArgs {
    const uint8_t* layer;          // layer base
    const float* statics;          // layer's static scale table (static modes)
    const uint16_t* q;             // BF16 [num_seqs][H][hd]
    const float* q_scales;         // [H] static FP8 query scales (FP8-query kernels)
    const int32_t* block_table;    // [num_seqs][max_blocks]
    const int32_t* seq_lens;       // [num_seqs]
    uint16_t* out;                 // BF16 [num_seqs][H][hd]      (one split)
    float* part_o;                 // [num_seqs][H][splits][hd]   (several splits)
    float* part_ml;                // [num_seqs][H][splits][2]
    int64_t block_bytes;
    int64_t num_blocks;
    int32_t code_bytes;            // offset of the scale trailer in a block
    int32_t hkv;
    int32_t num_q_heads;
    int32_t group;                 // query heads per KV head
    int32_t qgroups;               // ceil(group / 16)
    int32_t heads_per_wg;          // waves per workgroup
    int32_t head_chunks;           // hkv / heads_per_wg
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t splits;
    int32_t tiles_per_split;
    int32_t bs_log2;
    int32_t max_len;               // max_blocks * block_size, 0 for a layer without blocks
    uint32_t total_wg;
    float c;                       // sm_scale * log2(e)
    int32_t kind;                  // AttnKind: the kernel the plan sized the grid for
};

// ------------------------------------------------------------ lane helpers

template <int N, bool NT>
__device__ __forceinline__ void load_n(uint32_t* dst, const uint8_t* p) {
    if constexpr (N >= 16) {
#pragma unroll
        for (int k = 0; k < N / 16; ++k) {
            const uint4 v = ld16<NT>(p + 16 * k);
            dst[4 * k] = v.x;
            dst[4 * k + 1] = v.y;
            dst[4 * k + 2] = v.z;
            dst[4 * k + 3] = v.w;
        }
    } else if constexpr (N == 8) {
        u32x2 v;
        if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        else v = *reinterpret_cast<const u32x2*>(p);
        dst[0] = v[0];
        dst[1] = v[1];
    } else {
        static_assert(N == 4, "row slice of 4, 8 or a multiple of 16 bytes");
        if constexpr (NT) dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
        else dst[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// Raw buffer loads (gfx9 descriptor word 3; cache-policy bit 1 = non-temporal).
constexpr int kBufferDword3 = 0x00020000;
constexpr int kNonTemporal = 2;

template <int N, int AUX>
__device__ __forceinline__ void buf_load(uint32_t* dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
    if constexpr (N >= 16) {
#pragma unroll
        for (int k = 0; k < N / 16; ++k) {
            const u32x4 v = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff) + 16 * k, soff, AUX));
            dst[4 * k] = v[0];
            dst[4 * k + 1] = v[1];
            dst[4 * k + 2] = v[2];
            dst[4 * k + 3] = v[3];
        }
    } else if constexpr (N == 8) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>(voff), soff, AUX));
        dst[0] = v[0];
        dst[1] = v[1];
    } else {
        static_assert(N == 4, "row slice of 4, 8 or a multiple of 16 bytes");
        dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(voff), soff, AUX);
    }
}

// Pair (a, b) of a wave's lanes l and l ^ 16, and of l and l ^ 32, through
// the gfx950 row swaps: each lane receives its partner's value beside its own.
__device__ __forceinline__ float max_q4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_q4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two E4M3 codes (byte pair HI of w) -> two BF16 values, exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// K step j of the lane's K slice -> 8 BF16 A-operand values (dims 8j .. 8j+7
// of the slice).
template <int HD, int MODE>
__device__ __forceinline__ bf16x8 k_operand(const uint32_t* k, int j) {
    uint32_t o[4];
    if constexpr (MODE == KVQ_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = k[4 * j + e];
    } else if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
        // Biased keys: a nibble n (two's complement) XOR 8 is n + 8 in 0..15,
        // and alone in its byte it is the E4M3 code of (n + 8) 2^-9 (codes
        // 0x00..0x0F are m 2^-9 exactly: the subnormal step runs on through
        // the first binade); converted with the scale 2^5 it is (n + 8) / 16,
        // exact in BF16.  Element 2b is the low nibble of byte b, 2b + 1 the
        // high one, so the dwords hold elements (0, 2), (4, 6), (1, 3), (5, 7)
        // of the code dword; the query operand is permuted alike
        // (int4_query_order) and the bias (8 / 16) sum(q) leaves through the
        // product's initial accumulator (int4_key_bias).
        const uint32_t w = k[j];
        const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;
        const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 32.0f, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 32.0f, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 32.0f, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 32.0f, true));
    } else {
        o[0] = fp8x2_to_bf16x2<false>(k[2 * j]);
        o[1] = fp8x2_to_bf16x2<true>(k[2 * j]);
        o[2] = fp8x2_to_bf16x2<false>(k[2 * j + 1]);
        o[3] = fp8x2_to_bf16x2<true>(k[2 * j + 1]);
    }
    const u32x4 v = {o[0], o[1], o[2], o[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// V operands of the J P V tiles from the lane's 4 token slices
// (v[i] = J dims of token 4q+i): A_j = (V[0][j], V[1][j], V[2][j], V[3][j]).
template <int HD, int MODE>
__device__ __forceinline__ void v_operands(const uint32_t (*v)[Geo<HD, MODE>::VW], s16x4* a) {
    constexpr int J = Geo<HD, MODE>::J;
    if constexpr (MODE == KVQ_BF16) {
#pragma unroll
        for (int j = 0; j < J; j += 2) {
            // dword j/2 of each token holds dims j (low half) and j+1 (high half)
            const uint32_t lo01 = __builtin_amdgcn_perm(v[1][j / 2], v[0][j / 2], 0x05040100u);
            const uint32_t lo23 = __builtin_amdgcn_perm(v[3][j / 2], v[2][j / 2], 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(v[1][j / 2], v[0][j / 2], 0x07060302u);
            const uint32_t hi23 = __builtin_amdgcn_perm(v[3][j / 2], v[2][j / 2], 0x07060302u);
            const u32x2 x = {lo01, lo23};
            const u32x2 y = {hi01, hi23};
            a[j] = __builtin_bit_cast(s16x4, x);
            a[j + 1] = __builtin_bit_cast(s16x4, y);
        }
    } else if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
        static_assert(MODE != KVQ_INT4_PER_TOKEN_HEAD, "INT4 values widen in v_operands_int4");
    } else {
#pragma unroll
        for (int j = 0; j < J; j += 2) {
            // bytes b, b+1 of dword j/4 hold dims j, j+1; interleave two tokens
            const int w = j / 4, b = j % 4;
            const uint32_t sel = static_cast<uint32_t>(b) | (static_cast<uint32_t>(4 + b) << 8) |
                                 (static_cast<uint32_t>(b + 1) << 16) | (static_cast<uint32_t>(5 + b) << 24);
            const uint32_t t01 = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
            const uint32_t t23 = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
            const u32x2 x = {fp8x2_to_bf16x2<false>(t01), fp8x2_to_bf16x2<false>(t23)};
            const u32x2 y = {fp8x2_to_bf16x2<true>(t01), fp8x2_to_bf16x2<true>(t23)};
            a[j] = __builtin_bit_cast(s16x4, x);
            a[j + 1] = __builtin_bit_cast(s16x4, y);
        }
    }
}

// INT4 V operands, biased like the keys: the lane's slice of a token is J
// dims, dim j the low (j even) or high (j odd) nibble of slice byte j / 2.
// One byte permute interleaves two tokens' byte pair p (dims 4p .. 4p+3):
// [t0.B2p, t1.B2p, t0.B2p+1, t1.B2p+1]; XOR 8 per nibble makes n + 8 in
// 0..15, and split into low and high nibbles each byte is the E4M3 code of
// (n + 8) 2^-9, which the scaled conversion (2^5) turns into (n + 8) / 16,
// exact in BF16.  So a pair of conversions gives one operand half: two
// tokens of one dim.  The bias (8 / 16) sum_t P'_t leaves through its own
// MFMA (int4_value_bias) and a subtraction at the end.  Every biased code is
// finite, so masked tokens need no zeroing: their weight is 0.  vsel picks
// the lane's byte pair from a token dword (2-byte slices at head_dim 64).
template <int HD>
__device__ __forceinline__ void v_operands_int4(const uint32_t (*v)[Geo<HD, KVQ_INT4_PER_TOKEN_HEAD>::VW],
                                                uint32_t vsel, s16x4* a) {
    using G = Geo<HD, KVQ_INT4_PER_TOKEN_HEAD>;
#pragma unroll
    for (int p = 0; p < G::J / 4; ++p) {
        const int w = G::VB == 2 ? 0 : p / 2;
        const uint32_t sel = G::VB == 2 ? vsel : ((p & 1) ? 0x07030602u : 0x05010400u);
        const uint32_t x01 = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
        const uint32_t lo01 = (x01 & 0x0F0F0F0Fu) ^ 0x08080808u, hi01 = ((x01 >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
        const uint32_t lo23 = (x23 & 0x0F0F0F0Fu) ^ 0x08080808u, hi23 = ((x23 >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
        const u32x2 d0 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo01, 32.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo23, 32.0f, false))};
        const u32x2 d1 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi01, 32.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi23, 32.0f, false))};
        const u32x2 d2 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo01, 32.0f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo23, 32.0f, true))};
        const u32x2 d3 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi01, 32.0f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi23, 32.0f, true))};
        a[4 * p] = __builtin_bit_cast(s16x4, d0);
        a[4 * p + 1] = __builtin_bit_cast(s16x4, d1);
        a[4 * p + 2] = __builtin_bit_cast(s16x4, d2);
        a[4 * p + 3] = __builtin_bit_cast(s16x4, d3);
    }
}

// The value bias of one tile: (8 / 16) sum_t P'_t for each query column, in
// every row of the accumulator, through the P V product with every value 1/2.
__device__ __forceinline__ f32x4 int4_value_bias(s16x4 b, f32x4 acc) {
    const u32x2 halves = {0x3F003F00u, 0x3F003F00u};   // BF16 0.5
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, halves), b, acc, 0, 0, 0);
}

// ------------------------------------------------------------ the kernel

// Tiles in flight per wave: enough bytes outstanding to cover the memory
// latency with the waves a CU holds, within the register budget.
template <int HD, int MODE>
constexpr int attention_depth() {
    return HD == 64 ? 4 : 2;
}

// Tiles per softmax round: one, or two when their columns are packed (PACK:
// a query group of at most 8 heads fills at most half of the 16 MFMA
// columns, so two tiles' scores share one set of lanes and one softmax).
// Rounds of two unpacked tiles measured no faster: the path is then bound by
// the memory requests in flight, not by the round's latency.
template <int HD, int MODE, bool PACK>
constexpr int attention_round() {
    return PACK ? 2 : 1;
}

// Whether a tile's K and V rows are read as whole lines and regrouped in LDS
// (one L2 request per line) instead of straight into the MFMA operand lanes
// (where the K and the V slices of a line are separate requests): every
// case, whose tiles of row pairs are 1 to 16 KiB.
template <int HD, int MODE>
constexpr bool attention_staged() {
    return Geo<HD, MODE>::NC >= 1 && Geo<HD, MODE>::NC <= kMaxStagedPieces;
}

// Whether rounds with no token to mask take a path of their own (at head_dim
// 256 the second copy of the round costs more registers than it saves).
template <int HD>
constexpr bool attention_fast_path() {
    return HD < 256;
}

// Waves per SIMD the register allocation must allow: one workgroup of eight
// waves per CU.
template <int HD>
constexpr int attention_waves() {
    return 2;
}

template <int HD, int MODE>
struct Tile {
    uint32_t k[Geo<HD, MODE>::KW];
    uint32_t v[4][Geo<HD, MODE>::VW];
    f32x2 s[4];                    // (s_K, s_V) of tokens 4q+i (per-token-head modes)
    uint32_t ok;                   // bit i: token 4q+i's block names a block of the layer
};

// A tile read for LDS regrouping: this lane's whole 16-byte pieces of the
// tile's 16 K|V row pairs, plus the same scales and mask as Tile.
template <int HD, int MODE>
struct RawTile {
    uint32_t kv[4 * Geo<HD, MODE>::NC];
    f32x2 s[4];
    uint32_t ok;
};

// Per-lane byte offsets inside a block, fixed for a wave (KV head h, lane
// r, q4): the tile's first position adds a wave-uniform term, so the loads
// take a scalar base and a 32-bit lane offset.
struct LaneOff {
    uint32_t kv[kMaxStagedPieces]; // staged reads: the lane's 16-byte pieces of the tile's row pairs
    uint32_t vsh;                  // right shift that moves a 2-byte V slice to bits 0..15
    uint32_t vsel;                 // byte-permute selector of the lane's 2-byte V slice (INT4 at head_dim 64)
    uint32_t k;                    // K slice of token r
    uint32_t v[4];                 // V slices of tokens 4q4+i
    uint32_t s[4];                 // (s_K, s_V) of tokens 4q4+i, from the scale trailer
};

template <int HD, int MODE>
__device__ __forceinline__ LaneOff lane_offsets(const AttnArgs& a, int h, int r, int q4) {
    using G = Geo<HD, MODE>;
    const uint32_t hkv = static_cast<uint32_t>(a.hkv), uh = static_cast<uint32_t>(h);
    LaneOff o;
    const uint32_t lane = static_cast<uint32_t>(16 * q4 + r);
#pragma unroll
    for (int c = 0; c < (G::PIECE_IS_ROW ? 1 : (G::NC < kMaxStagedPieces ? G::NC : kMaxStagedPieces)); ++c) {
        const uint32_t g = static_cast<uint32_t>(c) * 1024u + lane * 16u;       // byte of the tile's row-pair image
        const uint32_t tok = g / (2 * G::RB), off = g % (2 * G::RB);
        o.kv[c] = (tok * hkv + uh) * (2 * G::RB) + off;
    }
    o.vsh = G::VB == 2 ? 16u * static_cast<uint32_t>(r & 1) : 0u;
    o.vsel = (r & 1) ? 0x07030602u : 0x05010400u;
    o.k = ((static_cast<uint32_t>(r) * hkv + uh) * 2) * G::RB + static_cast<uint32_t>(q4) * G::KB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pos = static_cast<uint32_t>(4 * q4 + i);
        o.v[i] = (((pos * hkv + uh) * 2 + 1) * G::RB + static_cast<uint32_t>(r) * G::VB) & ~static_cast<uint32_t>(G::VL - 1);
        o.s[i] = static_cast<uint32_t>(a.code_bytes) + (pos * hkv + uh) * 8;
    }
    return o;
}

// Loads of tile tau of sequence b for KV head h.  Entries of the block table
// that do not name a block of the layer read block 0 instead and are masked.
// With blocks of 16 or more tokens a tile lies in one block, whose id (blk,
// read by the caller one tile ahead) is the same for the whole wave.
template <int HD, int MODE, bool SMALL_BS>
__device__ __forceinline__ void load_tile(const AttnArgs& a, const int32_t* bt_row, int blk, int h, int tau, int r,
                                          int q4, const LaneOff& lo, Tile<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
    const int t0 = tau * kTile;
    const int bs_mask = (1 << a.bs_log2) - 1;
    if constexpr (!SMALL_BS) {
        // (layers hold at most 2^31 blocks, so the unsigned compare also
        // rejects negative ids)
        const bool ok = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks);
        const uint32_t ublk = ok ? static_cast<uint32_t>(blk) : 0u;
        const uint32_t pos0 = static_cast<uint32_t>(t0 & bs_mask);
        // a buffer descriptor of the block: lane offsets in VGPRs, the tile's
        // first row as a scalar offset, no 64-bit address arithmetic per lane
        const uint8_t* base = a.layer + static_cast<uint64_t>(ublk) * static_cast<uint64_t>(a.block_bytes);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(base), 0, static_cast<int>(a.block_bytes), kBufferDword3);
        const int srow = static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * (2 * G::RB));
        buf_load<G::KB, kNonTemporal>(T.k, rs, lo.k, srow);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            buf_load<G::VL, kNonTemporal>(T.v[i], rs, lo.v[i], srow);
            if constexpr (G::DYN) {
                uint32_t w[2];
                buf_load<8, 0>(w, rs, lo.s[i], static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * 8u));
                T.s[i] = f32x2{__uint_as_float(w[0]), __uint_as_float(w[1])};
            }
        }
        T.ok = ok ? 0xFu : 0u;
    } else {
        const int last = a.max_blocks - 1;
        {
            const int t = t0 + r;
            int blk = bt_row[min(t >> a.bs_log2, last)];
            blk = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks) ? blk : 0;
            const uint8_t* base = a.layer + static_cast<uint64_t>(static_cast<uint32_t>(blk)) * a.block_bytes;
            load_n<G::KB, true>(T.k, base + ((((t & bs_mask) * a.hkv) + h) * 2) * G::RB + q4 * G::KB);
        }
        uint32_t ok = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * q4 + i;
            int blk = bt_row[min(t >> a.bs_log2, last)];
            const bool good = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks);
            blk = good ? blk : 0;
            ok |= good ? (1u << i) : 0u;
            const uint8_t* base = a.layer + static_cast<uint64_t>(static_cast<uint32_t>(blk)) * a.block_bytes;
            const int pos = t & bs_mask;
            load_n<G::VL, true>(T.v[i], base + ((((pos * a.hkv + h) * 2) + 1) * G::RB + r * G::VB) / G::VL * G::VL);
            if constexpr (G::DYN)
                T.s[i] = *reinterpret_cast<const f32x2*>(base + a.code_bytes + (pos * a.hkv + h) * 8);
        }
        T.ok = ok;
    }
}

// Staged loads of tile tau (blocks of 16 or more tokens only).
template <int HD, int MODE>
__device__ __forceinline__ void load_raw(const AttnArgs& a, int blk, int tau, const LaneOff& lo, RawTile<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
    const int t0 = tau * kTile;
    const bool ok = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks);
    const uint32_t ublk = ok ? static_cast<uint32_t>(blk) : 0u;
    const uint32_t pos0 = static_cast<uint32_t>(t0 & ((1 << a.bs_log2) - 1));
    const uint8_t* base = a.layer + static_cast<uint64_t>(ublk) * static_cast<uint64_t>(a.block_bytes);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base), 0, static_cast<int>(a.block_bytes), kBufferDword3);
    const int srow = static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * (2 * G::RB));
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        if constexpr (G::PIECE_IS_ROW)
            buf_load<16, kNonTemporal>(T.kv + 4 * c, rs, lo.kv[0], srow + c * a.hkv * 1024);
        else
            buf_load<16, kNonTemporal>(T.kv + 4 * c, rs, lo.kv[c], srow);
    }
    if constexpr (G::DYN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[2];
            buf_load<8, 0>(w, rs, lo.s[i], static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * 8u));
            T.s[i] = f32x2{__uint_as_float(w[0]), __uint_as_float(w[1])};
        }
    }
    T.ok = ok ? 0xFu : 0u;
}

// The staged tile into the wave's LDS rows.
template <int HD, int MODE>
__device__ __forceinline__ void stage_write(const RawTile<HD, MODE>& R, uint8_t* lds, int r, int q4) {
    using G = Geo<HD, MODE>;
    const uint32_t lane = static_cast<uint32_t>(16 * q4 + r);
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        const uint32_t g = static_cast<uint32_t>(c) * 1024u + lane * 16u;
        const uint32_t tok = g / (2 * G::RB), off = g % (2 * G::RB);
        const u32x4 v = {R.kv[4 * c], R.kv[4 * c + 1], R.kv[4 * c + 2], R.kv[4 * c + 3]};
        *reinterpret_cast<u32x4*>(lds + tok * G::LDS_ROW + off) = v;
    }
}

// The K and V operand slices back out of the wave's LDS rows (the same
// registers Tile holds when read directly), with the raw tile's scales and
// mask.
template <int HD, int MODE>
__device__ __forceinline__ void stage_read(const RawTile<HD, MODE>& R, const uint8_t* lds, int r, int q4,
                                           Tile<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
    const uint8_t* kp = lds + r * G::LDS_ROW + q4 * G::KB;
#pragma unroll
    for (int w = 0; w < G::KW; w += 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(kp + 4 * w);
        T.k[w] = v[0];
        T.k[w + 1] = v[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint8_t* vp = lds + (4 * q4 + i) * G::LDS_ROW + G::RB + ((r * G::VB) & ~(G::VL - 1));
#pragma unroll
        for (int w = 0; w < G::VW; ++w) T.v[i][w] = reinterpret_cast<const uint32_t*>(vp)[w];
        T.s[i] = R.s[i];
    }
    T.ok = R.ok;
}

template <int HD, int MODE>
__device__ __forceinline__ void unstage(const RawTile<HD, MODE>& R, uint8_t* lds, int r, int q4, Tile<HD, MODE>& T) {
    stage_write<HD, MODE>(R, lds, r, q4);
    stage_read<HD, MODE>(R, lds, r, q4, T);
}

// Staged tiles of 16 KiB (BF16 at head_dim 256) are written to LDS before the
// next tile's loads are issued: the raw registers of the tile in hand are then
// free when the next tile's loads take theirs, so one raw tile, not two, is
// live beside the operands.  Smaller tiles issue the next loads first.
template <int HD, int MODE>
constexpr bool attention_late_prefetch() {
    return Geo<HD, MODE>::NC > 8;
}

template <int HD, int MODE>
__device__ __forceinline__ void consume(const RawTile<HD, MODE>& T) {
#pragma unroll
    for (int w = 0; w < 4 * Geo<HD, MODE>::NC; ++w) asm volatile("" ::"v"(T.kv[w]));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if constexpr (Geo<HD, MODE>::DYN) asm volatile("" ::"v"(T.s[i][0]), "v"(T.s[i][1]));
}

// An empty use of every register of T, so that no load of T is moved past
// the point where the loop may exit.
template <int HD, int MODE>
__device__ __forceinline__ void consume(const Tile<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
#pragma unroll
    for (int w = 0; w < G::KW; ++w) asm volatile("" ::"v"(T.k[w]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int w = 0; w < G::VW; ++w) asm volatile("" ::"v"(T.v[i][w]));
        if constexpr (G::DYN) asm volatile("" ::"v"(T.s[i][0]), "v"(T.s[i][1]));
    }
}

template <int HD, int MODE>
struct State {
    f32x4 o[Geo<HD, MODE>::J];     // O^T[dim slot 4q+i][head r], one per 16-dim tile
    f32x4 vb;                      // INT4: (8 / 16) sum_t P'_t of head r, the bias of the biased values
    float m;                       // running maximum of head r (log2 domain)
    float l;                       // this lane's share of the running sum
};

// The lane's query slice as the Q K^T B operand: BF16 values, or (QF8) the
// FP8 E4M3 codes of the query under its head's static scale.
template <int HD, bool QF8>
struct QOperand {
    bf16x8 b[HD / 32];
};
template <int HD>
struct QOperand<HD, true> {
    uint32_t c[HD / 16];           // hd/4 codes, 4 per dword, in slice order
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Q K^T of one tile: with BF16 queries the codes are widened to BF16 and go
// through the 16x16x32 BF16 product; with FP8 queries the FP8 codes of both
// go straight into the FP8 products (16x16x128 at head_dim 128 and 256,
// 16x16x32 at 64), whose products are exact, as the BF16 ones are.  Both
// operands hold the same contiguous slice of dims in every lane, so the
// hardware's order of k within a lane does not matter.
template <int HD, int MODE, bool QF8>
__device__ __forceinline__ f32x4 qk_product(const uint32_t* k, const QOperand<HD, QF8>& q, f32x4 acc) {
    if constexpr (!QF8) {
#pragma unroll
        for (int j = 0; j < HD / 32; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<HD, MODE>(k, j), q.b[j], acc, 0, 0, 0);
    } else if constexpr (HD == 64) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const long a = static_cast<long>((static_cast<uint64_t>(k[2 * j + 1]) << 32) | k[2 * j]);
            const long b = static_cast<long>((static_cast<uint64_t>(q.c[2 * j + 1]) << 32) | q.c[2 * j]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc, 0, 0, 0);
        }
    } else {
        // format 0 (E4M3) for both operands, block scales 2^0 (E8M0 127)
#pragma unroll
        for (int j = 0; j < HD / 128; ++j) {
            const i32x8 a = {static_cast<int>(k[8 * j]), static_cast<int>(k[8 * j + 1]), static_cast<int>(k[8 * j + 2]),
                             static_cast<int>(k[8 * j + 3]), static_cast<int>(k[8 * j + 4]), static_cast<int>(k[8 * j + 5]),
                             static_cast<int>(k[8 * j + 6]), static_cast<int>(k[8 * j + 7])};
            const i32x8 b = {static_cast<int>(q.c[8 * j]), static_cast<int>(q.c[8 * j + 1]), static_cast<int>(q.c[8 * j + 2]),
                             static_cast<int>(q.c[8 * j + 3]), static_cast<int>(q.c[8 * j + 4]), static_cast<int>(q.c[8 * j + 5]),
                             static_cast<int>(q.c[8 * j + 6]), static_cast<int>(q.c[8 * j + 7])};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
        }
    }
    return acc;
}

// The BF16 query slice in the order of the biased INT4 key operand: each k
// step's elements (0, 1, ..., 7) become (0, 2, 4, 6, 1, 3, 5, 7).
template <int HD>
__device__ __forceinline__ void int4_query_order(QOperand<HD, false>& q) {
#pragma unroll
    for (int j = 0; j < HD / 32; ++j) {
        const u32x4 w = __builtin_bit_cast(u32x4, q.b[j]);
        const u32x4 o = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                         __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
        q.b[j] = __builtin_bit_cast(bf16x8, o);
    }
}

// Minus the bias of the biased INT4 keys, (8 / 16) sum(q) for each query
// column, through the same products with every key element -1/2 (negated
// products sum to the exact negation, and the loop then reuses the
// accumulator as it stands): the initial accumulator of each tile's Q K^T
// product.
template <int HD>
__device__ __forceinline__ f32x4 int4_key_bias(const QOperand<HD, false>& q) {
    const u32x4 halves = {0xBF00BF00u, 0xBF00BF00u, 0xBF00BF00u, 0xBF00BF00u};   // BF16 -0.5
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < HD / 32; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, halves), q.b[j], acc, 0, 0, 0);
    return acc;
}

// One round of the online softmax over NT consecutive tiles (16 NT tokens):
// the tiles' Q K^T products, one running-maximum update, then their P V
// products.  MASK = false is the path of rounds whose tokens all lie below
// len in blocks of the layer (a wave-uniform fact).
template <int HD, int MODE, int NT, bool MASK, bool QF8, bool PACK>
__device__ __forceinline__ void tile_round(const Tile<HD, MODE>* const* T, State<HD, MODE>& st,
                                           const QOperand<HD, QF8>& qo, f32x4 qk_init, int t0, int len, int r,
                                           int q4, float k_factor, uint32_t vsh, uint32_t vsel) {
    using G = Geo<HD, MODE>;
    f32x4 sacc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) sacc[n] = qk_product<HD, MODE, QF8>(T[n]->k, qo, qk_init);

    bool valid[NT][4];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            valid[n][i] = !MASK || ((t0 + kTile * n + 4 * q4 + i < len) && ((T[n]->ok >> i) & 1u));

    float alpha;
    s16x4 b[NT];
    if constexpr (PACK) {
        static_assert(NT == 2, "two tiles share the 16 columns");
        // Lanes r < 8 hold tile 0's columns; lanes r >= 8 hold tile 1's,
        // whose column c moves from lane c to lane c + 8 (DPP row_shr:8).
        // Each score, weight and sum is the one the unpacked round computes;
        // only the lanes of unused columns are no longer spent on them.
        const bool hi = r >= 8;
        float s[4], fv[4];
        bool vl[4];
        float lmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s1 = __uint_as_float(dpp<0x118>(__float_as_uint(sacc[1][i])));
            vl[i] = hi ? valid[1][i] : valid[0][i];
            const float f = G::DYN ? (hi ? T[1]->s[i][0] : T[0]->s[i][0]) * k_factor : k_factor;
            fv[i] = G::DYN ? (hi ? T[1]->s[i][1] : T[0]->s[i][1]) : 1.0f;
            s[i] = vl[i] ? (hi ? s1 : sacc[0][i]) * f : -INFINITY;
            lmax = fmaxf(lmax, s[i]);
        }
        float tmax = max_q4(lmax);
        tmax = fmaxf(tmax, __uint_as_float(dpp<0x128>(__float_as_uint(tmax))));   // row_ror:8: both tiles
        const float mnew = fmaxf(st.m, tmax);
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        alpha = __builtin_amdgcn_exp2f(st.m - mref);
        float p[4], pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[i] - mref);
            pv[i] = vl[i] ? (G::DYN ? p[i] * fv[i] : p[i]) : 0.0f;
        }
        st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        st.m = mnew;
        const u32x2 pb = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
        b[0] = __builtin_bit_cast(s16x4, pb);
        // tile 1's weights back to their columns (DPP row_shl:8)
        const u32x2 pb1 = {dpp<0x108>(pb[0]), dpp<0x108>(pb[1])};
        b[1] = __builtin_bit_cast(s16x4, pb1);
    } else {
        float s[NT][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = G::DYN ? T[n]->s[i][0] * k_factor : k_factor;
                s[n][i] = valid[n][i] ? sacc[n][i] * f : -INFINITY;
                tmax = fmaxf(tmax, s[n][i]);
            }
        tmax = max_q4(tmax);
        const float mnew = fmaxf(st.m, tmax);
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        alpha = __builtin_amdgcn_exp2f(st.m - mref);
        float psum = 0.0f;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float p[4], pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(s[n][i] - mref);
                pv[i] = valid[n][i] ? (G::DYN ? p[i] * T[n]->s[i][1] : p[i]) : 0.0f;
            }
            psum += (p[0] + p[1]) + (p[2] + p[3]);
            const u32x2 pb = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
            b[n] = __builtin_bit_cast(s16x4, pb);
        }
        st.l = st.l * alpha + psum;
        st.m = mnew;
    }

    constexpr bool I4 = MODE == KVQ_INT4_PER_TOKEN_HEAD;
    s16x4 av[NT][G::J];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if constexpr (I4) {
            v_operands_int4<HD>(T[n]->v, vsel, av[n]);
        } else {
            // masked tokens may hold any bytes (NaN codes included): zero them
            uint32_t vz[4][G::VW];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int w = 0; w < G::VW; ++w)
                    vz[i][w] = valid[n][i] ? (G::VB == 2 ? T[n]->v[i][w] >> vsh : T[n]->v[i][w]) : 0u;
            v_operands<HD, MODE>(vz, av[n]);
        }
    }
    // once the running maxima settle, alpha is 1 in every lane: skip the rescale
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] *= alpha;
        if constexpr (I4) st.vb *= alpha;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int j = 0; j < G::J; ++j)
            st.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[n][j], b[n], st.o[j], 0, 0, 0);
        if constexpr (I4) st.vb = int4_value_bias(b[n], st.vb);
    }
}

template <int HD, int MODE, bool SMALL_BS, bool QF8, bool PACK>
__global__ void __launch_bounds__(kMaxAttnThreads, attention_waves<HD>()) attention_kernel(AttnArgs a) {
    using G = Geo<HD, MODE>;
    // Workgroup -> work item, spreading consecutive items over one XCD
    // (workgroups are dealt to the 8 XCDs round robin).
    const uint32_t p = blockIdx.x;
    const uint32_t xcd = p % 8u, slot = p / 8u;
    const uint32_t per = a.total_wg / 8u, rem = a.total_wg % 8u;
    uint32_t item = xcd * per + min(xcd, rem) + slot;
    const int qg = static_cast<int>(item % static_cast<uint32_t>(a.qgroups));
    item /= static_cast<uint32_t>(a.qgroups);
    const int chunk = static_cast<int>(item % static_cast<uint32_t>(a.head_chunks));
    item /= static_cast<uint32_t>(a.head_chunks);
    const int split = static_cast<int>(item % static_cast<uint32_t>(a.splits));
    const int b = static_cast<int>(item / static_cast<uint32_t>(a.splits));

    const int lane = threadIdx.x & 63;
    const int h = chunk * a.heads_per_wg + static_cast<int>(threadIdx.x >> 6);
    const int r = lane & 15, q4 = lane >> 4;

    const int len = max(0, min(a.seq_lens[b], a.max_len));
    const int ntiles = (len + kTile - 1) / kTile;
    const int tbeg = split * a.tiles_per_split;
    const int tend = min(ntiles, tbeg + a.tiles_per_split);
    if (a.splits > 1 && tbeg >= tend) return;      // the combine reads only non-empty splits

    // query head of this lane's column
    const int gi = qg * 16 + r;
    const bool qvalid = gi < a.group;
    const int qh = h * a.group + (qvalid ? gi : 0);
    QOperand<HD, QF8> qo;
    float q_factor = 1.0f;
    {
        const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.num_q_heads + qh) * HD + q4 * (HD / 4);
        if constexpr (!QF8) {
#pragma unroll
            for (int j = 0; j < G::KSTEPS; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const u32x4 w = {v.x, v.y, v.z, v.w};
                qo.b[j] = __builtin_bit_cast(bf16x8, w);
            }
        } else {
            // E4M3(RN32(q / s_q)), saturating, exactly as the cache encodes K
            q_factor = qvalid ? a.q_scales[qh] : 1.0f;
            const RowQ rq = row_prep(q_factor);
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const uint2 c = encode_fp8<true, true>(v, rq);
                qo.c[2 * j] = c.x;
                qo.c[2 * j + 1] = c.y;
            }
        }
    }

    // biased INT4 keys: the query in their element order, and the bias out
    f32x4 qk_init = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD && !QF8) {
        int4_query_order<HD>(qo);
        qk_init = int4_key_bias<HD>(qo);
    }

    // INT4 operands are n / 16 (v_cvt_off_f32_i4): the factor 16 is applied
    // once to the scores' factor and once to the output, never per token
    float k_factor = a.c * G::CODE_UNIT * q_factor;
    float v_factor = G::CODE_UNIT;
    if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
        k_factor *= a.statics[0];
        v_factor = a.statics[1];
    } else if constexpr (MODE == KVQ_FP8_PER_HEAD) {
        k_factor *= a.statics[h];
        v_factor = a.statics[a.hkv + h];
    }
    if constexpr (PACK) {
        // lanes r >= 8 score column r - 8 (of the round's second tile): they
        // take that column's factor, which differs per column with FP8 queries
        const float kf = __uint_as_float(dpp<0x118>(__float_as_uint(k_factor)));
        if (r >= 8) k_factor = kf;
    }

    State<HD, MODE> st;
#pragma unroll
    for (int j = 0; j < G::J; ++j) st.o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.vb = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.m = -INFINITY;
    st.l = 0.0f;

    const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
    if (tbeg < tend) {
        // Rounds of NT tiles, D tiles in flight: while a round is computed,
        // the loads of the next D - NT tiles are outstanding.  The loop runs
        // whole passes of D tiles; tiles at or past the split's end are fully
        // masked (they take no part) and their loads re-read the last tile,
        // so no loop exit falls between a load and its use, and the
        // prefetches still pending at the exit are consumed there.
        // a packed round at head_dim 128 keeps four tiles in flight
        constexpr int D = (PACK && HD == 128) ? 4 : attention_depth<HD, MODE>();
        constexpr int NT = attention_round<HD, MODE, PACK>();
        static_assert(D % NT == 0 && D > NT, "whole rounds, at least one round in flight");
        const int lim = min(len, tend * kTile);
        const int last = tend - 1;
        auto block_of = [&](int tau) { return SMALL_BS ? 0 : bt_row[(tau * kTile) >> a.bs_log2]; };
        const LaneOff lo = lane_offsets<HD, MODE>(a, h, r, q4);
        constexpr bool STAGE = attention_staged<HD, MODE>() && !SMALL_BS;
        using InFlight = typename std::conditional<STAGE, RawTile<HD, MODE>, Tile<HD, MODE>>::type;
        // each wave's own LDS rows for the regrouping of staged tiles, in
        // dynamic LDS sized by the launch for the workgroup's waves (a
        // workgroup of fewer KV heads then leaves room for more workgroups)
        extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
        uint8_t* lds = lds_dyn + (STAGE ? (threadIdx.x >> 6) * Geo<HD, MODE>::LDS_TILE : 0);
        auto load = [&](int blk, int tau, InFlight& x) {
            if constexpr (STAGE) load_raw<HD, MODE>(a, blk, tau, lo, x);
            else load_tile<HD, MODE, SMALL_BS>(a, bt_row, blk, h, tau, r, q4, lo, x);
        };
        InFlight t[D];
        // (in tile order, so that the loop's waits for the oldest tile also
        // hold on entry)
#pragma unroll
        for (int k = 0; k < D - NT; ++k) {
            load(block_of(min(tbeg + k, last)), min(tbeg + k, last), t[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        int nb = block_of(min(tbeg + D - NT, last));
        // (the scheduling barriers keep each prefetch ahead of the arithmetic)
        for (int tau = tbeg; tau < tend; tau += D) {
#pragma unroll
            for (int k = 0; k < D; k += NT) {
                constexpr bool LATE = STAGE && attention_late_prefetch<HD, MODE>();
                static_assert(!LATE || NT == 1, "a late prefetch stages one tile per round");
                if constexpr (LATE) stage_write<HD, MODE>(t[k], lds, r, q4);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    load(nb, min(tau + k + D - NT + n, last), t[(k + D - NT + n) % D]);
                    nb = block_of(min(tau + k + D - NT + n + 1, last));
                }
                __builtin_amdgcn_sched_barrier(0);
                Tile<HD, MODE> staged[STAGE ? NT : 1];
                const Tile<HD, MODE>* rt[NT];
                bool all_ok = true;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if constexpr (LATE) {
                        stage_read<HD, MODE>(t[k + n], lds, r, q4, staged[n]);
                        rt[n] = &staged[n];
                    } else if constexpr (STAGE) {
                        unstage<HD, MODE>(t[k + n], lds, r, q4, staged[n]);
                        rt[n] = &staged[n];
                    } else {
                        rt[n] = &t[k + n];
                    }
                    all_ok = all_ok && t[k + n].ok != 0;
                }
                const int t0 = (tau + k) * kTile;
                if (attention_fast_path<HD>() && !SMALL_BS && t0 + NT * kTile <= lim && all_ok)
                    tile_round<HD, MODE, NT, false, QF8, PACK>(rt, st, qo, qk_init, t0, lim, r, q4, k_factor, lo.vsh,
                                                               lo.vsel);
                else
                    tile_round<HD, MODE, NT, true, QF8, PACK>(rt, st, qo, qk_init, t0, lim, r, q4, k_factor, lo.vsh,
                                                              lo.vsel);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int k = 0; k < D - NT; ++k) consume(t[k]);
    }

    float l = sum_q4(st.l);
    if constexpr (PACK) l += __uint_as_float(dpp<0x128>(__float_as_uint(l)));   // + the other tile's lanes
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
        // the biased values' excess, the same in every dim of head r
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] -= st.vb;
    }
    // lane holds dims J*(4*q4 + i) + j, i < 4, j < J: hd/4 contiguous dims
    const int64_t row = static_cast<int64_t>(b) * a.num_q_heads + qh;
    if (a.splits == 1) {
        if (!qvalid) return;
        const float inv = l > 0.0f ? v_factor / l : 0.0f;
        uint16_t* op = a.out + row * HD + q4 * (HD / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[G::J / 2];
#pragma unroll
            for (int j = 0; j < G::J; j += 2) w[j / 2] = pack_bf16(st.o[j][i] * inv, st.o[j + 1][i] * inv);
            uint16_t* dst = op + i * G::J;
            if constexpr (G::J >= 8) {
#pragma unroll
                for (int k = 0; k < G::J / 8; ++k) st16<false>(dst + 8 * k, make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]));
            } else {
                st8<false>(dst, make_uint2(w[0], w[1]));
            }
        }
    } else {
        if (!qvalid) return;
        const int64_t prow = row * a.splits + split;
        float* op = a.part_o + prow * HD + q4 * (HD / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < G::J; j += 4) {
                const uint4 w = make_uint4(__float_as_uint(st.o[j][i] * v_factor), __float_as_uint(st.o[j + 1][i] * v_factor),
                                           __float_as_uint(st.o[j + 2][i] * v_factor),
                                           __float_as_uint(st.o[j + 3][i] * v_factor));
                st16<false>(op + i * G::J + j, w);
            }
        }
        if (q4 == 0) {
            const u32x2 ml = {__float_as_uint(st.m), __float_as_uint(l)};
            *reinterpret_cast<u32x2*>(a.part_ml + prow * 2) = ml;
        }
    }
}

// ------------------------------------------------------ the quad kernel
//
// Query groups of at most 4 heads fill at most 4 of the 16 MFMA columns of
// a KV head's products, so the per-tile softmax would run on 12 idle
// columns.  Here a wave serves a quad of 4 KV heads at once: column r is
// query g = r % 4 of KV head h0 + r / 4.  The Q K^T product of a tile runs
// each of the quad's 4 heads' keys (the A operand) against all 16 query
// columns into an accumulator of its own, and each column then selects its
// own head's scores (3 selects per score); the P V product takes each
// head's values with the weights of that head's columns only (the others
// zero).  The softmax then runs once per tile for all 16 columns.
//
// The grid, the plan and the partial results are those of attention_kernel:
// a workgroup still covers a run of heads_per_wg (4 or 8) KV heads of one
// sequence over one split, with one wave per KV head; here its waves are
// heads_per_wg / 4 quads times 4 waves, and the 4 waves of a quad take every
// fourth tile of the split (interleaved, so the workgroup streams adjacent
// tiles), then merge their (O, m, l) through LDS before the output.
//
// Used for per-token-head layers: FP8 at head_dim 64 (BF16 or FP8
// queries) and INT4 at head_dim 64 and 128 (tiles of 4 or 8 KiB per quad),
// with blocks of at least 16 tokens and query groups of at most 4.  With FP8 queries the Q K^T product takes the
// raw K codes and block-diagonal FP8 query codes (FP8 zero in the other
// heads' columns) through the FP8 MFMA, whose products are exact.
template <int HD, int MODE>
struct QuadGeo {
    using G = Geo<HD, MODE>;
    static constexpr int QROW = 4 * 2 * G::RB;            // a position's K|V rows of the quad's 4 heads
    static constexpr int NC = 16 * QROW / 1024;            // 16-byte pieces per lane of a tile
    static constexpr int TPP = 1024 / QROW;                // tokens per 1 KiB piece
    static_assert(QROW <= 1024 && 1024 % QROW == 0, "whole tokens per 1 KiB piece");
    static constexpr int LDS_ROW = QROW + 16;
    static constexpr int LDS_TILE = 16 * LDS_ROW;
    static constexpr int MERGE = 64 * (2 + 4 * G::J) * 4;  // a wave's (m, l, O) for the merge
    static constexpr int LDS_WAVE = LDS_TILE > MERGE ? LDS_TILE : MERGE;
    static constexpr int D = NC <= 4 ? 3 : 2;              // tiles in flight per wave
    // Q K^T by per-head accumulators and a select at head_dim 128, where the
    // block-diagonal query operands (4 x HD / 32 registers of 4) would not
    // fit beside the tiles; at head_dim 64 the block-diagonal single chain
    // measured 11% (INT4) and 2% (FP8) faster than the select
    static constexpr bool SELECT = HD >= 128;
};

template <int HD, int MODE>
constexpr bool attention_quads() {
    // The per-token-head layouts only: a static layer's softmax has no
    // per-token scales to apply, and there the packed rounds of
    // attention_kernel measured 1.2-1.4% faster at head_dim 64 (BF16 and FP8
    // queries alike).  FP8 at head_dim 128 (16 KiB quad tiles) is bound by
    // memory already.
    return (MODE == KVQ_FP8_PER_TOKEN_HEAD && HD == 64) ||
           (MODE == KVQ_INT4_PER_TOKEN_HEAD && (HD == 64 || HD == 128));
}

// The layers the tile quads serve (workgroups of one or two KV heads): the
// head quads' layers, and FP8 per-token-head at head_dim 128 (two heads,
// as a pair).
template <int HD, int MODE>
constexpr bool attention_tquads() {
    return attention_quads<HD, MODE>() || (MODE == KVQ_FP8_PER_TOKEN_HEAD && HD == 128);
}

// the host's choice of kernel (attention_kind, which sizes the plan) names
// only kernels this file instantiates
template <int MODE>
constexpr bool attention_kind_matches() {
    return ((attention_kind(MODE, 64, 4, 16, 8, false) == kAttnHeadQuads) == attention_quads<64, MODE>()) &&
           ((attention_kind(MODE, 128, 4, 16, 8, false) == kAttnHeadQuads) == attention_quads<128, MODE>()) &&
           ((attention_kind(MODE, 256, 4, 16, 8, false) == kAttnHeadQuads) == attention_quads<256, MODE>()) &&
           ((attention_kind(MODE, 64, 4, 16, 2, false) == kAttnTileQuads) == attention_tquads<64, MODE>()) &&
           ((attention_kind(MODE, 128, 4, 16, 2, false) == kAttnTileQuads) == attention_tquads<128, MODE>()) &&
           ((attention_kind(MODE, 256, 4, 16, 1, false) == kAttnTileQuads) == attention_tquads<256, MODE>()) &&
           attention_kind(MODE, 128, 4, 16, 8, true) == kAttnOneHead;
}
static_assert(attention_kind_matches<KVQ_BF16>() && attention_kind_matches<KVQ_FP8_PER_TENSOR>() &&
                  attention_kind_matches<KVQ_FP8_PER_HEAD>() && attention_kind_matches<KVQ_FP8_PER_TOKEN_HEAD>() &&
                  attention_kind_matches<KVQ_INT4_PER_TOKEN_HEAD>(),
              "attention_kind and attention_quads agree");

template <int HD, int MODE>
struct QuadRaw {
    uint32_t kv[4 * QuadGeo<HD, MODE>::NC];
    f32x2 s[4];                    // (s_K, s_V) of tokens 4q+i, KV head h0 + r / 4
    uint32_t ok;
};

// The query operands of a quad's 16 columns: BF16 (the lane's own, for the
// per-head select, or 4 block-diagonal copies), or FP8 codes in 4
// block-diagonal copies.
template <int HD, int MODE, bool QF8>
struct QuadQuery {
    static constexpr int N = QuadGeo<HD, MODE>::SELECT ? HD / 32 : 4 * (HD / 32);
    bf16x8 b[N];
};
template <int HD, int MODE>
struct QuadQuery<HD, MODE, true> {
    uint32_t c[4 * (HD / 16)];
};

// A quad tile's row image is QROW <= 1024 bytes per token, so 1 KiB piece c
// of the tile starts TPP = 1024 / QROW tokens after piece c - 1: the lane's
// byte offset of piece c is its offset in piece 0 plus a wave-uniform step.
struct QuadLaneOff {
    uint32_t kv;                   // the lane's 16 bytes of piece 0 in the block
    uint32_t lds;                  // ... and where they go in the wave's LDS rows
    int kv_step;                   // block bytes from one piece to the next (uniform)
    uint32_t s[4];                 // (s_K, s_V) of tokens 4q+i for the lane's column head
};

template <int HD, int MODE>
__device__ __forceinline__ void quad_load(const AttnArgs& a, int blk, int tau, const QuadLaneOff& lo,
                                          QuadRaw<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
    using Q = QuadGeo<HD, MODE>;
    const bool ok = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks);
    const uint32_t ublk = ok ? static_cast<uint32_t>(blk) : 0u;
    const uint32_t pos0 = static_cast<uint32_t>((tau * kTile) & ((1 << a.bs_log2) - 1));
    const uint8_t* base = a.layer + static_cast<uint64_t>(ublk) * static_cast<uint64_t>(a.block_bytes);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base), 0, static_cast<int>(a.block_bytes), kBufferDword3);
    const int srow = static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * (2 * G::RB));
#pragma unroll
    for (int c = 0; c < Q::NC; ++c) buf_load<16, kNonTemporal>(T.kv + 4 * c, rs, lo.kv, srow + c * lo.kv_step);
    if constexpr (G::DYN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[2];
            buf_load<8, 0>(w, rs, lo.s[i], static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * 8u));
            T.s[i] = f32x2{__uint_as_float(w[0]), __uint_as_float(w[1])};
        }
    }
    T.ok = ok ? 0xFu : 0u;
}

template <int HD, int MODE>
__device__ __forceinline__ void consume(const QuadRaw<HD, MODE>& T) {
#pragma unroll
    for (int w = 0; w < 4 * QuadGeo<HD, MODE>::NC; ++w) asm volatile("" ::"v"(T.kv[w]));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if constexpr (Geo<HD, MODE>::DYN) asm volatile("" ::"v"(T.s[i][0]), "v"(T.s[i][1]));
}

// Head h's K slice of token r for the lane (hd / 4 dims from q4 * hd / 4)
// out of the wave's LDS rows.
template <int HD, int MODE>
__device__ __forceinline__ void quad_keys(const uint8_t* lds, int r, int q4, int h, uint32_t* k) {
    using G = Geo<HD, MODE>;
    using Q = QuadGeo<HD, MODE>;
    const uint8_t* kp = lds + r * Q::LDS_ROW + h * 2 * G::RB + q4 * G::KB;
#pragma unroll
    for (int w = 0; w < G::KW; w += 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(kp + 4 * w);
        k[w] = v[0];
        k[w + 1] = v[1];
    }
}

// One tile of the quad: scores of all 16 columns, one softmax update, the
// 4 heads' value products.  MASK = false: every token of the tile lies below
// len in a block of the layer.
// TILES: the 4 column groups are 4 / HPR consecutive tiles of HPR adjacent
// KV heads (group h: tile t0 / 16 + h / HPR, its block's bit h / HPR of R.ok,
// head h % HPR) instead of 4 heads of one tile (every bit of R.ok the same).
template <int HD, int MODE, bool MASK, bool QF8, bool TILES = false, int HPR = 1>
__device__ __forceinline__ void quad_round(const QuadRaw<HD, MODE>& R, const uint8_t* lds, State<HD, MODE>& st,
                                           const QuadQuery<HD, MODE, QF8>& qq, f32x4 qk_init, int t0, int len, int r,
                                           int q4, float k_factor, uint32_t vsh, uint32_t vsel) {
    using G = Geo<HD, MODE>;
    using Q = QuadGeo<HD, MODE>;
    constexpr bool I4 = MODE == KVQ_INT4_PER_TOKEN_HEAD;
    const int hq = r >> 2;
    // token tok of column group h's tile in a TILES round lies in the range,
    // in a block of the layer
    auto tile_token_ok = [&](int h, int tok) {
        return !MASK || ((t0 + kTile * (h / HPR) + tok < len) && ((R.ok >> (h / HPR)) & 1u));
    };
    f32x4 sacc;
    if constexpr (QF8) {
        // FP8 queries: each head's raw K codes against its block-diagonal
        // query codes (zero codes in the other heads' columns), 2 FP8
        // products of 32 dims per head, one accumulator
        static_assert(HD == 64, "FP8-query quads at head_dim 64");
        sacc = qk_init;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t k[G::KW];
            quad_keys<HD, MODE>(lds, r, q4, h, k);
            if constexpr (TILES && MASK && !I4) {
                // a stale FP8 key of tile h (NaN codes included) would reach
                // the other groups' columns through their zero queries
                if (!tile_token_ok(h, r))
#pragma unroll
                    for (int w = 0; w < G::KW; ++w) k[w] = 0u;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const long ka = static_cast<long>((static_cast<uint64_t>(k[2 * j + 1]) << 32) | k[2 * j]);
                const long qa = static_cast<long>((static_cast<uint64_t>(qq.c[h * 4 + 2 * j + 1]) << 32) |
                                                  qq.c[h * 4 + 2 * j]);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka, qa, sacc, 0, 0, 0);
            }
        }
    } else if constexpr (Q::SELECT) {
        // each head's keys against all 16 columns, into an accumulator of its
        // own; each column then takes its own head's scores
        f32x4 acc[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t k[G::KW];
            quad_keys<HD, MODE>(lds, r, q4, h, k);
            if constexpr (TILES && MASK && !I4) {
                // a stale FP8 key of tile h (NaN codes included) would reach
                // the other groups' columns through their zero queries
                if (!tile_token_ok(h, r))
#pragma unroll
                    for (int w = 0; w < G::KW; ++w) k[w] = 0u;
            }
            acc[h] = qk_init;
#pragma unroll
            for (int j = 0; j < HD / 32; ++j)
                acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<HD, MODE>(k, j), qq.b[j], acc[h], 0, 0, 0);
        }
        // two levels of per-lane selects on the bits of hq (a chain of
        // comparisons with hq compiled to divergent branches with copies:
        // 1.5-5% slower at head_dim 128)
        const bool odd = (hq & 1) != 0, upper = (hq & 2) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = odd ? acc[1][i] : acc[0][i];
            const float hi = odd ? acc[3][i] : acc[2][i];
            sacc[i] = upper ? hi : lo;
        }
    } else {
        // head by head into one accumulator, each head's query operand
        // holding only its own columns (block diagonal: qb[h * HD / 32 + j])
        sacc = qk_init;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t k[G::KW];
            quad_keys<HD, MODE>(lds, r, q4, h, k);
            if constexpr (TILES && MASK && !I4) {
                // a stale FP8 key of tile h (NaN codes included) would reach
                // the other groups' columns through their zero queries
                if (!tile_token_ok(h, r))
#pragma unroll
                    for (int w = 0; w < G::KW; ++w) k[w] = 0u;
            }
#pragma unroll
            for (int j = 0; j < HD / 32; ++j)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<HD, MODE>(k, j), qq.b[h * (HD / 32) + j],
                                                               sacc, 0, 0, 0);
        }
    }
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (TILES)
            valid[i] = tile_token_ok(hq, 4 * q4 + i);
        else
            valid[i] = !MASK || ((t0 + 4 * q4 + i < len) && ((R.ok >> i) & 1u));
    }
    float s[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float f = G::DYN ? R.s[i][0] * k_factor : k_factor;
        s[i] = valid[i] ? sacc[i] * f : -INFINITY;
        tmax = fmaxf(tmax, s[i]);
    }
    tmax = max_q4(tmax);
    const float mnew = fmaxf(st.m, tmax);
    const float mref = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mref);
    float p[4], pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - mref);
        pv[i] = valid[i] ? (G::DYN ? p[i] * R.s[i][1] : p[i]) : 0.0f;
    }
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m = mnew;
    const u32x2 pb = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] *= alpha;
        if constexpr (I4) st.vb *= alpha;
    }
    // P V, head by head: head h's values with the weights of its columns only
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        uint32_t v[4][G::VW];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t* vp = lds + (4 * q4 + i) * Q::LDS_ROW + (2 * h + 1) * G::RB + ((r * G::VB) & ~(G::VL - 1));
#pragma unroll
            for (int w = 0; w < G::VW; ++w) {
                const uint32_t x = reinterpret_cast<const uint32_t*>(vp)[w];
                // masked tokens may hold any bytes (NaN codes included): zero
                // them, except INT4, whose biased codes are all finite
                v[i][w] = (I4 || (TILES ? tile_token_ok(h, 4 * q4 + i) : valid[i])) ? x : 0u;
            }
        }
        s16x4 av[G::J];
        if constexpr (I4) {
            v_operands_int4<HD>(v, vsel, av);
        } else {
            if constexpr (G::VB == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int w = 0; w < G::VW; ++w) v[i][w] >>= vsh;
            }
            v_operands<HD, MODE>(v, av);
        }
        const u32x2 pbh = {hq == h ? pb[0] : 0u, hq == h ? pb[1] : 0u};
#pragma unroll
        for (int j = 0; j < G::J; ++j)
            st.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], __builtin_bit_cast(s16x4, pbh), st.o[j], 0, 0, 0);
    }
    if constexpr (I4) st.vb = int4_value_bias(__builtin_bit_cast(s16x4, pb), st.vb);
}

template <int HD, int MODE, bool QF8>
__global__ void __launch_bounds__(kMaxAttnThreads, 2) attention_quad_kernel(AttnArgs a) {
    using G = Geo<HD, MODE>;
    using Q = QuadGeo<HD, MODE>;
    // work item: as attention_kernel (qgroups is 1: groups of at most 4)
    const uint32_t p = blockIdx.x;
    const uint32_t xcd = p % 8u, slot = p / 8u;
    const uint32_t per = a.total_wg / 8u, rem = a.total_wg % 8u;
    uint32_t item = xcd * per + min(xcd, rem) + slot;
    const int chunk = static_cast<int>(item % static_cast<uint32_t>(a.head_chunks));
    item /= static_cast<uint32_t>(a.head_chunks);
    const int split = static_cast<int>(item % static_cast<uint32_t>(a.splits));
    const int b = static_cast<int>(item / static_cast<uint32_t>(a.splits));

    // (scalar: the tile indices, block ids and buffer descriptors derived
    // from it stay wave-uniform)
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int sr = wave & 3;                                   // the wave's share of the tiles
    const int h0 = chunk * a.heads_per_wg + (wave >> 2) * 4;   // the quad's first KV head
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const int hq = r >> 2, g = r & 3;
    const int hk = h0 + hq;                                    // the column's KV head

    const int len = max(0, min(a.seq_lens[b], a.max_len));
    const int ntiles = (len + kTile - 1) / kTile;
    const int tbeg = split * a.tiles_per_split;
    const int tend = min(ntiles, tbeg + a.tiles_per_split);
    if (a.splits > 1 && tbeg >= tend) return;      // (the whole workgroup) the combine reads only non-empty splits

    const bool qvalid = g < a.group;
    const int qh = hk * a.group + (qvalid ? g : 0);
    QOperand<HD, QF8> qo;
    float q_factor = 1.0f;
    {
        const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.num_q_heads + qh) * HD + q4 * (HD / 4);
        if constexpr (!QF8) {
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const u32x4 w = {v.x, v.y, v.z, v.w};
                qo.b[j] = __builtin_bit_cast(bf16x8, w);
            }
        } else {
            // E4M3(RN32(q / s_q)), saturating, exactly as the cache encodes K
            q_factor = qvalid ? a.q_scales[qh] : 1.0f;
            const RowQ rq = row_prep(q_factor);
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const uint2 c = encode_fp8<true, true>(v, rq);
                qo.c[2 * j] = c.x;
                qo.c[2 * j + 1] = c.y;
            }
        }
    }
    f32x4 qk_init = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD && !QF8) {
        int4_query_order<HD>(qo);
        qk_init = int4_key_bias<HD>(qo);
    }
    // the query operands: the lane's own (SELECT), or block-diagonal copies
    // in which head h's products see only its own columns
    QuadQuery<HD, MODE, QF8> qq;
    if constexpr (QF8) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int w = 0; w < HD / 16; ++w) qq.c[h * (HD / 16) + w] = hq == h ? qo.c[w] : 0u;
    } else {
        constexpr int NQB = QuadQuery<HD, MODE, false>::N;
#pragma unroll
        for (int h = 0; h < NQB / (HD / 32); ++h)
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const u32x4 w = __builtin_bit_cast(u32x4, qo.b[j]);
                const bool keep = Q::SELECT || hq == h;
                const u32x4 z = {keep ? w[0] : 0u, keep ? w[1] : 0u, keep ? w[2] : 0u, keep ? w[3] : 0u};
                qq.b[h * (HD / 32) + j] = __builtin_bit_cast(bf16x8, z);
            }
    }

    float k_factor = a.c * G::CODE_UNIT * q_factor;
    float v_factor = G::CODE_UNIT;
    if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
        k_factor *= a.statics[0];
        v_factor = a.statics[1];
    } else if constexpr (MODE == KVQ_FP8_PER_HEAD) {
        k_factor *= a.statics[hk];
        v_factor = a.statics[a.hkv + hk];
    }

    State<HD, MODE> st;
#pragma unroll
    for (int j = 0; j < G::J; ++j) st.o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.vb = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.m = -INFINITY;
    st.l = 0.0f;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    uint8_t* const lds = lds_dyn + wave * Q::LDS_WAVE;
    QuadLaneOff lo;
    {
        const uint32_t hkv = static_cast<uint32_t>(a.hkv), uh0 = static_cast<uint32_t>(h0);
        const uint32_t gb = static_cast<uint32_t>(lane) * 16u;
        const uint32_t tok = gb / Q::QROW, off = gb % Q::QROW;
        lo.kv = (tok * hkv + uh0) * (2 * G::RB) + off;
        lo.lds = tok * Q::LDS_ROW + off;
        lo.kv_step = Q::TPP * a.hkv * 2 * G::RB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo.s[i] = static_cast<uint32_t>(a.code_bytes) +
                      ((static_cast<uint32_t>(4 * q4 + i) * hkv + static_cast<uint32_t>(hk)) * 8u);
    }
    const uint32_t vsh = G::VB == 2 ? 16u * static_cast<uint32_t>(r & 1) : 0u;
    const uint32_t vsel = (r & 1) ? 0x07030602u : 0x05010400u;

    const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
    const int first = tbeg + sr;
    const int nt = first < tend ? (tend - first + 3) / 4 : 0;     // this wave's tiles: first, first + 4, ...
    if (nt > 0) {
        constexpr int D = Q::D;
        const int lim = min(len, tend * kTile);
        // tiles past the wave's last re-read the last (and are not used)
        auto tile_of = [&](int k) { return first + 4 * min(k, nt - 1); };
        auto block_of = [&](int k) { return bt_row[(tile_of(k) * kTile) >> a.bs_log2]; };
        QuadRaw<HD, MODE> t[D];
#pragma unroll
        for (int k = 0; k < D - 1; ++k) {
            quad_load<HD, MODE>(a, block_of(k), tile_of(k), lo, t[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        int nb = block_of(D - 1);
        for (int k0 = 0; k0 < nt; k0 += D) {
#pragma unroll
            for (int kk = 0; kk < D; ++kk) {
                const int k = k0 + kk;
                quad_load<HD, MODE>(a, nb, tile_of(k + D - 1), lo, t[(kk + D - 1) % D]);
                nb = block_of(k + D);
                __builtin_amdgcn_sched_barrier(0);
                if (k < nt) {
                    // the tile into the wave's LDS rows, then its operands back out
#pragma unroll
                    for (int c = 0; c < Q::NC; ++c) {
                        const u32x4 v = {t[kk].kv[4 * c], t[kk].kv[4 * c + 1], t[kk].kv[4 * c + 2], t[kk].kv[4 * c + 3]};
                        *reinterpret_cast<u32x4*>(lds + lo.lds + c * Q::TPP * Q::LDS_ROW) = v;
                    }
                    const int t0 = tile_of(k) * kTile;
                    if (t0 + kTile <= lim && t[kk].ok != 0)
                        quad_round<HD, MODE, false, QF8>(t[kk], lds, st, qq, qk_init, t0, lim, r, q4, k_factor, vsh,
                                                         vsel);
                    else
                        quad_round<HD, MODE, true, QF8>(t[kk], lds, st, qq, qk_init, t0, lim, r, q4, k_factor, vsh,
                                                        vsel);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int k = 0; k < D - 1; ++k) consume(t[k]);
    }

    float l = sum_q4(st.l);
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] -= st.vb;
    }
    // merge the quad's 4 waves: each writes (m, l, O) to its LDS, the first
    // of the quad rescales and adds the others' to its own
    __syncthreads();
    float* const mine = reinterpret_cast<float*>(lds_dyn + wave * Q::LDS_WAVE);
    mine[lane] = st.m;
    mine[64 + lane] = l;
#pragma unroll
    for (int j = 0; j < G::J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(2 + 4 * j + i) * 64 + lane] = st.o[j][i];
    __syncthreads();
    if (sr != 0) return;
    float m = st.m;
#pragma unroll
    for (int w = 1; w < 4; ++w) m = fmaxf(m, reinterpret_cast<const float*>(lds_dyn + (wave + w) * Q::LDS_WAVE)[lane]);
    const float mref = m == -INFINITY ? 0.0f : m;
    {
        const float f0 = __builtin_amdgcn_exp2f(st.m - mref);
        l *= f0;
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] *= f0;
    }
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const float* other = reinterpret_cast<const float*>(lds_dyn + (wave + w) * Q::LDS_WAVE);
        const float f = __builtin_amdgcn_exp2f(other[lane] - mref);
        l += f * other[64 + lane];
#pragma unroll
        for (int j = 0; j < G::J; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[j][i] += f * other[(2 + 4 * j + i) * 64 + lane];
    }
    st.m = m;
    // lane holds dims J*(4*q4 + i) + j of query head qh, as attention_kernel
    const int64_t row = static_cast<int64_t>(b) * a.num_q_heads + qh;
    if (!qvalid) return;
    if (a.splits == 1) {
        const float inv = l > 0.0f ? v_factor / l : 0.0f;
        uint16_t* op = a.out + row * HD + q4 * (HD / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[G::J / 2];
#pragma unroll
            for (int j = 0; j < G::J; j += 2) w[j / 2] = pack_bf16(st.o[j][i] * inv, st.o[j + 1][i] * inv);
            uint16_t* dst = op + i * G::J;
            if constexpr (G::J >= 8) {
#pragma unroll
                for (int k = 0; k < G::J / 8; ++k) st16<false>(dst + 8 * k, make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]));
            } else {
                st8<false>(dst, make_uint2(w[0], w[1]));
            }
        }
    } else {
        const int64_t prow = row * a.splits + split;
        float* op = a.part_o + prow * HD + q4 * (HD / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < G::J; j += 4) {
                const uint4 w = make_uint4(__float_as_uint(st.o[j][i] * v_factor), __float_as_uint(st.o[j + 1][i] * v_factor),
                                           __float_as_uint(st.o[j + 2][i] * v_factor),
                                           __float_as_uint(st.o[j + 3][i] * v_factor));
                st16<false>(op + i * G::J + j, w);
            }
        }
        if (q4 == 0) {
            const u32x2 ml = {__float_as_uint(st.m), __float_as_uint(l)};
            *reinterpret_cast<u32x2*>(a.part_ml + prow * 2) = ml;
        }
    }
}

// ------------------------------------------------ tile quads (few KV heads)
//
// A workgroup of fewer than 4 KV heads (one or two: a tensor-parallel shard,
// a multi-query model) has no quad of heads.  Here the 4 column groups of a
// wave are instead 4 consecutive tiles of one KV head: column r is query
// r % 4 against tile base + r / 4.  The products and the softmax are those
// of the head quads (quad_round with TILES): head h's role is taken by tile
// h of the round, each column group keeps its own running (m, l, O), and a
// round covers 64 tokens.  A workgroup holds WPH waves per KV head (4, or 8
// for INT4 on one KV head), which take every WPH-th round of the split; at
// the end each head's 4 * WPH partial states per query (waves x column
// groups) merge through LDS, every thread of the head merging its own dims.
// A workgroup of two KV heads runs them as a pair (HPR = 2): the column
// groups are 2 tiles x the 2 heads, a round covers 32 tokens of both, and
// the pair's 8 waves take every eighth round; both heads' K|V rows of a
// position are adjacent in the block, so a round's loads are whole runs.
//
// A round's row image is the 4 tiles' 16 K|V rows of the head side by side
// (row p: tiles 0..3 at position p), the same LDS layout as a head quad's
// tile, loaded as 1 KiB pieces of one tile each.  The per-token scales of a
// lane's tile come from that tile's block, so they are read by address
// rather than through a block's buffer descriptor.
template <int HD, int MODE, int HPR = 1>
struct TquadGeo {
    using G = Geo<HD, MODE>;
    static constexpr int TR = 2 * G::RB;                   // one token's K|V rows of one head
    static constexpr int UR = HPR * TR;                    // ... of the round's HPR adjacent heads
    static constexpr int TPR = 4 / HPR;                    // tiles per round
    static constexpr int PPT = kTile * UR / 1024;          // 1 KiB pieces per tile
    static constexpr int TPC = 1024 / UR;                  // tokens per piece
    static_assert(HPR == 1 || HPR == 2, "one head of 4 tiles or two heads of 2 tiles per round");
    static_assert(PPT >= 1 && PPT * TPR == QuadGeo<HD, MODE>::NC, "a round is TPR tiles of whole pieces");
};

struct TquadLaneOff {
    uint32_t kv;                   // the lane's 16 bytes of a tile's first piece
    uint32_t lds;                  // ... and where they go in the wave's LDS rows
    int kv_step;                   // block bytes from one piece of a tile to the next (uniform)
    uint32_t s;                    // (s_K, s_V) of token 4 q4 of the lane's tile, from its block
};

template <int HD, int MODE, int HPR>
__device__ __forceinline__ void tquad_load(const AttnArgs& a, const int (&blk)[4], const int (&tau)[4], int jt,
                                           const TquadLaneOff& lo, QuadRaw<HD, MODE>& T) {
    using G = Geo<HD, MODE>;
    using TQ = TquadGeo<HD, MODE, HPR>;
    const uint32_t pmask = (1u << a.bs_log2) - 1u;
    uint32_t ok = 0u;
    uint64_t lane_base = 0;
    uint32_t lane_pos0 = 0;
#pragma unroll
    for (int j = 0; j < TQ::TPR; ++j) {
        const bool okj = static_cast<uint32_t>(blk[j]) < static_cast<uint32_t>(a.num_blocks);
        ok |= okj ? (1u << j) : 0u;
        const uint32_t ublk = okj ? static_cast<uint32_t>(blk[j]) : 0u;
        const uint32_t pos0 = static_cast<uint32_t>(tau[j] * kTile) & pmask;
        const uint64_t boff = static_cast<uint64_t>(ublk) * static_cast<uint64_t>(a.block_bytes);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.layer + boff), 0, static_cast<int>(a.block_bytes), kBufferDword3);
        const int srow = static_cast<int>(pos0 * static_cast<uint32_t>(a.hkv) * TQ::TR);
#pragma unroll
        for (int pc = 0; pc < TQ::PPT; ++pc)
            buf_load<16, kNonTemporal>(T.kv + 4 * (j * TQ::PPT + pc), rs, lo.kv, srow + pc * lo.kv_step);
        lane_base = jt == j ? boff : lane_base;
        lane_pos0 = jt == j ? pos0 : lane_pos0;
    }
    if constexpr (G::DYN) {
        const uint8_t* sp = a.layer + lane_base + static_cast<uint64_t>(a.code_bytes) +
                            static_cast<uint64_t>(lane_pos0 * static_cast<uint32_t>(a.hkv) * 8u + lo.s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            T.s[i] = *reinterpret_cast<const f32x2*>(sp + static_cast<uint64_t>(i) * static_cast<uint32_t>(a.hkv) * 8u);
    }
    T.ok = ok;
}

template <int HD, int MODE, bool QF8, int WPH, int HPR>
__global__ void __launch_bounds__(kMaxAttnThreads, 2) attention_tquad_kernel(AttnArgs a) {
    using G = Geo<HD, MODE>;
    using Q = QuadGeo<HD, MODE>;
    using TQ = TquadGeo<HD, MODE, HPR>;
    // work item: as attention_kernel (qgroups is 1: groups of at most 4)
    const uint32_t p = blockIdx.x;
    const uint32_t xcd = p % 8u, slot = p / 8u;
    const uint32_t per = a.total_wg / 8u, rem = a.total_wg % 8u;
    uint32_t item = xcd * per + min(xcd, rem) + slot;
    const int chunk = static_cast<int>(item % static_cast<uint32_t>(a.head_chunks));
    item /= static_cast<uint32_t>(a.head_chunks);
    const int split = static_cast<int>(item % static_cast<uint32_t>(a.splits));
    const int b = static_cast<int>(item / static_cast<uint32_t>(a.splits));

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int sr = wave % WPH;                                 // the wave's share of the rounds
    const int hh0 = chunk * a.heads_per_wg + (wave / WPH) * HPR;   // the wave's first KV head
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const int hq = r >> 2, g = r & 3;                          // column group, query
    const int jt = hq / HPR;                                   // the group's tile of the round
    const int hh = hh0 + hq % HPR;                             // ... and KV head

    const int len = max(0, min(a.seq_lens[b], a.max_len));
    const int ntiles = (len + kTile - 1) / kTile;
    const int tbeg = split * a.tiles_per_split;
    const int tend = min(ntiles, tbeg + a.tiles_per_split);
    if (a.splits > 1 && tbeg >= tend) return;      // (the whole workgroup) the combine reads only non-empty splits

    const bool qvalid = g < a.group;
    const int qh = hh * a.group + (qvalid ? g : 0);
    QOperand<HD, QF8> qo;
    float q_factor = 1.0f;
    {
        const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.num_q_heads + qh) * HD + q4 * (HD / 4);
        if constexpr (!QF8) {
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const u32x4 w = {v.x, v.y, v.z, v.w};
                qo.b[j] = __builtin_bit_cast(bf16x8, w);
            }
        } else {
            // E4M3(RN32(q / s_q)), saturating, exactly as the cache encodes K
            q_factor = qvalid ? a.q_scales[qh] : 1.0f;
            const RowQ rq = row_prep(q_factor);
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const uint4 v = qvalid ? ld16<false>(qp + 8 * j) : make_uint4(0, 0, 0, 0);
                const uint2 c = encode_fp8<true, true>(v, rq);
                qo.c[2 * j] = c.x;
                qo.c[2 * j + 1] = c.y;
            }
        }
    }
    f32x4 qk_init = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD && !QF8) {
        int4_query_order<HD>(qo);
        qk_init = int4_key_bias<HD>(qo);
    }
    // query operands: tile h's products see only the columns of group h
    QuadQuery<HD, MODE, QF8> qq;
    if constexpr (QF8) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int w = 0; w < HD / 16; ++w) qq.c[h * (HD / 16) + w] = hq == h ? qo.c[w] : 0u;
    } else {
        constexpr int NQB = QuadQuery<HD, MODE, false>::N;
#pragma unroll
        for (int h = 0; h < NQB / (HD / 32); ++h)
#pragma unroll
            for (int j = 0; j < HD / 32; ++j) {
                const u32x4 w = __builtin_bit_cast(u32x4, qo.b[j]);
                const bool keep = Q::SELECT || hq == h;
                const u32x4 z = {keep ? w[0] : 0u, keep ? w[1] : 0u, keep ? w[2] : 0u, keep ? w[3] : 0u};
                qq.b[h * (HD / 32) + j] = __builtin_bit_cast(bf16x8, z);
            }
    }

    float k_factor = a.c * G::CODE_UNIT * q_factor;
    float v_factor = G::CODE_UNIT;
    if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
        k_factor *= a.statics[0];
        v_factor = a.statics[1];
    } else if constexpr (MODE == KVQ_FP8_PER_HEAD) {
        k_factor *= a.statics[hh];
        v_factor = a.statics[a.hkv + hh];
    }

    State<HD, MODE> st;
#pragma unroll
    for (int j = 0; j < G::J; ++j) st.o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.vb = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.m = -INFINITY;
    st.l = 0.0f;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    uint8_t* const lds = lds_dyn + wave * Q::LDS_WAVE;
    TquadLaneOff lo;
    {
        const uint32_t hkv = static_cast<uint32_t>(a.hkv);
        const uint32_t bl = static_cast<uint32_t>(lane) * 16u;
        const uint32_t tok = bl / TQ::UR, off = bl % TQ::UR;
        lo.kv = (tok * hkv + static_cast<uint32_t>(hh0)) * TQ::TR + off;
        lo.lds = tok * Q::LDS_ROW + off;
        lo.kv_step = TQ::TPC * a.hkv * TQ::TR;
        lo.s = (static_cast<uint32_t>(4 * q4) * hkv + static_cast<uint32_t>(hh)) * 8u;
    }
    const uint32_t vsh = G::VB == 2 ? 16u * static_cast<uint32_t>(r & 1) : 0u;
    const uint32_t vsel = (r & 1) ? 0x07030602u : 0x05010400u;

    const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
    const int nr = (tend - tbeg + TQ::TPR - 1) / TQ::TPR;          // rounds of TPR tiles in the split
    const int nt = sr < nr ? (nr - sr + WPH - 1) / WPH : 0;        // this wave's rounds: sr, sr + WPH, ...
    if (nt > 0) {
        constexpr int D = Q::D;
        const int lim = min(len, tend * kTile);
        // rounds past the wave's last re-read the last; tiles past the
        // split's end read its last tile (masked: their tokens lie at or past lim)
        auto base_of = [&](int k) { return tbeg + TQ::TPR * (sr + WPH * min(k, nt - 1)); };
        auto tiles_of = [&](int k, int (&tau)[4], int (&blk)[4]) {
            const int t = base_of(k);
#pragma unroll
            for (int j = 0; j < TQ::TPR; ++j) {
                tau[j] = min(t + j, tend - 1);
                blk[j] = bt_row[(tau[j] * kTile) >> a.bs_log2];
            }
        };
        QuadRaw<HD, MODE> t[D];
#pragma unroll
        for (int k = 0; k < D - 1; ++k) {
            int tau[4], blk[4];
            tiles_of(k, tau, blk);
            tquad_load<HD, MODE, HPR>(a, blk, tau, jt, lo, t[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int k0 = 0; k0 < nt; k0 += D) {
#pragma unroll
            for (int kk = 0; kk < D; ++kk) {
                const int k = k0 + kk;
                {
                    int tau[4], blk[4];
                    tiles_of(k + D - 1, tau, blk);
                    tquad_load<HD, MODE, HPR>(a, blk, tau, jt, lo, t[(kk + D - 1) % D]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (k < nt) {
                    // the round's tiles into the wave's LDS rows, side by side
#pragma unroll
                    for (int c = 0; c < Q::NC; ++c) {
                        const int j = c / TQ::PPT, pc = c % TQ::PPT;
                        const u32x4 v = {t[kk].kv[4 * c], t[kk].kv[4 * c + 1], t[kk].kv[4 * c + 2], t[kk].kv[4 * c + 3]};
                        *reinterpret_cast<u32x4*>(lds + lo.lds + pc * TQ::TPC * Q::LDS_ROW + j * TQ::UR) = v;
                    }
                    const int t0 = base_of(k) * kTile;
                    if (t0 + TQ::TPR * kTile <= lim && t[kk].ok == (1u << TQ::TPR) - 1u)
                        quad_round<HD, MODE, false, QF8, true, HPR>(t[kk], lds, st, qq, qk_init, t0, lim, r, q4,
                                                                    k_factor, vsh, vsel);
                    else
                        quad_round<HD, MODE, true, QF8, true, HPR>(t[kk], lds, st, qq, qk_init, t0, lim, r, q4,
                                                                   k_factor, vsh, vsel);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int k = 0; k < D - 1; ++k) consume(t[k]);
    }

    float l = sum_q4(st.l);
    if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
#pragma unroll
        for (int j = 0; j < G::J; ++j) st.o[j] -= st.vb;
    }
    // merge each head's 4 / HPR * WPH partial states of each query (the
    // round's WPH waves x its column groups of the head): each wave writes
    // (m, l, O) to its LDS, then every thread of the waves merges PER adjacent
    // output dims of one query of one head
    __syncthreads();
    float* const mine = reinterpret_cast<float*>(lds_dyn + wave * Q::LDS_WAVE);
    mine[lane] = st.m;
    mine[64 + lane] = l;
#pragma unroll
    for (int j = 0; j < G::J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(2 + 4 * j + i) * 64 + lane] = st.o[j][i];
    __syncthreads();
    constexpr int HT = 64 * WPH;                               // threads of the round's waves
    constexpr int OUTS = HPR * 4 * HD;                         // their outputs: heads x queries x dims
    constexpr int PER = OUTS > HT ? OUTS / HT : 1;             // output dims per thread
    static_assert(PER <= G::J && G::J % PER == 0, "a thread's dims share one source lane");
    const int t = sr * 64 + lane;
    if (t * PER >= OUTS) return;
    const int eh = t * PER / (4 * HD);                         // head of the round
    const int gq = t * PER % (4 * HD) / HD, d0 = t * PER % HD; // query of the group, first dim
    if (gq >= a.group) return;
    const int dq = d0 / G::J, jj = d0 % G::J;                  // source slots: i = dq % 4, j = jj + e
    const int src = (dq / 4) * 16 + 4 * eh + gq;               // lane of the head's first column group
    const float* const hw = reinterpret_cast<const float*>(lds_dyn + (wave - sr) * Q::LDS_WAVE);
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPH; ++w)
#pragma unroll
        for (int c = 0; c < TQ::TPR; ++c) m = fmaxf(m, hw[w * (Q::LDS_WAVE / 4) + src + 4 * HPR * c]);
    const float mref = m == -INFINITY ? 0.0f : m;
    float lsum = 0.0f;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.0f;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
        const float* const other = hw + w * (Q::LDS_WAVE / 4);
#pragma unroll
        for (int c = 0; c < TQ::TPR; ++c) {
            const int ln = src + 4 * HPR * c;                  // the head's column group of tile c
            const float f = __builtin_amdgcn_exp2f(other[ln] - mref);
            lsum += f * other[64 + ln];
#pragma unroll
            for (int e = 0; e < PER; ++e) o[e] += f * other[(2 + 4 * (jj + e) + dq % 4) * 64 + ln];
        }
    }
    const int64_t row = static_cast<int64_t>(b) * a.num_q_heads + (hh0 + eh) * a.group + gq;
    if (a.splits == 1) {
        const float inv = lsum > 0.0f ? v_factor / lsum : 0.0f;
        uint16_t* op = a.out + row * HD + d0;
        if constexpr (PER == 1) {
            *op = static_cast<uint16_t>(pack_bf16(o[0] * inv, 0.0f) & 0xFFFFu);
        } else {
            uint32_t w[PER / 2];
#pragma unroll
            for (int e = 0; e < PER; e += 2) w[e / 2] = pack_bf16(o[e] * inv, o[e + 1] * inv);
            if constexpr (PER == 2) st4<false>(op, w[0]);
            else st8<false>(op, make_uint2(w[0], w[1]));
        }
    } else {
        const int64_t prow = row * a.splits + split;
        float* op = a.part_o + prow * HD + d0;
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = o[e] * v_factor;
        if (d0 == 0) {
            const u32x2 ml = {__float_as_uint(m), __float_as_uint(lsum)};
            *reinterpret_cast<u32x2*>(a.part_ml + prow * 2) = ml;
        }
    }
}

// Combine of the splits' partial results: one wave per (sequence, query head).
struct CombineArgs {
    const float* part_o;
    const float* part_ml;
    const int32_t* seq_lens;
    uint16_t* out;
    int64_t rows;                  // num_seqs * H
    int32_t num_q_heads;
    int32_t splits;
    int32_t tiles_per_split;
    int32_t max_len;               // as in AttnArgs
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int k = 32; k > 0; k >>= 1) v = fmaxf(v, __shfl_xor(v, k, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int k = 32; k > 0; k >>= 1) v += __shfl_xor(v, k, 64);
    return v;
}

// A row's split count is small here (below kWideCombineSplits), so every
// load of the row is issued at once, together with the sequence length:
// lane s takes split s's (m, l), and each lane loads its dims of every
// planned split's O before the weights are known.  The merge is then one
// memory latency, not one per split.  Splits past the sequence's last hold
// stale workspace bytes: they are loaded (in bounds) but never used.  The
// loads take clamped indices rather than branches, so none waits on another.
template <int HD>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    constexpr int DPL = HD / 64;   // dims per lane
    constexpr int NS = kWideCombineSplits - 1;
    static_assert(NS <= 64, "one split per lane");
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int lane = threadIdx.x & 63;
    const int sp = min(a.splits, NS);                 // at least 2: a combine follows a split launch
    const f32x2 mlr = *reinterpret_cast<const f32x2*>(a.part_ml + (row * a.splits + min(lane, sp - 1)) * 2);
    const float* po = a.part_o + row * a.splits * HD + lane * DPL;
    float o[NS][DPL];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int sc = min(s, sp - 1);
        if constexpr (DPL == 1) {
            o[s][0] = po[sc * HD];
        } else if constexpr (DPL == 2) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(po + sc * HD);
            o[s][0] = v[0];
            o[s][1] = v[1];
        } else {
            const f32x4 v = *reinterpret_cast<const f32x4*>(po + sc * HD);
#pragma unroll
            for (int d = 0; d < 4; ++d) o[s][d] = v[d];
        }
    }
    const int b = static_cast<int>(row / a.num_q_heads);
    const int len = max(0, min(a.seq_lens[b], a.max_len));
    const int ntiles = (len + kTile - 1) / kTile;
    const int nsp = min((ntiles + a.tiles_per_split - 1) / a.tiles_per_split, sp);
    const f32x2 ml = lane < nsp ? mlr : f32x2{-INFINITY, 0.0f};
    const float M = wave_max(ml[0]);
    // lane s's weight; lanes past the last split weigh exp2(-inf) = 0
    const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[0] - M);
    const float L = wave_sum(w * ml[1]);
    float acc[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[d] = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float ws = __shfl(w, s, 64);
        if (s < nsp) {
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[d] += ws * o[s][d];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t* dst = a.out + row * HD + lane * DPL;
    if constexpr (DPL == 1) {
        dst[0] = static_cast<uint16_t>(pack_bf16(acc[0] * inv, 0.0f) & 0xFFFFu);
    } else {
        uint32_t wd[DPL / 2];
#pragma unroll
        for (int d = 0; d < DPL; d += 2) wd[d / 2] = pack_bf16(acc[d] * inv, acc[d + 1] * inv);
        if constexpr (DPL == 2) st4<false>(dst, wd[0]);
        else st8<false>(dst, make_uint2(wd[0], wd[1]));
    }
}

// The same combine with the splits spread over a workgroup, one workgroup
// per (sequence, query head): for long single sequences, whose few rows
// each carry hundreds of splits.  Thread t sums 4 dims (quad t % (HD/4)) of
// every (T / (HD/4))-th split; the loads of U such splits are in flight
// together, the first U (and the first T splits' (m, l)) issued with the
// sequence length's load, before anything is known of the row, so a row of
// up to U * T / (HD/4) splits costs one memory latency.  Splits past the
// sequence's last hold stale workspace bytes: loaded (in bounds, clamped
// indices), never used.  The weights go through LDS, the quads' sums too.
constexpr int kWideCombineThreads = 256;

template <int HD>
__global__ void __launch_bounds__(kWideCombineThreads) combine_wide_kernel(CombineArgs a) {
    constexpr int T = kWideCombineThreads;
    constexpr int NW = T / 64;
    constexpr int Q4 = HD / 4;         // 4-dim quads of a split's O
    constexpr int SPP = T / Q4;        // splits one pass of the workgroup covers
    constexpr int U = 8;               // passes whose loads are in flight together
    __shared__ float wts[kMaxSplits];
    __shared__ float red[2 * NW];
    __shared__ f32x4 part[T];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int sp = a.splits;
    const float* ml = a.part_ml + row * sp * 2;
    const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o + row * sp * HD);
    const int q = tid % Q4, s0 = tid / Q4;
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

    const f32x2 mlr = *reinterpret_cast<const f32x2*>(ml + 2 * min(tid, sp - 1));
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = po[min(s0 + SPP * u, sp - 1) * Q4 + q];
    const int b = static_cast<int>(row / a.num_q_heads);
    const int len = max(0, min(a.seq_lens[b], a.max_len));
    const int ntiles = (len + kTile - 1) / kTile;
    const int nsp = min((ntiles + a.tiles_per_split - 1) / a.tiles_per_split, sp);
    const f32x2 ml0 = tid < nsp ? mlr : f32x2{-INFINITY, 0.0f};
    float mx = ml0[0];
    for (int s = tid + T; s < nsp; s += T) mx = fmaxf(mx, ml[2 * s]);
    mx = wave_max(mx);
    if (lane == 0) red[wv] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
    float lsum = 0.0f;
    if (tid < nsp) {
        const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml0[0] - M);
        wts[tid] = w;
        lsum = w * ml0[1];
    }
    for (int s = tid + T; s < nsp; s += T) {
        const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[2 * s] - M);
        wts[s] = w;
        lsum += w * ml[2 * s + 1];
    }
    lsum = wave_sum(lsum);
    if (lane == 0) red[NW + wv] = lsum;
    __syncthreads();
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += red[NW + w];

    f32x4 acc = zero;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int s = s0 + SPP * u;
        if (s < nsp) acc += wts[s] * v[u];
    }
    for (int k0 = s0 + SPP * U; k0 < nsp; k0 += SPP * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = po[min(k0 + SPP * u, nsp - 1) * Q4 + q];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = k0 + SPP * u;
            if (s < nsp) acc += wts[s] * v[u];
        }
    }
    part[tid] = acc;
    __syncthreads();
    if (tid < Q4) {
        f32x4 sum = part[tid];
#pragma unroll
        for (int g = 1; g < SPP; ++g) sum += part[g * Q4 + tid];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        st8<false>(a.out + row * HD + 4 * tid,
                   make_uint2(pack_bf16(sum[0] * inv, sum[1] * inv), pack_bf16(sum[2] * inv, sum[3] * inv)));
    }
}

// Packed softmax rounds (two tiles per set of columns) where the query group
// leaves at least half of the columns free: at head_dim 64, where the
// per-tile softmax is the largest share of the instructions, and for INT4 at
// head_dim 128, whose widening makes it the most VALU-heavy case (+3.5%
// there; FP8 at head_dim 128 measured 0.7% slower).
template <int HD, int MODE>
constexpr bool attention_packs() {
    return HD == 64 || (HD == 128 && MODE == KVQ_INT4_PER_TOKEN_HEAD);
}

template <int HD, int MODE, bool QF8>
void launch_attention_q(const AttnArgs& p, int threads, bool small_bs, hipStream_t st) {
    // the plan's kind (attention_kind): head quads, with FP8 queries at
    // head_dim 64 only; tile quads with 4 waves per KV head
    if constexpr (attention_quads<HD, MODE>() && (!QF8 || HD == 64)) {
        if (p.kind == kAttnHeadQuads) {
            const unsigned qlds = static_cast<unsigned>(threads / 64) * QuadGeo<HD, MODE>::LDS_WAVE;
            hipLaunchKernelGGL((attention_quad_kernel<HD, MODE, QF8>), dim3(p.total_wg), dim3(threads), qlds, st, p);
            return;
        }
    }
    if constexpr (attention_tquads<HD, MODE>() && (!QF8 || HD == 64)) {
        if (p.kind == kAttnTileQuads) {
            const int wph = tquad_waves_per_head(MODE, p.heads_per_wg);
            const int tthreads = wph * threads;
            const unsigned qlds = static_cast<unsigned>(tthreads / 64) * QuadGeo<HD, MODE>::LDS_WAVE;
            if (tquad_head_pairs(p.heads_per_wg)) {
                // two KV heads of two tiles per round, the pair's 8 waves
                hipLaunchKernelGGL((attention_tquad_kernel<HD, MODE, QF8, 8, 2>), dim3(p.total_wg), dim3(tthreads),
                                   qlds, st, p);
                return;
            }
            if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
                if (wph == 8) {
                    hipLaunchKernelGGL((attention_tquad_kernel<HD, MODE, QF8, 8, 1>), dim3(p.total_wg),
                                       dim3(tthreads), qlds, st, p);
                    return;
                }
            }
            hipLaunchKernelGGL((attention_tquad_kernel<HD, MODE, QF8, 4, 1>), dim3(p.total_wg), dim3(tthreads), qlds,
                               st, p);
            return;
        }
    }
    // staged tiles: one LDS tile image per wave of the workgroup
    const unsigned lds = attention_staged<HD, MODE>() ? static_cast<unsigned>(threads / 64) * Geo<HD, MODE>::LDS_TILE : 0u;
    if (small_bs)
        hipLaunchKernelGGL((attention_kernel<HD, MODE, true, QF8, false>), dim3(p.total_wg), dim3(threads), 0, st, p);
    else if (attention_packs<HD, MODE>() && p.group <= 8)
        hipLaunchKernelGGL((attention_kernel<HD, MODE, false, QF8, attention_packs<HD, MODE>()>), dim3(p.total_wg),
                           dim3(threads), lds, st, p);
    else
        hipLaunchKernelGGL((attention_kernel<HD, MODE, false, QF8, false>), dim3(p.total_wg), dim3(threads), lds, st, p);
}

template <int HD, int MODE>
void launch_attention_v(const AttnArgs& p, int threads, bool small_bs, hipStream_t st) {
    if constexpr (MODE == KVQ_FP8_PER_TENSOR || MODE == KVQ_FP8_PER_HEAD || MODE == KVQ_FP8_PER_TOKEN_HEAD) {
        if (p.q_scales != nullptr) {
            launch_attention_q<HD, MODE, true>(p, threads, small_bs, st);
            return;
        }
    }
    launch_attention_q<HD, MODE, false>(p, threads, small_bs, st);
}

template <int HD>
void launch_attention_hd(const AttnArgs& p, int mode, int threads, bool small_bs, hipStream_t st) {
    switch (mode) {
        case KVQ_BF16: launch_attention_v<HD, KVQ_BF16>(p, threads, small_bs, st); break;
        case KVQ_FP8_PER_TENSOR: launch_attention_v<HD, KVQ_FP8_PER_TENSOR>(p, threads, small_bs, st); break;
        case KVQ_FP8_PER_HEAD: launch_attention_v<HD, KVQ_FP8_PER_HEAD>(p, threads, small_bs, st); break;
        case KVQ_FP8_PER_TOKEN_HEAD: launch_attention_v<HD, KVQ_FP8_PER_TOKEN_HEAD>(p, threads, small_bs, st); break;
        default: launch_attention_v<HD, KVQ_INT4_PER_TOKEN_HEAD>(p, threads, small_bs, st); break;
    }
}

}  // namespace

// Split partials of the allocation-free entry point live in this fixed
// device array instead of a caller workspace.  Each GPU holds its own copy
// (allocated with the code object, kept until the process ends); host code
// never passes `scratch` itself to a kernel: the name is only a host-side
// stand-in for the symbol, and its device address comes from
// hipGetSymbolAddress once per device (attention_scratch below).
static __device__ __align__(256) uint8_t scratch[KVQ_ATTENTION_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int attention_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return static_cast<int>(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        if (!p) return static_cast<int>(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int launch_attention(const AttnLaunch& a, const AttnPlan& pl, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    AttnArgs p;
    p.layer = a.layer;
    p.statics = a.static_scales;
    p.q = static_cast<const uint16_t*>(a.q);
    p.q_scales = a.q_scales;
    p.block_table = a.block_table;
    p.seq_lens = a.seq_lens;
    p.out = static_cast<uint16_t*>(a.out);
    const uint64_t o_bytes = static_cast<uint64_t>(a.num_seqs) * a.num_q_heads * pl.splits * a.head_dim * 4;
    p.part_o = pl.splits > 1 ? static_cast<float*>(a.workspace) : nullptr;
    p.part_ml = pl.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(a.workspace) + o_bytes) : nullptr;
    p.block_bytes = static_cast<int64_t>(a.block_bytes);
    p.num_blocks = a.num_blocks;
    p.code_bytes = static_cast<int32_t>(a.code_bytes);
    p.hkv = a.num_kv_heads;
    p.num_q_heads = a.num_q_heads;
    p.group = a.num_q_heads / a.num_kv_heads;
    p.qgroups = pl.qgroups;
    p.heads_per_wg = pl.heads_per_wg;
    p.head_chunks = a.num_kv_heads / pl.heads_per_wg;
    p.max_blocks = a.max_blocks;
    p.num_seqs = a.num_seqs;
    p.splits = pl.splits;
    p.tiles_per_split = pl.tiles_per_split;
    p.bs_log2 = a.bs_log2;
    p.max_len = a.num_blocks > 0 ? a.max_blocks << a.bs_log2 : 0;
    p.total_wg = static_cast<uint32_t>(pl.grid);
    p.c = a.sm_scale * kLog2e;
    p.kind = pl.kind;
    const int threads = 64 * pl.heads_per_wg;
    const bool small_bs = a.bs_log2 < 4;
    switch (a.head_dim) {
        case 64: launch_attention_hd<64>(p, a.mode, threads, small_bs, st); break;
        case 128: launch_attention_hd<128>(p, a.mode, threads, small_bs, st); break;
        default: launch_attention_hd<256>(p, a.mode, threads, small_bs, st); break;
    }
    int e = static_cast<int>(hipGetLastError());
    if (e != 0 || pl.splits == 1) return e;
    CombineArgs c;
    c.part_o = p.part_o;
    c.part_ml = p.part_ml;
    c.seq_lens = a.seq_lens;
    c.out = p.out;
    c.rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
    c.num_q_heads = a.num_q_heads;
    c.splits = pl.splits;
    c.tiles_per_split = pl.tiles_per_split;
    c.max_len = p.max_len;
    if (pl.splits >= kWideCombineSplits) {
        const uint32_t grid = static_cast<uint32_t>(c.rows);
        switch (a.head_dim) {
            case 64: hipLaunchKernelGGL(combine_wide_kernel<64>, dim3(grid), dim3(kWideCombineThreads), 0, st, c); break;
            case 128: hipLaunchKernelGGL(combine_wide_kernel<128>, dim3(grid), dim3(kWideCombineThreads), 0, st, c); break;
            default: hipLaunchKernelGGL(combine_wide_kernel<256>, dim3(grid), dim3(kWideCombineThreads), 0, st, c); break;
        }
        return static_cast<int>(hipGetLastError());
    }
    const uint32_t grid = static_cast<uint32_t>((c.rows + 3) / 4);
    switch (a.head_dim) {
        case 64: hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, st, c); break;
        case 128: hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, st, c); break;
        default: hipLaunchKernelGGL(combine_kernel<256>, dim3(grid), dim3(256), 0, st, c); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
