// kvq_kernels.hip -- gfx950 kernels of the quantized paged KV cache.
//
//  store_kernel   quantize-and-scatter of new K/V vectors ("Per-tensor vs
//                 per-head FP8 KV cache scales", "Dynamic per-token-head
//                 scales add 3.125 percent": reduce over each new head vector,
//                 write its scales, write its codes into the cache slot).
//  gather_kernel  paged read through a block table with dequantization back
//                 to BF16 (the same section: the scales are read back when the
//                 cache is consumed).
//
// Both are HBM-bound streams with a few VALU operations per byte: no MFMA
// (nothing here is a contraction).  Work is laid out for 64-wide wavefronts:
// a K/V row of head_dim elements (one token-head) is owned by LPR adjacent
// lanes of one DPP row, each lane holding EPL contiguous-in-groups-of-8
// elements, so the absmax reduction is a few DPP steps inside a 16-lane row.
//
// Exactness.  The stored quotient must be the correctly rounded FP32 x / s.
// Each row computes r = RN(1/s) once with an IEEE division; each element then
// takes y = RN(|x| r), e = fma(-y, s, |x|) (exact), q = fma(e, r, y), which is
// the correctly rounded quotient when r is the correctly rounded reciprocal
// and nothing is subnormal (P. Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", IBM J. R&D 34(1), 1990;
// see also Cornea, Harrison & Tang, "Scientific Computing on Itanium-based
// Systems", 2002).  Rows whose scale lies outside [2^-64, 2^64] scale both x
// and s by the same power of two first, which leaves the quotient unchanged
// and keeps s and r normal.  Quotients small enough to be subnormal encode to
// zero in both formats, so their rounding does not matter; the sign is taken
// from x, never from the quotient.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;          // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int MODE>
constexpr uint32_t row_bytes_of(int hd) {
    return MODE == KVQ_BF16 ? 2 * hd : (MODE == KVQ_INT4_PER_TOKEN_HEAD ? hd / 2 : hd);
}

template <int MODE>
constexpr bool dynamic_mode() {
    return MODE == KVQ_FP8_PER_TOKEN_HEAD || MODE == KVQ_INT4_PER_TOKEN_HEAD;
}

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Max over the LPR adjacent lanes that own one row (LPR a power of two <= 32).
// quad_perm [1,0,3,2] and [2,3,0,1] make each quad uniform, row_half_mirror
// joins quad pairs, row_mirror joins half-rows, a swizzle with xor 16 joins
// rows.
template <int LPR>
__device__ __forceinline__ uint32_t row_max(uint32_t v) {
    if constexpr (LPR >= 2) v = umax(v, dpp<0xB1>(v));
    if constexpr (LPR >= 4) v = umax(v, dpp<0x4E>(v));
    if constexpr (LPR >= 8) v = umax(v, dpp<0x141>(v));
    if constexpr (LPR >= 16) v = umax(v, dpp<0x140>(v));
    if constexpr (LPR >= 32)
        v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F)));
    return v;
}

// Packed max of |bf16| bit patterns (sign cleared): unsigned order of
// 0x7FFF-masked BF16 bits is the order of finite magnitudes.
__device__ __forceinline__ u16x2 abs_bits2(uint32_t w) {
    return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
}

__device__ __forceinline__ u16x2 absmax_chunk(const uint4& w, u16x2 acc) {
    u16x2 m01 = __builtin_elementwise_max(abs_bits2(w.x), abs_bits2(w.y));
    u16x2 m23 = __builtin_elementwise_max(abs_bits2(w.z), abs_bits2(w.w));
    return __builtin_elementwise_max(acc, __builtin_elementwise_max(m01, m23));
}

// Per-row quotient constants: s' = s * f, r = RN(1 / s') (0 when s == 0).
struct RowQ {
    float s;
    float r;
    float f;
};

__device__ __forceinline__ RowQ row_prep(float s) {
    RowQ q;
    q.f = (s < 0x1p-64f) ? 0x1p64f : ((s > 0x1p64f) ? 0x1p-64f : 1.0f);
    q.s = s * q.f;
    q.r = (q.s == 0.0f) ? 0.0f : 1.0f / q.s;       // IEEE division
    return q;
}

// RN(|x| / s) for |x| >= 0.  CLAMP bounds y for static scales, whose
// quotients may overflow; any y >= 2^20 saturates both formats anyway.
template <bool PRESCALE, bool CLAMP>
__device__ __forceinline__ float quotient(float x, const RowQ& q) {
    float ax = fabsf(x);
    if constexpr (PRESCALE) ax *= q.f;
    float y = ax * q.r;
    if constexpr (CLAMP) y = fminf(y, 0x1p20f);
    const float e = fmaf(-y, q.s, ax);
    return fmaf(e, q.r, y);
}

// 8 BF16 values -> 8 E4M3FN codes.  The magnitude is clamped to 448 and
// converted (round to nearest even); the sign bits of the inputs are then
// copied into the code bytes, so zero and tiny quotients keep their sign.
template <bool PRESCALE, bool CLAMP>
__device__ __forceinline__ uint2 encode_fp8(const uint4& w, const RowQ& q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t w0 = ws[2 * i], w1 = ws[2 * i + 1];
        const float q0 = fminf(quotient<PRESCALE, CLAMP>(bf16_lo(w0), q), 448.0f);
        const float q1 = fminf(quotient<PRESCALE, CLAMP>(bf16_hi(w0), q), 448.0f);
        const float q2 = fminf(quotient<PRESCALE, CLAMP>(bf16_lo(w1), q), 448.0f);
        const float q3 = fminf(quotient<PRESCALE, CLAMP>(bf16_hi(w1), q), 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, pk, true);
        // high byte of each BF16 (bit 7 = sign) -> byte lanes 0..3
        const uint32_t sign = __builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u;
        out[i] = static_cast<uint32_t>(pk) | sign;
    }
    return make_uint2(out[0], out[1]);
}

// 8 BF16 values -> 8 two's-complement nibbles, element 2j in the low nibble
// of byte j.  Adding 1.5 * 2^23 rounds the signed quotient to the nearest
// integer, ties to even, and leaves that integer in the low mantissa bits.
// Dynamic INT4 quotients are at most a / RN(a / 7) < 7.5 in magnitude, so the
// rounded value already lies in [-7, 7] and the clamp to [-8, 7] is a no-op.
template <bool PRESCALE>
__device__ __forceinline__ uint32_t encode_int4(const uint4& w, const RowQ& q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t xb = (e & 1) ? (ws[e >> 1] & 0xFFFF0000u) : (ws[e >> 1] << 16);
        const float mag = quotient<PRESCALE, false>(__uint_as_float(xb), q);
        const float sq = __uint_as_float((__float_as_uint(mag) & 0x7FFFFFFFu) | (xb & 0x80000000u));
        const float t = sq + 12582912.0f;
        acc |= (__float_as_uint(t) & 0xFu) << (4 * e);
    }
    return acc;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ------------------------------------------------------------------ store

struct StoreArgs {
    const uint4* __restrict__ keys;
    const uint4* __restrict__ values;
    const int64_t* __restrict__ slots;
    uint8_t* __restrict__ layer;
    const float* __restrict__ static_scales;
    int64_t num_rows;
    int64_t num_slots;
    uint64_t block_bytes;
    uint32_t code_bytes;
    uint32_t hkv;
    uint32_t hkv_magic;
    uint32_t hkv_shift;
    uint32_t bs_log2;
};

// One row = one (token, KV head) of K and the same of V.  LPR = HD / EPL
// lanes per row; chunk k of a lane is elements [(k * LPR + sub) * 8, +8), so
// each load instruction reads LPR * 16 contiguous bytes of every row.
template <int HD, int MODE, int EPL>
__global__ __launch_bounds__(kThreads) void store_kernel(StoreArgs p) {
    constexpr int LPR = HD / EPL;
    constexpr int CPL = EPL / 8;
    constexpr int RPW = 64 / LPR;
    constexpr int RPB = RPW * kWaves;
    constexpr uint32_t HB = row_bytes_of<MODE>(HD);
    static_assert(LPR >= 1 && LPR <= 32 && CPL >= 1, "bad row split");

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t sub = lane % LPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + wave * RPW + lane / LPR;
    const bool valid = row < p.num_rows;
    const uint32_t rowc = valid ? static_cast<uint32_t>(row) : 0u;

    uint4 kx[CPL], vx[CPL];
    const uint4* kp = p.keys + static_cast<uint64_t>(rowc) * (HD / 8) + sub;
    const uint4* vp = p.values + static_cast<uint64_t>(rowc) * (HD / 8) + sub;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        kx[k] = valid ? kp[k * LPR] : make_uint4(0, 0, 0, 0);
        vx[k] = valid ? vp[k * LPR] : make_uint4(0, 0, 0, 0);
    }

    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(rowc) * p.hkv_magic) >> p.hkv_shift);
    const uint32_t h = rowc - t * p.hkv;
    const int64_t slot = valid ? p.slots[t] : -1;
    const bool write = slot >= 0 && slot < p.num_slots;
    const uint64_t blk = static_cast<uint64_t>(slot) >> p.bs_log2;
    const uint32_t pos = static_cast<uint32_t>(slot) & ((1u << p.bs_log2) - 1u);
    uint8_t* const bp = p.layer + blk * p.block_bytes;
    const uint32_t ph = pos * p.hkv + h;
    uint8_t* const krow = bp + static_cast<uint64_t>(ph) * (2 * HB);
    uint8_t* const vrow = krow + HB;

    if constexpr (MODE == KVQ_BF16) {
        if (write) {
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const uint32_t c = k * LPR + sub;
                *reinterpret_cast<uint4*>(krow + c * 16) = kx[k];
                *reinterpret_cast<uint4*>(vrow + c * 16) = vx[k];
            }
        }
        return;
    } else {
        float sK, sV;
        if constexpr (dynamic_mode<MODE>()) {
            u16x2 ak = {0, 0}, av = {0, 0};
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                ak = absmax_chunk(kx[k], ak);
                av = absmax_chunk(vx[k], av);
            }
            const uint32_t amk = row_max<LPR>(umax(ak.x, ak.y));
            const uint32_t amv = row_max<LPR>(umax(av.x, av.y));
            constexpr float qmax = (MODE == KVQ_FP8_PER_TOKEN_HEAD) ? 448.0f : 7.0f;
            sK = __uint_as_float(amk << 16) / qmax;     // IEEE division
            sV = __uint_as_float(amv << 16) / qmax;
        } else if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
            sK = p.static_scales[0];
            sV = p.static_scales[1];
        } else {
            sK = p.static_scales[h];
            sV = p.static_scales[p.hkv + h];
        }
        const RowQ qk = row_prep(sK);
        const RowQ qv = row_prep(sV);
        const bool scaled = (qk.f != 1.0f) || (qv.f != 1.0f);
        const bool any_scaled = __builtin_amdgcn_ballot_w64(scaled) != 0;
        constexpr bool CLAMP = !dynamic_mode<MODE>();

        if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
            uint32_t ck[CPL], cv[CPL];
            if (any_scaled) {
#pragma unroll
                for (int k = 0; k < CPL; ++k) { ck[k] = encode_int4<true>(kx[k], qk); cv[k] = encode_int4<true>(vx[k], qv); }
            } else {
#pragma unroll
                for (int k = 0; k < CPL; ++k) { ck[k] = encode_int4<false>(kx[k], qk); cv[k] = encode_int4<false>(vx[k], qv); }
            }
            if (write) {
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const uint32_t c = k * LPR + sub;
                    *reinterpret_cast<uint32_t*>(krow + c * 4) = ck[k];
                    *reinterpret_cast<uint32_t*>(vrow + c * 4) = cv[k];
                }
            }
        } else {
            uint2 ck[CPL], cv[CPL];
            if (any_scaled) {
#pragma unroll
                for (int k = 0; k < CPL; ++k) { ck[k] = encode_fp8<true, CLAMP>(kx[k], qk); cv[k] = encode_fp8<true, CLAMP>(vx[k], qv); }
            } else {
#pragma unroll
                for (int k = 0; k < CPL; ++k) { ck[k] = encode_fp8<false, CLAMP>(kx[k], qk); cv[k] = encode_fp8<false, CLAMP>(vx[k], qv); }
            }
            if (write) {
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const uint32_t c = k * LPR + sub;
                    *reinterpret_cast<uint2*>(krow + c * 8) = ck[k];
                    *reinterpret_cast<uint2*>(vrow + c * 8) = cv[k];
                }
            }
        }
        if constexpr (dynamic_mode<MODE>()) {
            if (write && sub == 0)
                *reinterpret_cast<float2*>(bp + p.code_bytes + static_cast<uint64_t>(ph) * 8) = make_float2(sK, sV);
        }
    }
}

// ----------------------------------------------------------------- gather

struct GatherArgs {
    const uint8_t* __restrict__ layer;
    const float* __restrict__ static_scales;
    const int32_t* __restrict__ block_table;
    const int32_t* __restrict__ seq_lens;
    uint16_t* __restrict__ out_k;
    uint16_t* __restrict__ out_v;
    int64_t num_blocks;
    uint64_t block_bytes;
    uint32_t code_bytes;
    uint32_t hkv;
    uint32_t hkv_magic;
    uint32_t hkv_shift;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t block_size;
};

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// One workgroup per (sequence, logical block).  The block's code bytes are
// contiguous in the cache, rows ordered [position][head][K, V]; a 16-byte
// chunk c belongs to row c / (HB / 16), and the row's FP32 scale sits at the
// same row index in the block's scale trailer.
template <int HD, int MODE>
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs p) {
    constexpr uint32_t HB = row_bytes_of<MODE>(HD);
    constexpr uint32_t CPR = HB / 16;                        // chunks per row
    constexpr uint32_t EPC = (MODE == KVQ_BF16) ? 8 : (MODE == KVQ_INT4_PER_TOKEN_HEAD ? 32 : 16);
    constexpr int U = 4;

    const uint32_t wg = blockIdx.x;
    const uint32_t b = wg / static_cast<uint32_t>(p.max_blocks);
    const uint32_t j = wg - b * static_cast<uint32_t>(p.max_blocks);
    int64_t len = max(p.seq_lens[b], 0);
    len = min<int64_t>(len, static_cast<int64_t>(p.max_blocks) * p.block_size);
    const int64_t t0 = static_cast<int64_t>(j) * p.block_size;
    if (t0 >= len) return;
    const int32_t pb = p.block_table[static_cast<int64_t>(b) * p.max_blocks + j];
    if (pb < 0 || pb >= p.num_blocks) return;

    const uint32_t lane = threadIdx.x & 63u;
    int64_t off = 0;
    for (uint32_t i = lane; i < b; i += 64) off += max(p.seq_lens[i], 0);
    off = wave_sum(off);

    const uint32_t ntok = static_cast<uint32_t>(min<int64_t>(p.block_size, len - t0));
    const uint32_t nchunks = ntok * p.hkv * 2 * CPR;
    const uint8_t* const bp = p.layer + static_cast<uint64_t>(pb) * p.block_bytes;
    const uint4* const codes = reinterpret_cast<const uint4*>(bp);
    const float* const trailer = reinterpret_cast<const float*>(bp + p.code_bytes);
    const int64_t out_row0 = (off + t0) * p.hkv;

    float s_static[2] = {0.0f, 0.0f};
    if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
        s_static[0] = p.static_scales[0];
        s_static[1] = p.static_scales[1];
    }

    for (uint32_t base = threadIdx.x; base < nchunks; base += kThreads * U) {
        uint4 cw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = base + u * kThreads;
            cw[u] = (c < nchunks) ? codes[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = base + u * kThreads;
            if (c >= nchunks) continue;
            const uint32_t row = c / CPR;
            const uint32_t col = c % CPR;
            uint16_t* const outp = ((row & 1u) ? p.out_v : p.out_k) +
                                   static_cast<uint64_t>(out_row0 + (row >> 1)) * HD + col * EPC;
            uint4* const o = reinterpret_cast<uint4*>(outp);
            if constexpr (MODE == KVQ_BF16) {
                o[0] = cw[u];
            } else {
                float s;
                if constexpr (dynamic_mode<MODE>()) {
                    s = trailer[row];
                } else if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
                    s = s_static[row & 1u];
                } else {
                    const uint32_t th = row >> 1;
                    const uint32_t tt = static_cast<uint32_t>((static_cast<uint64_t>(th) * p.hkv_magic) >> p.hkv_shift);
                    s = p.static_scales[(row & 1u) * p.hkv + (th - tt * p.hkv)];
                }
                const uint32_t ws[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
                if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t r[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float a = static_cast<float>(static_cast<int32_t>(ws[d] << (28 - 8 * e)) >> 28);
                            const float bb = static_cast<float>(static_cast<int32_t>(ws[d] << (24 - 8 * e)) >> 28);
                            r[e] = pack_bf16(a * s, bb * s);
                        }
                        o[d] = make_uint4(r[0], r[1], r[2], r[3]);
                    }
                } else {
                    uint32_t r[8];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(ws[d]), false);
                        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(ws[d]), true);
                        r[2 * d] = pack_bf16(lo[0] * s, lo[1] * s);
                        r[2 * d + 1] = pack_bf16(hi[0] * s, hi[1] * s);
                    }
                    o[0] = make_uint4(r[0], r[1], r[2], r[3]);
                    o[1] = make_uint4(r[4], r[5], r[6], r[7]);
                }
            }
        }
    }
}

// ---------------------------------------------------------- static table

struct StaticValues {
    float v[2 * KVQ_MAX_STATIC_KV_HEADS];
};

__global__ void write_static_kernel(float* dst, StaticValues vals, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = vals.v[i];
}

// --------------------------------------------------------------- dispatch

template <int HD, int MODE>
int launch_store_t(const StoreLaunch& a, void* stream) {
    constexpr int EPL = 32;
    constexpr int RPB = (64 / (HD / EPL)) * kWaves;
    StoreArgs p;
    p.keys = static_cast<const uint4*>(a.keys);
    p.values = static_cast<const uint4*>(a.values);
    p.slots = a.slots;
    p.layer = a.layer;
    p.static_scales = a.static_scales;
    p.num_rows = a.num_rows;
    p.num_slots = a.num_slots;
    p.block_bytes = a.block_bytes;
    p.code_bytes = static_cast<uint32_t>(a.code_bytes);
    p.hkv = static_cast<uint32_t>(a.num_kv_heads);
    const DivMagic dm = div_magic(p.hkv);
    p.hkv_magic = dm.magic;
    p.hkv_shift = dm.shift;
    p.bs_log2 = static_cast<uint32_t>(a.bs_log2);
    const uint32_t grid = static_cast<uint32_t>((a.num_rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((store_kernel<HD, MODE, EPL>), dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return static_cast<int>(hipGetLastError());
}

template <int MODE>
int launch_store_m(const StoreLaunch& a, void* stream) {
    switch (a.head_dim) {
        case 64: return launch_store_t<64, MODE>(a, stream);
        case 128: return launch_store_t<128, MODE>(a, stream);
        default: return launch_store_t<256, MODE>(a, stream);
    }
}

template <int HD, int MODE>
int launch_gather_t(const GatherLaunch& a, void* stream) {
    GatherArgs p;
    p.layer = a.layer;
    p.static_scales = a.static_scales;
    p.block_table = a.block_table;
    p.seq_lens = a.seq_lens;
    p.out_k = static_cast<uint16_t*>(a.out_keys);
    p.out_v = static_cast<uint16_t*>(a.out_values);
    p.num_blocks = a.num_blocks;
    p.block_bytes = a.block_bytes;
    p.code_bytes = static_cast<uint32_t>(a.code_bytes);
    p.hkv = static_cast<uint32_t>(a.num_kv_heads);
    const DivMagic dm = div_magic(p.hkv);
    p.hkv_magic = dm.magic;
    p.hkv_shift = dm.shift;
    p.max_blocks = a.max_blocks;
    p.num_seqs = a.num_seqs;
    p.block_size = a.block_size;
    const uint32_t grid = static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * a.max_blocks);
    hipLaunchKernelGGL((gather_kernel<HD, MODE>), dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return static_cast<int>(hipGetLastError());
}

template <int MODE>
int launch_gather_m(const GatherLaunch& a, void* stream) {
    switch (a.head_dim) {
        case 64: return launch_gather_t<64, MODE>(a, stream);
        case 128: return launch_gather_t<128, MODE>(a, stream);
        default: return launch_gather_t<256, MODE>(a, stream);
    }
}

}  // namespace

int launch_store(const StoreLaunch& a, void* stream) {
    switch (a.mode) {
        case KVQ_BF16: return launch_store_m<KVQ_BF16>(a, stream);
        case KVQ_FP8_PER_TENSOR: return launch_store_m<KVQ_FP8_PER_TENSOR>(a, stream);
        case KVQ_FP8_PER_HEAD: return launch_store_m<KVQ_FP8_PER_HEAD>(a, stream);
        case KVQ_FP8_PER_TOKEN_HEAD: return launch_store_m<KVQ_FP8_PER_TOKEN_HEAD>(a, stream);
        default: return launch_store_m<KVQ_INT4_PER_TOKEN_HEAD>(a, stream);
    }
}

int launch_gather(const GatherLaunch& a, void* stream) {
    switch (a.mode) {
        case KVQ_BF16: return launch_gather_m<KVQ_BF16>(a, stream);
        case KVQ_FP8_PER_TENSOR: return launch_gather_m<KVQ_FP8_PER_TENSOR>(a, stream);
        case KVQ_FP8_PER_HEAD: return launch_gather_m<KVQ_FP8_PER_HEAD>(a, stream);
        case KVQ_FP8_PER_TOKEN_HEAD: return launch_gather_m<KVQ_FP8_PER_TOKEN_HEAD>(a, stream);
        default: return launch_gather_m<KVQ_INT4_PER_TOKEN_HEAD>(a, stream);
    }
}

int launch_write_static(float* dst, const float* values, int n, void* stream) {
    StaticValues v{};
    for (int i = 0; i < n && i < 2 * KVQ_MAX_STATIC_KV_HEADS; ++i) v.v[i] = values[i];
    hipLaunchKernelGGL(write_static_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), dst, v, n);
    return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
