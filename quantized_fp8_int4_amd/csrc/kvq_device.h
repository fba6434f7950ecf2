// kvq_device.h -- device helpers shared by the gfx950 kernels: BF16 widening,
// DPP row reductions, packed absmax, FP8/INT4 encoders, BF16 packing and
// (non-)temporal memory accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_exact.h"

namespace kvq {
namespace dev {

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
    q.s = s * q.f;                                  // normal unless s == 0
    q.r = (q.s == 0.0f) ? 0.0f : rcp_exact(q.s);
    return q;
}

// RN(x / s), sign included.  y = RN(x r) is within an ulp of the quotient;
// the residual d = y s - x is exact in one FMA, and q = RN(y - d r) is the
// correctly rounded quotient (Markstein).  Every step is odd in x, so the
// result is the sign of x times RN(|x| / s).  Writing the residual as y s - x,
// not x - y s, keeps the sign of zero: x = -0 gives y = -0, d = +0 and
// q = -0 + -0 = -0 (and s = 0, where r = 0, gives q = x * 0).  CLAMP bounds y
// for static scales, whose quotients may overflow; any |y| >= 2^20 saturates
// both formats anyway.
template <bool PRESCALE, bool CLAMP>
__device__ __forceinline__ float quotient(float x, const RowQ& q) {
    if constexpr (PRESCALE) x *= q.f;
    float y = x * q.r;
    if constexpr (CLAMP) y = __builtin_amdgcn_fmed3f(y, -0x1p20f, 0x1p20f);
    const float d = fmaf(y, q.s, -x);
    return fmaf(-d, q.r, y);
}

// 8 BF16 values -> 8 E4M3FN codes.  The conversion rounds to nearest even and
// keeps the sign of zero and of quotients too small for E4M3.  Static scales
// (CLAMP) clamp the quotient to [-448, 448] first.  Dynamic scales need no
// clamp: s = RN(a / 448) >= (a / 448)(1 - 2^-24), so |q| <= RN(448 (1 + 2^-23))
// = 448 + 2^-15, which the conversion rounds to 448 like any value below 464.
template <bool PRESCALE, bool CLAMP>
__device__ __forceinline__ uint2 encode_fp8(const uint4& w, const RowQ& q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t w0 = ws[2 * i], w1 = ws[2 * i + 1];
        float q0 = quotient<PRESCALE, CLAMP>(bf16_lo(w0), q);
        float q1 = quotient<PRESCALE, CLAMP>(bf16_hi(w0), q);
        float q2 = quotient<PRESCALE, CLAMP>(bf16_lo(w1), q);
        float q3 = quotient<PRESCALE, CLAMP>(bf16_hi(w1), q);
        if constexpr (CLAMP) {
            q0 = __builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f);
            q1 = __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f);
            q2 = __builtin_amdgcn_fmed3f(q2, -448.0f, 448.0f);
            q3 = __builtin_amdgcn_fmed3f(q3, -448.0f, 448.0f);
        }
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, pk, true);
        out[i] = static_cast<uint32_t>(pk);
    }
    return make_uint2(out[0], out[1]);
}

// 8 BF16 values -> 8 two's-complement nibbles, element 2j in the low nibble
// of byte j.  Dynamic INT4 quotients are at most a / RN(a / 7) < 7.5 in
// magnitude, so n = rint_even(q) lies in [-7, 7] and no clamp is needed.
// t = RN(q + 2^23 + 8) = 2^23 + 8 + n exactly (one rounding, to an integer,
// ties to even): its bit pattern is the exponent of 2^23, zeros, and n + 8
// in bits 0..3.  Shifted left by 8 or more, only that nibble survives (bit 23,
// the exponent's lowest bit, is 0).  Element 1 (shift 4) uses
// RN(1024 q + 2^33 + 2^13) instead, whose exponent field has its five lowest
// bits clear.  The nibbles n + 8 are then flipped to two's complement with
// one XOR by 8.
template <bool PRESCALE>
__device__ __forceinline__ uint32_t encode_int4(const uint4& w, const RowQ& q) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(ws[e >> 1]) : bf16_lo(ws[e >> 1]);
        const float qe = quotient<PRESCALE, false>(x, q);
        if (e == 0) {
            acc = __float_as_uint(qe + 0x1.00001p23f) & 0xFu;
        } else if (e == 1) {
            acc |= __float_as_uint(fmaf(qe, 1024.0f, 0x1.00001p33f)) << 4;
        } else {
            acc |= __float_as_uint(qe + 0x1.00001p23f) << (4 * e);
        }
    }
    return acc ^ 0x88888888u;
}

// The low INT4 nibble of byte B of x -> n / 16 as FP32, exact
// (v_cvt_off_f32_i4).  Written as byte extracts so that the conversion reads
// the byte through an SDWA operand select instead of a separate shift.
template <int B>
__device__ __forceinline__ float int4_over16(uint32_t x) {
    const uint32_t b = B == 0 ? x : (B == 3 ? x >> 24 : (x >> (8 * B)) & 0xFFu);
    return __builtin_amdgcn_cvt_off_f32_i4(static_cast<int>(b));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ------------------------------------------------------- memory helpers

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// NT selects the non-temporal form: data read or written once by this call
// is streamed instead of kept in the caches.
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
    u32x4 v;
    if constexpr (NT) v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    else v = *static_cast<const u32x4*>(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool NT>
__device__ __forceinline__ void st16(void* p, const uint4& x) {
    const u32x4 v = {x.x, x.y, x.z, x.w};
    if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
    else *static_cast<u32x4*>(p) = v;
}

template <bool NT>
__device__ __forceinline__ void st8(void* p, const uint2& x) {
    const u32x2 v = {x.x, x.y};
    if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x2*>(p));
    else *static_cast<u32x2*>(p) = v;
}

template <bool NT>
__device__ __forceinline__ void st4(void* p, uint32_t x) {
    if constexpr (NT) __builtin_nontemporal_store(x, static_cast<uint32_t*>(p));
    else *static_cast<uint32_t*>(p) = x;
}


}  // namespace dev
}  // namespace kvq
