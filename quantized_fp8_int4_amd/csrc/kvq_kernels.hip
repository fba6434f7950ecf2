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
// Each row computes r = RN(1/s) once (rcp_exact); each element then
// takes y = RN(x r), d = fma(y, s, -x) (exact), q = fma(-d, r, y), which is
// the correctly rounded quotient when r is the correctly rounded reciprocal
// and nothing is subnormal (P. Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", IBM J. R&D 34(1), 1990;
// see also Cornea, Harrison & Tang, "Scientific Computing on Itanium-based
// Systems", 2002).  Rows whose scale lies outside [2^-64, 2^64] scale both x
// and s by the same power of two first, which leaves the quotient unchanged
// and keeps s and r normal.  Quotients small enough to be subnormal encode to
// zero in both formats, so their rounding does not matter; the steps are odd
// in x and keep the sign of x on a zero quotient.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

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
    const int32_t* __restrict__ order;   // ORD: token order[i] is processed i-th
    uint32_t num_tokens;
};

// Tuning knobs of the store kernel: EPL elements of a row per lane (LPR =
// HD / EPL lanes per row), RPL rows per lane (more loads in flight per
// wave), NTL non-temporal loads of the new K/V, NTS non-temporal stores of
// the codes.

// Quantize the K and V chunks of one row (already loaded) and scatter them.
template <int LPR, int CPL, bool CONTIG>
__device__ __forceinline__ uint32_t chunk_index(int k, uint32_t sub) {
    return CONTIG ? sub * CPL + k : k * LPR + sub;
}

template <int HD, int MODE, int LPR, int CPL, bool CONTIG, bool NTS, bool WT>
__device__ __forceinline__ void store_row(const StoreArgs& p, uint32_t rowc, bool valid, uint32_t sub,
                                          const uint4 (&kx)[CPL], const uint4 (&vx)[CPL], uint64_t wrow) {
    constexpr uint32_t HB = row_bytes_of<MODE>(HD);
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(rowc) * p.hkv_magic) >> p.hkv_shift);
    const uint32_t h = rowc - t * p.hkv;
    const int64_t slot = p.slots[t];
    const bool write = valid && slot >= 0 && slot < p.num_slots;
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
                const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                st16<NTS>(krow + c * 16, kx[k]);
                st16<NTS>(vrow + c * 16, vx[k]);
            }
        }
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
            constexpr int QMAX = (MODE == KVQ_FP8_PER_TOKEN_HEAD) ? 448 : 7;
            const float aK = __uint_as_float(amk << 16);
            const float aV = __uint_as_float(amv << 16);
            // Waves holding a row with absmax below 2^-100 (a subnormal or
            // near-subnormal scale) take the IEEE division.
            if (__builtin_amdgcn_ballot_w64(fminf(aK, aV) < 0x1p-100f) != 0) {
                sK = aK / static_cast<float>(QMAX);
                sV = aV / static_cast<float>(QMAX);
            } else {
                sK = div_by_const<QMAX>(aK);
                sV = div_by_const<QMAX>(aV);
            }
        } else if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
            sK = p.static_scales[0];
            sV = p.static_scales[1];
        } else if constexpr (WT) {
            // a table of at most 32 KV heads (64 entries): lane l loads entry
            // l, once per wave, and each lane reads its head's pair across
            // lanes.  Two table loads per lane measured 2.2% slower on the
            // GQA-32 per-head store.
            const uint32_t ln = threadIdx.x & 63u;
            const float tv = p.static_scales[ln < 2u * p.hkv ? ln : 0u];
            sK = __shfl(tv, static_cast<int>(h), 64);
            sV = __shfl(tv, static_cast<int>(p.hkv + h), 64);
        } else {
            // larger tables: the wave's RPW rows (from wrow on) need RPW
            // (K, V) pairs; lane r < RPW loads row r's K scale and lane
            // RPW + r its V scale, and each lane reads its own row's pair
            // across lanes
            constexpr uint32_t RPW = 64 / LPR;
            static_assert(2 * RPW <= 64, "a wave's K and V scales fit its lanes");
            const uint32_t ln = threadIdx.x & 63u;
            // (rows past the end take the last row's head: every index stays
            // inside the table and below the division's 2^31 bound)
            const uint64_t rs = min(wrow + (ln % RPW), static_cast<uint64_t>(p.num_rows - 1));
            const uint32_t ts = static_cast<uint32_t>((rs * p.hkv_magic) >> p.hkv_shift);
            const uint32_t hs = static_cast<uint32_t>(rs) - ts * p.hkv;
            const float tv = p.static_scales[(ln / RPW == 1u ? p.hkv : 0u) + hs];
            const int r = static_cast<int>(ln / LPR);
            sK = __shfl(tv, r, 64);
            sV = __shfl(tv, static_cast<int>(RPW) + r, 64);
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
            if constexpr (!CONTIG && LPR == 8 && (2 * HB) % 128 == 0) {
                // whole-line stores through the wave's LDS, as for FP8 (a
                // direct store wrote 4 bytes per lane, a quarter line per
                // row): measured +2.8% at head_dim 128 and +6.8% at 256; at
                // 64 a row's K|V codes are half a line and keep the direct
                // stores
                __shared__ __attribute__((aligned(16))) uint8_t stage4[4][8][2 * HB];
                const uint32_t wv = (threadIdx.x >> 6) & 3u, rl = (threadIdx.x & 63u) / LPR;
                uint8_t* const sr = &stage4[wv][rl][0];
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                    *reinterpret_cast<uint32_t*>(sr + c * 4) = ck[k];
                    *reinterpret_cast<uint32_t*>(sr + HB + c * 4) = cv[k];
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                constexpr int NL = 2 * HB / 128;
                uint4 ln[NL];
#pragma unroll
                for (int l = 0; l < NL; ++l) ln[l] = *reinterpret_cast<const uint4*>(sr + 128 * l + 16 * sub);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                if (write) {
#pragma unroll
                    for (int l = 0; l < NL; ++l) st16<NTS>(krow + 128 * l + 16 * sub, ln[l]);
                }
            } else if (write) {
                if constexpr (CONTIG && CPL % 2 == 0) {
#pragma unroll
                    for (int k = 0; k < CPL; k += 2) {
                        const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                        st8<NTS>(krow + c * 4, make_uint2(ck[k], ck[k + 1]));
                        st8<NTS>(vrow + c * 4, make_uint2(cv[k], cv[k + 1]));
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < CPL; ++k) {
                        const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                        st4<NTS>(krow + c * 4, ck[k]);
                        st4<NTS>(vrow + c * 4, cv[k]);
                    }
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
            if constexpr (!CONTIG && LPR == 8 && (2 * HB) % 128 == 0) {
                // staged through the wave's LDS so that each store
                // instruction writes whole 128-byte lines: lane sub of a row
                // writes bytes [128 l + 16 sub, +16) of the row's K|V codes
                // (2 HB contiguous bytes), where each direct store had
                // written 64-byte half lines.  Measured on 32768-token
                // prefills: head_dim 128 +3% in slot order and 0 to +2% in
                // token order, head_dim 64 +3%, head_dim 256 +2 to +3%.
                __shared__ __attribute__((aligned(16))) uint8_t stage[4][8][2 * HB];
                const uint32_t wv = (threadIdx.x >> 6) & 3u, rl = (threadIdx.x & 63u) / LPR;
                uint8_t* const sr = &stage[wv][rl][0];
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                    *reinterpret_cast<uint2*>(sr + c * 8) = ck[k];
                    *reinterpret_cast<uint2*>(sr + HB + c * 8) = cv[k];
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                // the row's K|V codes are 2 HB contiguous bytes: NL whole lines
                constexpr int NL = 2 * HB / 128;
                uint4 ln[NL];
#pragma unroll
                for (int l = 0; l < NL; ++l) ln[l] = *reinterpret_cast<const uint4*>(sr + 128 * l + 16 * sub);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                if (write) {
#pragma unroll
                    for (int l = 0; l < NL; ++l) st16<NTS>(krow + 128 * l + 16 * sub, ln[l]);
                }
            } else if (write) {
                if constexpr (CONTIG && CPL % 2 == 0) {
#pragma unroll
                    for (int k = 0; k < CPL; k += 2) {
                        const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                        st16<NTS>(krow + c * 8, make_uint4(ck[k].x, ck[k].y, ck[k + 1].x, ck[k + 1].y));
                        st16<NTS>(vrow + c * 8, make_uint4(cv[k].x, cv[k].y, cv[k + 1].x, cv[k + 1].y));
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < CPL; ++k) {
                        const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, sub);
                        st8<NTS>(krow + c * 8, ck[k]);
                        st8<NTS>(vrow + c * 8, cv[k]);
                    }
                }
            }
        }
        if constexpr (dynamic_mode<MODE>()) {
            if (write && sub == 0)
                *reinterpret_cast<float2*>(bp + p.code_bytes + static_cast<uint64_t>(ph) * 8) = make_float2(sK, sV);
        }
    }
}

// One row = one (token, KV head) of K and the same of V, owned by LPR
// adjacent lanes.  Chunk k of a lane is elements [(k * LPR + sub) * 8, +8),
// so each load instruction reads LPR * 16 contiguous bytes of every row.  A
// wave owns RPL groups of 64 / LPR consecutive rows and loads all of them
// before quantizing any.  ORD: the rows are taken in the caller's token
// order (row i * Hkv + h is token order[i]'s head h), which, sorted by slot,
// makes the writes run through the layer in address order and the reads
// scattered instead; an entry outside [0, num_tokens) stores nothing.
template <int HD, int MODE, int EPL, int RPL, bool NTL, bool NTS, bool CONTIG, int TPB, bool WT, bool ORD>
__global__ __launch_bounds__(TPB) void store_kernel(StoreArgs p) {
    constexpr int LPR = HD / EPL;
    constexpr int CPL = EPL / 8;
    constexpr int RPW = 64 / LPR;
    constexpr int RPB = RPW * RPL * (TPB / 64);
    static_assert(LPR >= 1 && LPR <= 32 && CPL >= 1 && RPL >= 1, "bad row split");

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t sub = lane % LPR;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * RPB + wave * (RPW * RPL) + lane / LPR;

    uint4 kx[RPL][CPL], vx[RPL][CPL];
    uint32_t src[RPL];             // the source row of each group (the row itself without ORD)
    bool ok[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int64_t row = row0 + j * RPW;
        bool valid = row < p.num_rows;
        uint64_t rowc = valid ? static_cast<uint64_t>(row) : 0u;
        if constexpr (ORD) {
            const uint32_t r32 = static_cast<uint32_t>(rowc);
            const uint32_t i = static_cast<uint32_t>((static_cast<uint64_t>(r32) * p.hkv_magic) >> p.hkv_shift);
            const uint32_t tok = static_cast<uint32_t>(p.order[i]);
            valid = valid && tok < p.num_tokens;
            rowc = valid ? static_cast<uint64_t>(tok) * p.hkv + (r32 - i * p.hkv) : 0u;
        }
        src[j] = static_cast<uint32_t>(rowc);
        ok[j] = valid;
        const uint4* kp = p.keys + rowc * (HD / 8) + sub;
        const uint4* vp = p.values + rowc * (HD / 8) + sub;
        // Unconditional loads (rows past the end read row 0 and never write):
        // no branch, so every load of the wave stays in flight together.
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const uint32_t c = chunk_index<LPR, CPL, CONTIG>(k, 0) + (CONTIG ? sub * (CPL - 1) : 0);
            kx[j][k] = ld16<NTL>(kp + c);
            vx[j][k] = ld16<NTL>(vp + c);
        }
    }
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        // the wave's first row of this group (the same KV heads, row for row,
        // as its source rows: an order moves whole tokens)
        const uint64_t wrow = static_cast<uint64_t>(blockIdx.x) * RPB + wave * (RPW * RPL) + j * RPW;
        store_row<HD, MODE, LPR, CPL, CONTIG, NTS, WT>(p, src[j], ok[j], sub, kx[j], vx[j], wrow);
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
    int64_t out_th;           // token-head rows each output holds (out_rows * hkv)
    int64_t num_blocks;
    uint64_t block_bytes;
    uint32_t code_bytes;
    uint32_t hkv;
    uint32_t hkv_magic;
    uint32_t hkv_shift;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t block_size;
    uint32_t parts;           // workgroups per logical block
};

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Codes are read once per call: 8- and 16-byte chunks are loaded
// non-temporally (+1.7% at FP8 head_dim 128); 4-byte chunks are not, which
// measured up to 19% slower in that form.
template <int N>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&w)[N]) {
    if constexpr (N == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else if constexpr (N == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[0] = v[0]; w[1] = v[1];
    } else {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// Decode the loaded chunks of one gather thread and store them as BF16 at
// their packed output rows; BOUNDED skips rows at or past `room`.
template <int HD, int MODE, int CB, int U, bool NTS, bool BOUNDED>
__device__ __forceinline__ void gather_decode_store(const GatherArgs& p, const uint32_t (&cw)[U][CB / 4],
                                                    const float (&sc)[U], const uint32_t (&chunk)[U],
                                                    int64_t out_row0, int64_t room) {
    constexpr uint32_t HB = row_bytes_of<MODE>(HD);
    constexpr int DW = CB / 4;
    constexpr uint32_t CPR = HB / CB;
    constexpr int OUT_PER_DW = (MODE == KVQ_BF16) ? 1 : (MODE == KVQ_INT4_PER_TOKEN_HEAD ? 4 : 2);
    constexpr int ODW = DW * OUT_PER_DW;
    constexpr uint32_t EPC = ODW * 2;

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t row = chunk[u] / CPR;
        const uint32_t col = chunk[u] % CPR;
        uint16_t* const outp = ((row & 1u) ? p.out_v : p.out_k) +
                               static_cast<uint64_t>(out_row0 + (row >> 1)) * HD + col * EPC;
        const float s = sc[u];
        uint32_t o[ODW];
        if constexpr (MODE == KVQ_BF16) {
#pragma unroll
            for (int d = 0; d < DW; ++d) o[d] = cw[u][d];
        } else if constexpr (MODE == KVQ_INT4_PER_TOKEN_HEAD) {
            // Byte e holds elements 2e (low nibble) and 2e+1.  While 16 s is
            // finite, (n / 16)(16 s) is the same real number as n s, so it
            // rounds alike; waves holding a larger scale widen n itself.
            if (__builtin_amdgcn_ballot_w64(s > 0x1p120f) == 0) {
                const float s16 = s * 16.0f;
#pragma unroll
                for (int d = 0; d < DW; ++d) {
                    const uint32_t w = cw[u][d], hi = __builtin_amdgcn_alignbit(w, w, 4);
                    o[4 * d + 0] = pack_bf16(int4_over16<0>(w) * s16, int4_over16<0>(hi) * s16);
                    o[4 * d + 1] = pack_bf16(int4_over16<1>(w) * s16, int4_over16<1>(hi) * s16);
                    o[4 * d + 2] = pack_bf16(int4_over16<2>(w) * s16, int4_over16<2>(hi) * s16);
                    o[4 * d + 3] = pack_bf16(int4_over16<3>(w) * s16, int4_over16<3>(hi) * s16);
                }
            } else {
#pragma unroll
                for (int d = 0; d < DW; ++d) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a = static_cast<float>(static_cast<int32_t>(cw[u][d] << (28 - 8 * e)) >> 28);
                        const float bb = static_cast<float>(static_cast<int32_t>(cw[u][d] << (24 - 8 * e)) >> 28);
                        o[4 * d + e] = pack_bf16(a * s, bb * s);
                    }
                }
            }
        } else {
#pragma unroll
            for (int d = 0; d < DW; ++d) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw[u][d]), false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw[u][d]), true);
                o[2 * d] = pack_bf16(lo[0] * s, lo[1] * s);
                o[2 * d + 1] = pack_bf16(hi[0] * s, hi[1] * s);
            }
        }
        if (!BOUNDED || static_cast<int64_t>(row >> 1) < room) {
#pragma unroll
            for (int q = 0; q < ODW / 4; ++q)
                st16<NTS>(outp + 8 * q, make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]));
        }
    }
}

// Sequences whose offset is summed without a loop: 64 lanes x kOffsetLoads.
constexpr int kOffsetLoads = 4;

// Tuning knobs of the gather kernel: CB code bytes per thread chunk, U
// chunks per thread, NTS non-temporal stores of the BF16 output, LDSS stage
// the part's per-row scales in LDS (one load per row instead of one per
// chunk).
//
// One workgroup per (sequence, logical block, part); a part is up to
// TPB * U chunks of the block.  The block's code bytes are contiguous in
// the cache with rows ordered [position][head][K, V]; a chunk of CB code bytes
// belongs to row c / (HB / CB), and the row's FP32 scale sits at the same row
// index of the block's scale trailer.  The body is straight-line so every
// load of a workgroup is in flight at once: lanes past the last chunk load,
// decode and store the last chunk again (identical bytes to the same place).
template <int HD, int MODE, int CB, int U, bool NTS, bool LDSS, int TPB>
__global__ __launch_bounds__(TPB) void gather_kernel(GatherArgs p) {
    constexpr int kThreads = TPB;
    constexpr uint32_t HB = row_bytes_of<MODE>(HD);
    constexpr int DW = CB / 4;                               // code dwords per chunk
    constexpr uint32_t CPR = HB / CB;                        // chunks per row
    constexpr int OUT_PER_DW = (MODE == KVQ_BF16) ? 1 : (MODE == KVQ_INT4_PER_TOKEN_HEAD ? 4 : 2);
    constexpr int ODW = DW * OUT_PER_DW;                     // output dwords per chunk
    constexpr uint32_t EPC = ODW * 2;                        // output elements per chunk
    static_assert(ODW % 4 == 0, "output chunk must be whole 16-byte stores");
    static_assert(HB % CB == 0, "row must be whole chunks");

    const uint32_t wg = blockIdx.x;
    const uint32_t bj = wg / p.parts;
    const uint32_t part = wg - bj * p.parts;
    const uint32_t b = bj / static_cast<uint32_t>(p.max_blocks);
    const uint32_t j = bj - b * static_cast<uint32_t>(p.max_blocks);
    // Both scalar loads are in bounds for every (b, j); issue them together.
    const int32_t raw_len = p.seq_lens[b];
    const int32_t pb = p.block_table[static_cast<int64_t>(b) * p.max_blocks + j];
    const int64_t len = min<int64_t>(max(raw_len, 0), static_cast<int64_t>(p.max_blocks) * p.block_size);
    const int64_t t0 = static_cast<int64_t>(j) * p.block_size;
    if (t0 >= len) return;
    if (pb < 0 || pb >= p.num_blocks) return;
    const uint32_t ntok = static_cast<uint32_t>(min<int64_t>(p.block_size, len - t0));
    const uint32_t nchunks = ntok * p.hkv * 2 * CPR;
    const uint32_t c0 = part * (kThreads * U);
    if (c0 >= nchunks) return;

    // Offset of sequence b in the packed output: sum of the earlier lengths.
    // These loads go out first, so waiting for them never waits for codes.
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t last_seq = static_cast<uint32_t>(p.num_seqs - 1);
    int32_t lens[kOffsetLoads];
#pragma unroll
    for (int k = 0; k < kOffsetLoads; ++k) lens[k] = p.seq_lens[min(lane + 64u * k, last_seq)];
    int64_t off_tail = 0;
    if (b > 64u * kOffsetLoads) {
        for (uint32_t i = lane + 64u * kOffsetLoads; i < b; i += 64) off_tail += max(p.seq_lens[i], 0);
    }

    const uint8_t* const bp = p.layer + static_cast<uint64_t>(pb) * p.block_bytes;
    const float* const trailer = reinterpret_cast<const float*>(bp + p.code_bytes);
    auto row_scale = [&](uint32_t row) -> float {
        if constexpr (dynamic_mode<MODE>()) {
            return trailer[row];
        } else if constexpr (MODE == KVQ_FP8_PER_HEAD) {
            const uint32_t th = row >> 1;
            const uint32_t tt = static_cast<uint32_t>((static_cast<uint64_t>(th) * p.hkv_magic) >> p.hkv_shift);
            return p.static_scales[(row & 1u) * p.hkv + (th - tt * p.hkv)];
        } else if constexpr (MODE == KVQ_FP8_PER_TENSOR) {
            return p.static_scales[row & 1u];
        } else {
            return 0.0f;
        }
    };
    // Rows this part touches: [row_lo, row_lo + kPartRows).
    constexpr uint32_t kPartRows = (kThreads * U + CPR - 1) / CPR + 1;
    constexpr bool STAGE = LDSS && MODE != KVQ_BF16;
    __shared__ float s_rows[STAGE ? kPartRows : 1];
    const uint32_t row_lo = c0 / CPR;
    const uint32_t nrows = nchunks / CPR;
    float staged = 0.0f;
    if constexpr (STAGE) {
        // issued before the code loads, so waiting for it never waits for codes
        if (threadIdx.x < kPartRows) staged = row_scale(min(row_lo + threadIdx.x, nrows - 1));
    }

    uint32_t cw[U][DW];
    float sc[U];
    uint32_t chunk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        chunk[u] = min(c0 + threadIdx.x + u * kThreads, nchunks - 1);
        load_codes<DW>(bp + static_cast<uint64_t>(chunk[u]) * CB, cw[u]);
    }
    if constexpr (STAGE) {
        if (threadIdx.x < kPartRows) s_rows[threadIdx.x] = staged;
        // LDS-only fence: the barrier waits for the LDS writes, not for the
        // code loads in flight.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
        for (int u = 0; u < U; ++u) sc[u] = s_rows[chunk[u] / CPR - row_lo];
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) sc[u] = row_scale(chunk[u] / CPR);
    }

    int64_t off = off_tail;
#pragma unroll
    for (int k = 0; k < kOffsetLoads; ++k)
        off += (lane + 64u * k < b) ? max(lens[k], 0) : 0;
    off = wave_sum(off);
    // (the same in every lane: made scalar, so that the fit test below is a
    // wave-uniform branch)
    off = static_cast<int64_t>(
        (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off >> 32)))) << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off))));
    const int64_t out_row0 = (off + t0) * p.hkv;
    // Token-head rows of this block that still fit the output (may be <= 0).
    // A block that fits whole, the normal case, stores unconditionally.
    const int64_t room = p.out_th - out_row0;
    if (room >= static_cast<int64_t>(nrows / 2))
        gather_decode_store<HD, MODE, CB, U, NTS, false>(p, cw, sc, chunk, out_row0, 0);
    else
        gather_decode_store<HD, MODE, CB, U, NTS, true>(p, cw, sc, chunk, out_row0, room);
}

// ---------------------------------------------------------- static table

struct StaticValues {
    float v[2 * KVQ_MAX_STATIC_KV_HEADS];
};

__global__ void write_static_kernel(float* dst, StaticValues vals, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = vals.v[i];
}

// --------------------------------------------------------------- dispatch

// Default store tuning, chosen by measurement on MI355X (32768 tokens x 8 KV
// heads per call): 8 lanes per row, so every load instruction reads whole
// 128-byte lines of each row; more rows per lane for BF16 (no arithmetic to
// hide latency behind); non-temporal streams for data that one call touches
// once.  The gather's tuning is shared with the host (gather_tune).
template <int HD, int MODE>
struct Tune {
    static constexpr int store_epl = HD / 8;
    static constexpr int store_rpl = (MODE == KVQ_BF16) ? (HD == 64 ? 4 : 2) : 1;
    static constexpr bool store_nt_load = true;
    static constexpr bool store_nt_store = true;
    static constexpr bool store_contig = false;
    static constexpr int store_tpb = 256;
    static constexpr int gather_cb = gather_tune(HD, MODE).cb;
    static constexpr int gather_u = gather_tune(HD, MODE).u;
    static constexpr bool gather_nt_store = true;
    static constexpr bool gather_lds_scales = true;
    static constexpr int gather_tpb = gather_tune(HD, MODE).tpb;
};

StoreArgs make_store_args(const StoreLaunch& a) {
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
    p.order = a.order;
    p.num_tokens = static_cast<uint32_t>(a.num_rows / a.num_kv_heads);
    return p;
}

GatherArgs make_gather_args(const GatherLaunch& a) {
    GatherArgs p;
    p.layer = a.layer;
    p.static_scales = a.static_scales;
    p.block_table = a.block_table;
    p.seq_lens = a.seq_lens;
    p.out_k = static_cast<uint16_t*>(a.out_keys);
    p.out_v = static_cast<uint16_t*>(a.out_values);
    p.out_th = a.out_rows * a.num_kv_heads;
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
    p.parts = 1;
    return p;
}

template <int HD, int MODE, int EPL, int RPL, bool NTL, bool NTS, bool CONTIG, int TPB, bool ORD>
int launch_store_o(const StoreArgs& p, int64_t num_rows, int32_t num_kv_heads, void* stream) {
    constexpr int RPB = (64 / (HD / EPL)) * RPL * (TPB / 64);
    const uint32_t grid = static_cast<uint32_t>((num_rows + RPB - 1) / RPB);
    // static per-head tables of at most 32 KV heads are fetched whole by each wave
    if constexpr (MODE == KVQ_FP8_PER_HEAD) {
        if (num_kv_heads <= 32) {
            hipLaunchKernelGGL((store_kernel<HD, MODE, EPL, RPL, NTL, NTS, CONTIG, TPB, true, ORD>), dim3(grid),
                               dim3(TPB), 0, static_cast<hipStream_t>(stream), p);
            return static_cast<int>(hipGetLastError());
        }
    }
    hipLaunchKernelGGL((store_kernel<HD, MODE, EPL, RPL, NTL, NTS, CONTIG, TPB, false, ORD>), dim3(grid), dim3(TPB),
                       0, static_cast<hipStream_t>(stream), p);
    return static_cast<int>(hipGetLastError());
}

template <int HD, int MODE, int EPL, int RPL, bool NTL, bool NTS, bool CONTIG = false, int TPB = 256>
int launch_store_v(const StoreLaunch& a, void* stream) {
    const StoreArgs p = make_store_args(a);
    if constexpr (store_follows_order(HD, MODE)) {
        if (a.order != nullptr)
            return launch_store_o<HD, MODE, EPL, RPL, NTL, NTS, CONTIG, TPB, true>(p, a.num_rows, a.num_kv_heads,
                                                                                  stream);
    }
    return launch_store_o<HD, MODE, EPL, RPL, NTL, NTS, CONTIG, TPB, false>(p, a.num_rows, a.num_kv_heads, stream);
}

template <int HD, int MODE, int CB, int U, bool NTS, bool LDSS, int TPB = 256>
int launch_gather_v(const GatherLaunch& a, void* stream) {
    GatherArgs p = make_gather_args(a);
    p.parts = static_cast<uint32_t>(gather_parts(a.block_size, a.num_kv_heads, row_bytes(a.mode, HD), CB, U, TPB));
    const uint32_t grid = static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * a.max_blocks * p.parts);
    hipLaunchKernelGGL((gather_kernel<HD, MODE, CB, U, NTS, LDSS, TPB>), dim3(grid), dim3(TPB), 0,
                       static_cast<hipStream_t>(stream), p);
    return static_cast<int>(hipGetLastError());
}

template <int HD, int MODE>
int launch_store_t(const StoreLaunch& a, void* stream) {
    using T = Tune<HD, MODE>;
    return launch_store_v<HD, MODE, T::store_epl, T::store_rpl, T::store_nt_load, T::store_nt_store,
                          T::store_contig, T::store_tpb>(a, stream);
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
    using T = Tune<HD, MODE>;
    // A block that half a workgroup already covers (few KV heads, as on a
    // tensor-parallel shard) takes half the chunks per thread, so no lane
    // repeats another lane's chunk.  The grid is the same: one part per block.
    const int64_t chunks = static_cast<int64_t>(a.block_size) * a.num_kv_heads * 2 *
                           static_cast<int64_t>(row_bytes(a.mode, HD) / T::gather_cb);
    if constexpr (T::gather_u % 2 == 0) {
        if (2 * chunks <= static_cast<int64_t>(T::gather_tpb) * T::gather_u)
            return launch_gather_v<HD, MODE, T::gather_cb, T::gather_u / 2, T::gather_nt_store, T::gather_lds_scales,
                                   T::gather_tpb>(a, stream);
    }
    return launch_gather_v<HD, MODE, T::gather_cb, T::gather_u, T::gather_nt_store, T::gather_lds_scales,
                           T::gather_tpb>(a, stream);
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
