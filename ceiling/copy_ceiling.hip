// copy_ceiling.hip -- bandwidth ceilings for the benchmark (gfx950); not part
// of libkvq.so and never called by it.
//
// Data movers with no arithmetic, timed beside the store and the gather so
// that their rates can be read against what the memory system gives the
// same traffic:
//
//  ceil_linear_copy    a non-temporal copy of `bytes` bytes: 16-byte loads
//                      and stores, 4 per thread, every instruction reading or
//                      writing whole 128-byte lines.
//  ceil_store_pattern  the store's exact accesses with the quantization left
//                      out: per (token, KV head) row, 16-byte non-temporal
//                      loads of the BF16 K and V rows (8 lanes per row, as
//                      the store kernel), the int64 slot, and writes of the
//                      row's code bytes (head_dim, or head_dim / 2 for INT4)
//                      and, for per-token-head layouts, its 8-byte scale pair,
//                      at the slot's (block, position, head) address of the
//                      cache layout.  The bytes written are a byte selection
//                      of the loaded ones, so nothing but data movement costs.
//                      Same launch shape as the store: 256 threads, 32 rows
//                      per workgroup.
//  ceil_gather_pattern the gather's exact accesses with the dequantization
//                      left out (block table, sequence offsets, code chunks
//                      and row scales of the paged blocks, BF16 output rows).
//  ceil_empty          a kernel that does nothing, for the fixed cost of one
//                      launch of a given grid (256-thread workgroups).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void empty_kernel() {}

__global__ __launch_bounds__(256) void linear_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          uint64_t n16) {
    const uint64_t base = static_cast<uint64_t>(blockIdx.x) * 1024 + threadIdx.x;
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t i = base + k * 256;
        v[k] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t i = base + k * 256;
        if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
    }
}

struct PatternArgs {
    const u32x4* __restrict__ keys;
    const u32x4* __restrict__ values;
    const int64_t* __restrict__ slots;
    uint8_t* __restrict__ layer;
    int64_t num_rows;
    int64_t num_slots;
    uint64_t block_bytes;
    uint32_t code_bytes;
    uint32_t hkv;
    uint32_t hkv_magic;
    uint32_t hkv_shift;
    uint32_t bs_log2;
    const int32_t* order;          // token order (nullptr: the tokens' own order)
};

// HD elements per row, HALF: INT4-sized code rows (HD / 2 bytes), SC: an
// 8-byte scale pair per row in the block's trailer.  A row's K and V code
// rows are 2 HB contiguous bytes of the block; the row's 8 lanes write them
// with 16-byte stores, store k of lane `sub` at byte 128 k + 16 sub, so that
// each store instruction writes whole 128-byte lines (8-byte stores at INT4
// head_dim 64, whose rows are 64 bytes).  Measured: 8-byte stores in the
// store kernel's chunk layout leave this copy 19% slower, and 16-byte stores
// of lane-contiguous 32-byte pieces (half lines per instruction) 6% slower.
template <int HD, bool HALF, bool SC>
__global__ __launch_bounds__(256) void store_pattern_kernel(PatternArgs p) {
    constexpr int CPL = HD / 64;                  // 16-byte chunks per lane of a K (or V) row
    constexpr uint32_t HB = HALF ? HD / 2 : HD;
    constexpr int LW = 2 * HB / 8;                // bytes this lane writes per row
    constexpr int OUTW = LW / 4;                  // ... as dwords
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t sub = lane & 7u;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x >> 6) * 8 + (lane >> 3);
    const bool valid = row < p.num_rows;
    uint32_t rowc = valid ? static_cast<uint32_t>(row) : 0u;
    if (p.order != nullptr) {
        // the same token order as the store's: row i * Hkv + h is token order[i]'s head h
        const uint32_t i = static_cast<uint32_t>((static_cast<uint64_t>(rowc) * p.hkv_magic) >> p.hkv_shift);
        rowc = static_cast<uint32_t>(p.order[i]) * p.hkv + (rowc - i * p.hkv);
    }
    uint32_t in[8 * CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const u32x4 kv = __builtin_nontemporal_load(p.keys + static_cast<uint64_t>(rowc) * (HD / 8) + k * 8 + sub);
        const u32x4 vv = __builtin_nontemporal_load(p.values + static_cast<uint64_t>(rowc) * (HD / 8) + k * 8 + sub);
        in[4 * k] = kv[0]; in[4 * k + 1] = kv[1]; in[4 * k + 2] = kv[2]; in[4 * k + 3] = kv[3];
        in[4 * CPL + 4 * k] = vv[0]; in[4 * CPL + 4 * k + 1] = vv[1];
        in[4 * CPL + 4 * k + 2] = vv[2]; in[4 * CPL + 4 * k + 3] = vv[3];
    }
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(rowc) * p.hkv_magic) >> p.hkv_shift);
    const uint32_t h = rowc - t * p.hkv;
    const int64_t slot = p.slots[t];
    if (!(valid && slot >= 0 && slot < p.num_slots)) return;
    const uint64_t blk = static_cast<uint64_t>(slot) >> p.bs_log2;
    const uint32_t pos = static_cast<uint32_t>(slot) & ((1u << p.bs_log2) - 1u);
    uint8_t* const bp = p.layer + blk * p.block_bytes;
    const uint32_t ph = pos * p.hkv + h;
    uint8_t* const rowp = bp + static_cast<uint64_t>(ph) * (2 * HB);
    // the high byte of every BF16 value (FP8-sized rows), or of every other
    // one combined (INT4-sized rows): a byte selection, no arithmetic
    uint32_t out[OUTW];
#pragma unroll
    for (int w = 0; w < OUTW; ++w) {
        if constexpr (HALF)
            out[w] = __builtin_amdgcn_perm(in[4 * w + 1], in[4 * w], 0x07050301u) ^
                     __builtin_amdgcn_perm(in[4 * w + 3], in[4 * w + 2], 0x07050301u);
        else
            out[w] = __builtin_amdgcn_perm(in[2 * w + 1], in[2 * w], 0x07050301u);
    }
    if constexpr (LW >= 16) {
#pragma unroll
        for (int w = 0; w < OUTW; w += 4) {
            const u32x4 v = {out[w], out[w + 1], out[w + 2], out[w + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(rowp + 128 * (w / 4) + 16 * sub));
        }
    } else {
        const u32x2 v = {out[0], out[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(rowp + 8 * sub));
    }
    if constexpr (SC) {
        if (sub == 0) {
            const u32x2 sv = {in[0], in[4 * CPL]};
            *reinterpret_cast<u32x2*>(bp + p.code_bytes + static_cast<uint64_t>(ph) * 8) = sv;
        }
    }
}

struct GatherPatternArgs {
    const uint8_t* __restrict__ layer;
    const int32_t* __restrict__ block_table;
    const int32_t* __restrict__ seq_lens;
    uint16_t* __restrict__ out_k;
    uint16_t* __restrict__ out_v;
    int64_t num_blocks;
    uint64_t block_bytes;
    uint32_t code_bytes;
    uint32_t hkv;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t block_size;
    uint32_t parts;
};

// The gather's accesses with the dequantization left out: one workgroup per
// (sequence, logical block, part), CB code bytes per thread chunk (U chunks
// per thread), each chunk's row scale, the block-table entry and the
// sequence offsets, and the chunk's BF16 output (2 bytes per element) at the
// packed output row, written with 16-byte non-temporal stores.
template <int HD, bool HALF, bool SC, int CB, int U>
__global__ __launch_bounds__(256) void gather_pattern_kernel(GatherPatternArgs p) {
    constexpr uint32_t HB = HALF ? HD / 2 : HD;
    constexpr uint32_t CPR = HB / CB;              // chunks per row
    constexpr int EPC = HALF ? 2 * CB : CB;        // output elements per chunk
    constexpr int ODW = EPC / 2;                   // output dwords per chunk
    const uint32_t wg = blockIdx.x;
    const uint32_t bj = wg / p.parts, part = wg - bj * p.parts;
    const uint32_t b = bj / static_cast<uint32_t>(p.max_blocks);
    const uint32_t j = bj - b * static_cast<uint32_t>(p.max_blocks);
    const int32_t raw_len = p.seq_lens[b];
    const int32_t pb = p.block_table[static_cast<int64_t>(b) * p.max_blocks + j];
    const int64_t len = min<int64_t>(max(raw_len, 0), static_cast<int64_t>(p.max_blocks) * p.block_size);
    const int64_t t0 = static_cast<int64_t>(j) * p.block_size;
    if (t0 >= len || pb < 0 || pb >= p.num_blocks) return;
    const uint32_t ntok = static_cast<uint32_t>(min<int64_t>(p.block_size, len - t0));
    const uint32_t nchunks = ntok * p.hkv * 2 * CPR;
    const uint32_t c0 = part * (256 * U);
    if (c0 >= nchunks) return;
    const uint32_t lane = threadIdx.x & 63u;
    int64_t off = 0;
    for (uint32_t i = lane; i < b; i += 64) off += max(p.seq_lens[i], 0);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) off += __shfl_xor(off, m, 64);
    const uint8_t* const bp = p.layer + static_cast<uint64_t>(pb) * p.block_bytes;
    uint32_t w[U][CB / 4];
    uint32_t sc[U];
    uint32_t chunk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        chunk[u] = min(c0 + threadIdx.x + u * 256, nchunks - 1);
        const uint8_t* src = bp + static_cast<uint64_t>(chunk[u]) * CB;
        if constexpr (CB == 8) {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
            w[u][0] = v[0]; w[u][1] = v[1];
        } else {
            w[u][0] = *reinterpret_cast<const uint32_t*>(src);
        }
        sc[u] = SC ? reinterpret_cast<const uint32_t*>(bp + p.code_bytes)[chunk[u] / CPR] : 0u;
    }
    const int64_t out_row0 = (off + t0) * p.hkv;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t row = chunk[u] / CPR, col = chunk[u] % CPR;
        uint16_t* const outp = ((row & 1u) ? p.out_v : p.out_k) + static_cast<uint64_t>(out_row0 + (row >> 1)) * HD +
                               col * EPC;
        uint32_t o[ODW];
#pragma unroll
        for (int d = 0; d < ODW; ++d) {
            // each code byte (or nibble pair) becomes the high byte of a BF16 value
            const uint32_t x = w[u][(d * 4) / (HALF ? 8 : 4) % (CB / 4)];
            // (selector byte 12 gives 0x00; 4..7 are the bytes of x)
            o[d] = __builtin_amdgcn_perm(x, 0u, (d % 2) ? 0x070C060Cu : 0x050C040Cu) ^ sc[u];
        }
#pragma unroll
        for (int q = 0; q < ODW / 4; ++q) {
            const u32x4 v = {o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outp + 8 * q));
        }
    }
}

// n / d == (n * magic) >> shift for n < 2^31 (Granlund & Montgomery, PLDI 1994).
void div_magic(uint32_t d, uint32_t* magic, uint32_t* shift) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint32_t s = 31 + l;
    const unsigned __int128 num = static_cast<unsigned __int128>(1) << s;
    *magic = static_cast<uint32_t>((num + d - 1) / d);
    *shift = s;
}

template <int HD>
void launch_pattern(const PatternArgs& p, bool half, bool sc, uint32_t grid, hipStream_t st) {
    if (half) {
        if (sc) hipLaunchKernelGGL((store_pattern_kernel<HD, true, true>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((store_pattern_kernel<HD, true, false>), dim3(grid), dim3(256), 0, st, p);
    } else {
        if (sc) hipLaunchKernelGGL((store_pattern_kernel<HD, false, true>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((store_pattern_kernel<HD, false, false>), dim3(grid), dim3(256), 0, st, p);
    }
}

template <int HD>
void launch_gather_pattern(const GatherPatternArgs& p, bool half, bool sc, uint32_t grid, hipStream_t st) {
    if (half) {
        if (sc) hipLaunchKernelGGL((gather_pattern_kernel<HD, true, true, 4, 8>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((gather_pattern_kernel<HD, true, false, 4, 8>), dim3(grid), dim3(256), 0, st, p);
    } else {
        if (sc) hipLaunchKernelGGL((gather_pattern_kernel<HD, false, true, 8, 4>), dim3(grid), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((gather_pattern_kernel<HD, false, false, 8, 4>), dim3(grid), dim3(256), 0, st, p);
    }
}

}  // namespace

extern "C" {

// Launch `grid` (1 .. 2^31 - 1) workgroups of 256 threads that do nothing.
// Returns 0 or the hipError_t of the launch; -1 on bad arguments.
__attribute__((visibility("default"))) int ceil_empty(int64_t grid, void* stream) {
    if (grid < 1 || grid >= (int64_t{1} << 31)) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, static_cast<hipStream_t>(stream));
    return static_cast<int>(hipGetLastError());
}

// Copy `bytes` (a multiple of 16, > 0) from src to dst (device, 16-byte
// aligned).  Returns 0 or the hipError_t of the launch; -1 on bad arguments.
__attribute__((visibility("default"))) int ceil_linear_copy(const void* src, void* dst, uint64_t bytes,
                                                            void* stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0) return -1;
    const uint64_t n16 = bytes / 16;
    const uint64_t grid = (n16 + 1023) / 1024;
    if (grid >= (uint64_t{1} << 31)) return -1;
    hipLaunchKernelGGL(linear_copy_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return static_cast<int>(hipGetLastError());
}

// The store's access pattern for num_tokens rows of num_kv_heads heads:
// keys/values BF16 [num_tokens][num_kv_heads][head_dim] (device, 16-byte
// aligned), slots int64 [num_tokens], layer = the layer's first block (device),
// num_blocks blocks of block_size tokens; order NULL (the tokens in their own
// order) or a permutation of 0 .. num_tokens-1 (device int32: the tokens in
// that order, as kvq_store_ordered takes them).  row_bytes = head_dim or
// head_dim / 2; scale_bytes = 8 (per-token-head trailer) or 0.  Returns 0,
// the launch's hipError_t, or -1 on bad arguments.
__attribute__((visibility("default"))) int ceil_store_pattern(const void* keys, const void* values,
                                                              const int64_t* slots, const int32_t* order,
                                                              void* layer, int64_t num_tokens,
                                                              int32_t num_kv_heads, int32_t head_dim,
                                                              int32_t row_bytes, int32_t scale_bytes,
                                                              int32_t block_size, int64_t num_blocks, void* stream) {
    if (!keys || !values || !slots || !layer || num_tokens < 1 || num_kv_heads < 1 || num_blocks < 1) return -1;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return -1;
    if (row_bytes != head_dim && row_bytes != head_dim / 2) return -1;
    if (scale_bytes != 0 && scale_bytes != 8) return -1;
    if (block_size < 1 || (block_size & (block_size - 1)) != 0) return -1;
    const int64_t rows = num_tokens * num_kv_heads;
    if (rows >= (int64_t{1} << 31)) return -1;
    PatternArgs p;
    p.keys = static_cast<const u32x4*>(keys);
    p.values = static_cast<const u32x4*>(values);
    p.slots = slots;
    p.order = order;
    p.layer = static_cast<uint8_t*>(layer);
    p.num_rows = rows;
    p.num_slots = num_blocks * block_size;
    p.code_bytes = static_cast<uint32_t>(block_size) * num_kv_heads * 2 * row_bytes;
    p.block_bytes = p.code_bytes + (scale_bytes ? static_cast<uint64_t>(block_size) * num_kv_heads * 8 : 0);
    p.hkv = static_cast<uint32_t>(num_kv_heads);
    div_magic(p.hkv, &p.hkv_magic, &p.hkv_shift);
    p.bs_log2 = 0;
    while ((1 << p.bs_log2) < block_size) ++p.bs_log2;
    const uint32_t grid = static_cast<uint32_t>((rows + 31) / 32);
    const bool half = row_bytes != head_dim, sc = scale_bytes != 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    switch (head_dim) {
        case 64: launch_pattern<64>(p, half, sc, grid, st); break;
        case 128: launch_pattern<128>(p, half, sc, grid, st); break;
        default: launch_pattern<256>(p, half, sc, grid, st); break;
    }
    return static_cast<int>(hipGetLastError());
}

// The gather's access pattern over one layer: block_table int32
// [num_seqs][max_blocks], seq_lens int32 [num_seqs] (device), out_keys and
// out_values BF16 [sum(seq_lens)][num_kv_heads][head_dim] (device, 16-byte
// aligned), layer = the layer's first block of num_blocks; row_bytes and
// scale_bytes as for ceil_store_pattern.  Chunks of 8 code bytes (4 for
// INT4-sized rows), 4 (8) per thread, 256 threads per workgroup, as the
// gather.  Returns 0, the launch's hipError_t, or -1 on bad arguments.
__attribute__((visibility("default"))) int ceil_gather_pattern(const void* layer, const int32_t* block_table,
                                                               int32_t max_blocks, const int32_t* seq_lens,
                                                               int32_t num_seqs, void* out_keys, void* out_values,
                                                               int32_t num_kv_heads, int32_t head_dim,
                                                               int32_t row_bytes, int32_t scale_bytes,
                                                               int32_t block_size, int64_t num_blocks, void* stream) {
    if (!layer || !block_table || !seq_lens || !out_keys || !out_values) return -1;
    if (num_seqs < 1 || max_blocks < 1 || num_kv_heads < 1 || num_blocks < 1) return -1;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return -1;
    if (row_bytes != head_dim && row_bytes != head_dim / 2) return -1;
    if (scale_bytes != 0 && scale_bytes != 8) return -1;
    if (block_size < 1 || (block_size & (block_size - 1)) != 0) return -1;
    const bool half = row_bytes != head_dim, sc = scale_bytes != 0;
    const int cb = half ? 4 : 8, u = half ? 8 : 4;
    GatherPatternArgs p;
    p.layer = static_cast<const uint8_t*>(layer);
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.out_k = static_cast<uint16_t*>(out_keys);
    p.out_v = static_cast<uint16_t*>(out_values);
    p.num_blocks = num_blocks;
    p.code_bytes = static_cast<uint32_t>(block_size) * num_kv_heads * 2 * row_bytes;
    p.block_bytes = p.code_bytes + (sc ? static_cast<uint64_t>(block_size) * num_kv_heads * 8 : 0);
    p.hkv = static_cast<uint32_t>(num_kv_heads);
    p.max_blocks = max_blocks;
    p.num_seqs = num_seqs;
    p.block_size = block_size;
    const int64_t chunks = static_cast<int64_t>(block_size) * num_kv_heads * 2 * (row_bytes / cb);
    p.parts = static_cast<uint32_t>((chunks + 256 * u - 1) / (256 * u));
    const int64_t grid = static_cast<int64_t>(num_seqs) * max_blocks * p.parts;
    if (grid >= (int64_t{1} << 31)) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    switch (head_dim) {
        case 64: launch_gather_pattern<64>(p, half, sc, static_cast<uint32_t>(grid), st); break;
        case 128: launch_gather_pattern<128>(p, half, sc, static_cast<uint32_t>(grid), st); break;
        default: launch_gather_pattern<256>(p, half, sc, static_cast<uint32_t>(grid), st); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
