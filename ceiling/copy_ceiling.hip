// copy_ceiling.hip -- bandwidth ceilings for the benchmark (gfx950); not part
// of libkvq.so and never called by it.
//
// Two data movers with no arithmetic, timed beside the store so that its
// rate can be read against what the memory system gives the same traffic:
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
//
// Same launch shape as the store: 256 threads, 32 rows per workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
};

// HD elements per row, HALF: INT4-sized code rows (HD / 2 bytes), SC: an
// 8-byte scale pair per row in the block's trailer.
template <int HD, bool HALF, bool SC>
__global__ __launch_bounds__(256) void store_pattern_kernel(PatternArgs p) {
    constexpr int CPL = HD / 64;                  // 16-byte chunks per lane of a K (or V) row
    constexpr uint32_t HB = HALF ? HD / 2 : HD;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t sub = lane & 7u;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x >> 6) * 8 + (lane >> 3);
    const bool valid = row < p.num_rows;
    const uint32_t rowc = valid ? static_cast<uint32_t>(row) : 0u;
    u32x4 kx[CPL], vx[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        kx[k] = __builtin_nontemporal_load(p.keys + static_cast<uint64_t>(rowc) * (HD / 8) + k * 8 + sub);
        vx[k] = __builtin_nontemporal_load(p.values + static_cast<uint64_t>(rowc) * (HD / 8) + k * 8 + sub);
    }
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(rowc) * p.hkv_magic) >> p.hkv_shift);
    const uint32_t h = rowc - t * p.hkv;
    const int64_t slot = p.slots[t];
    if (!(valid && slot >= 0 && slot < p.num_slots)) return;
    const uint64_t blk = static_cast<uint64_t>(slot) >> p.bs_log2;
    const uint32_t pos = static_cast<uint32_t>(slot) & ((1u << p.bs_log2) - 1u);
    uint8_t* const bp = p.layer + blk * p.block_bytes;
    const uint32_t ph = pos * p.hkv + h;
    uint8_t* const krow = bp + static_cast<uint64_t>(ph) * (2 * HB);
    uint8_t* const vrow = krow + HB;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t c = k * 8 + sub;
        // the high byte of every BF16 element (8 bytes), or of every other one (4)
        const uint32_t k0 = __builtin_amdgcn_perm(kx[k][1], kx[k][0], 0x07050301u);
        const uint32_t k1 = __builtin_amdgcn_perm(kx[k][3], kx[k][2], 0x07050301u);
        const uint32_t v0 = __builtin_amdgcn_perm(vx[k][1], vx[k][0], 0x07050301u);
        const uint32_t v1 = __builtin_amdgcn_perm(vx[k][3], vx[k][2], 0x07050301u);
        if constexpr (HALF) {
            __builtin_nontemporal_store(k0 ^ k1, reinterpret_cast<uint32_t*>(krow + c * 4));
            __builtin_nontemporal_store(v0 ^ v1, reinterpret_cast<uint32_t*>(vrow + c * 4));
        } else {
            const u32x2 kk = {k0, k1}, vv = {v0, v1};
            __builtin_nontemporal_store(kk, reinterpret_cast<u32x2*>(krow + c * 8));
            __builtin_nontemporal_store(vv, reinterpret_cast<u32x2*>(vrow + c * 8));
        }
    }
    if constexpr (SC) {
        if (sub == 0) {
            const u32x2 sv = {kx[0][0], vx[0][0]};
            *reinterpret_cast<u32x2*>(bp + p.code_bytes + static_cast<uint64_t>(ph) * 8) = sv;
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

}  // namespace

extern "C" {

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
// num_blocks blocks of block_size tokens.  row_bytes = head_dim or head_dim / 2;
// scale_bytes = 8 (per-token-head trailer) or 0.  Returns 0, the launch's
// hipError_t, or -1 on bad arguments.
__attribute__((visibility("default"))) int ceil_store_pattern(const void* keys, const void* values,
                                                              const int64_t* slots, void* layer, int64_t num_tokens,
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

}  // extern "C"
