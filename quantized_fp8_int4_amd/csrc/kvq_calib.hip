// kvq_calib.hip -- on-the-fly calibration for the static scale layouts: the
// running absolute maximum of K and V per KV head over warmup batches
// ("Per-tensor vs per-head FP8 KV cache scales", "Calibration changes which
// scale layout exists").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

// ------------------------------------------------------------ calibration

struct CalibArgs {
    const uint4* __restrict__ keys;
    const uint4* __restrict__ values;
    uint32_t* __restrict__ amax;   // FP32 bits of non-negative maxima
    int64_t num_rows;
    uint32_t hkv;
    uint32_t hkv_magic;
    uint32_t hkv_shift;
};

// Running absolute maximum per (K/V, KV head).  Rows are read with the store
// kernel's layout (8 lanes per row, whole 128-byte lines per instruction);
// each row's maximum goes into a per-workgroup LDS table with an LDS atomic
// max, and each workgroup then merges its table into amax with one global
// atomic max per entry.  Non-negative FP32 values order like their bits.
template <int HD, int RPL>
__global__ __launch_bounds__(256) void calib_kernel(CalibArgs p) {
    constexpr int LPR = 8;
    constexpr int CPL = HD / (8 * LPR);
    constexpr int RPW = 64 / LPR;
    constexpr int RPB = RPW * 4;
    __shared__ uint32_t smax[2 * KVQ_MAX_STATIC_KV_HEADS];
    for (uint32_t i = threadIdx.x; i < 2 * p.hkv; i += 256) smax[i] = 0;
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t sub = lane % LPR;
    // each iteration covers RPL groups of RPB rows; all of a lane's loads for
    // the iteration go out before any row is reduced
    const int64_t supers = (p.num_rows + RPB * RPL - 1) / (RPB * RPL);
    for (int64_t g = blockIdx.x; g < supers; g += gridDim.x) {
        uint4 kx[RPL][CPL], vx[RPL][CPL];
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int64_t row = (g * RPL + j) * RPB + wave * RPW + lane / LPR;
            const uint64_t rowc = row < p.num_rows ? static_cast<uint64_t>(row) : 0u;
            const uint4* kp = p.keys + rowc * (HD / 8) + sub;
            const uint4* vp = p.values + rowc * (HD / 8) + sub;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                kx[j][k] = ld16<true>(kp + k * LPR);
                vx[j][k] = ld16<true>(vp + k * LPR);
            }
        }
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int64_t row = (g * RPL + j) * RPB + wave * RPW + lane / LPR;
            u16x2 ak = {0, 0}, av = {0, 0};
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                ak = absmax_chunk(kx[j][k], ak);
                av = absmax_chunk(vx[j][k], av);
            }
            const uint32_t mk = row_max<LPR>(umax(ak.x, ak.y)) << 16;
            const uint32_t mv = row_max<LPR>(umax(av.x, av.y)) << 16;
            if (row < p.num_rows && sub == 0) {
                const uint32_t r32 = static_cast<uint32_t>(row);
                const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(r32) * p.hkv_magic) >> p.hkv_shift);
                const uint32_t h = r32 - t * p.hkv;
                atomicMax(&smax[h], mk);
                atomicMax(&smax[p.hkv + h], mv);
            }
        }
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < 2 * p.hkv; i += 256)
        if (smax[i] != 0) atomicMax(&p.amax[i], smax[i]);
}

__global__ void zero_kernel(uint32_t* dst, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = 0;
}

}  // namespace

int launch_calibrate(const CalibLaunch& a, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int n = 2 * a.num_kv_heads;
    if (!a.accumulate) {
        hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(a.amax), n);
        const int e = static_cast<int>(hipGetLastError());
        if (e != 0 || a.num_rows == 0) return e;
    }
    if (a.num_rows == 0) return 0;
    CalibArgs p;
    p.keys = static_cast<const uint4*>(a.keys);
    p.values = static_cast<const uint4*>(a.values);
    p.amax = reinterpret_cast<uint32_t*>(a.amax);
    p.num_rows = a.num_rows;
    p.hkv = static_cast<uint32_t>(a.num_kv_heads);
    const DivMagic dm = div_magic(p.hkv);
    p.hkv_magic = dm.magic;
    p.hkv_shift = dm.shift;
    // 8 rows per lane per iteration (32 KiB of loads in flight per wave) on
    // at most 256 workgroups that loop: measured on the GQA-32 prefill, 23.8
    // us per call against 24.9 for 4 rows on 512 workgroups, and 2048
    // workgroups of one iteration each took 34 us.  (The final global
    // atomics, 2 * Hkv per workgroup, cost under half a microsecond per call
    // at 256 workgroups.)
    constexpr int kCalibRpl = 8;
    constexpr int64_t kCalibMaxGrid = 256;
    const int64_t supers = (a.num_rows + 32 * kCalibRpl - 1) / (32 * kCalibRpl);
    const uint32_t grid = static_cast<uint32_t>(supers < kCalibMaxGrid ? supers : kCalibMaxGrid);
    switch (a.head_dim) {
        case 64: hipLaunchKernelGGL((calib_kernel<64, kCalibRpl>), dim3(grid), dim3(256), 0, st, p); break;
        case 128: hipLaunchKernelGGL((calib_kernel<128, kCalibRpl>), dim3(grid), dim3(256), 0, st, p); break;
        default: hipLaunchKernelGGL((calib_kernel<256, kCalibRpl>), dim3(grid), dim3(256), 0, st, p); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
