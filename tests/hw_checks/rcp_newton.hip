// Device check of the scale arithmetic the store kernel relies on: rcp_exact
// against the IEEE reciprocal on every normal FP32 input of a range, and
// div_by_const<448 / 7> against IEEE division on every BF16 magnitude >= 2^-100.
// Test infrastructure: loaded only by tests/test_gpu_hw_checks.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_exact.h"

namespace {

constexpr int kBlocks = 4096;
constexpr int kThreads = 256;

// Each thread counts its own mismatches; counts[i] has one slot per thread.
__global__ void rcp_kernel(uint32_t lo, uint32_t n, uint32_t* counts) {
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    uint32_t bad = 0;
    for (uint32_t i = tid; i < n; i += kBlocks * kThreads) {
        const float s = __uint_as_float(lo + i);
        bad += __float_as_uint(kvq::rcp_exact(s)) != __float_as_uint(1.0f / s);
    }
    counts[tid] = bad;
}

template <int Q>
__global__ void cdiv_kernel(uint32_t* counts) {
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    uint32_t bad = 0;
    if (tid >= 1 && tid < 0x7F80u) {
        const float a = __uint_as_float(tid << 16);
        if (a >= 0x1p-100f)
            bad = __float_as_uint(kvq::div_by_const<Q>(a)) != __float_as_uint(a / static_cast<float>(Q));
    }
    counts[tid] = bad;
}

uint64_t sum_counts(const uint32_t* d, int n, int* err) {
    uint32_t* h = new uint32_t[n];
    *err = static_cast<int>(hipMemcpy(h, d, sizeof(uint32_t) * n, hipMemcpyDeviceToHost));
    uint64_t t = 0;
    for (int i = 0; i < n; ++i) t += h[i];
    delete[] h;
    return t;
}

}  // namespace

extern "C" {

// Mismatches of rcp_exact over FP32 bit patterns [lo_bits, hi_bits).
// Returns 0 or a hipError_t value.
__attribute__((visibility("default"))) int kvq_hw_rcp_mismatches(uint32_t lo_bits, uint32_t hi_bits,
                                                                 uint64_t* out) {
    uint32_t* d = nullptr;
    const int n = kBlocks * kThreads;
    int e = static_cast<int>(hipMalloc(&d, sizeof(uint32_t) * n));
    if (e) return e;
    hipLaunchKernelGGL(rcp_kernel, dim3(kBlocks), dim3(kThreads), 0, 0, lo_bits, hi_bits - lo_bits, d);
    e = static_cast<int>(hipDeviceSynchronize());
    if (!e) *out = sum_counts(d, n, &e);
    hipFree(d);
    return e;
}

// Mismatches of div_by_const<q> over all BF16 magnitudes >= 2^-100; q is 448 or 7.
__attribute__((visibility("default"))) int kvq_hw_cdiv_mismatches(int q, uint64_t* out) {
    uint32_t* d = nullptr;
    const int blocks = (0x7F80 + kThreads - 1) / kThreads;
    const int n = blocks * kThreads;
    int e = static_cast<int>(hipMalloc(&d, sizeof(uint32_t) * n));
    if (e) return e;
    if (q == 448) hipLaunchKernelGGL(cdiv_kernel<448>, dim3(blocks), dim3(kThreads), 0, 0, d);
    else hipLaunchKernelGGL(cdiv_kernel<7>, dim3(blocks), dim3(kThreads), 0, 0, d);
    e = static_cast<int>(hipDeviceSynchronize());
    if (!e) *out = sum_counts(d, n, &e);
    hipFree(d);
    return e;
}

}  // extern "C"
