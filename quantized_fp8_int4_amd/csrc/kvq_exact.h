// kvq_exact.h -- device helpers for correctly rounded FP32 scale arithmetic.
// Shared by the kernels and by the device test that checks them exhaustively
// on gfx950 (tests/hw_checks/rcp_newton.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// RN(1 / s) for a normal s: the hardware reciprocal (within 1 ulp) and one
// Newton step with FMA.  On gfx950 this equals the IEEE quotient 1 / s for
// every normal FP32 input (checked exhaustively on the device).
__device__ __forceinline__ float rcp_exact(float s) {
    const float y = __builtin_amdgcn_rcpf(s);
    const float e = fmaf(-s, y, 1.0f);
    return fmaf(e, y, y);
}

// RN(a / Q) for a >= 2^-100 (the quotient is then normal): s0 = RN(a *
// RN(1/Q)) and one Markstein correction (P. Markstein, IBM J. R&D 34(1),
// 1990: exact when the reciprocal of Q is correctly rounded and nothing is
// subnormal).  Checked against IEEE division for every BF16 a in range, for
// Q = 448 and 7.
template <int Q>
__device__ __forceinline__ float div_by_const(float a) {
    constexpr float q = static_cast<float>(Q);
    constexpr float c = 1.0f / q;
    const float s0 = a * c;
    const float e = fmaf(-s0, q, a);
    return fmaf(e, c, s0);
}

}  // namespace kvq
