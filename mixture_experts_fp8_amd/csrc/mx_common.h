// Device helpers shared by the micro-scaled (one UE8M0 scale per 32 elements) kernels of
// k_mx.hip (16-row tiles) and k_ffn.hip (128-row tiles).
#pragma once

#include "moe_common.h"
#include "moe_plan.h"

namespace moe {

constexpr int kMx = 32;

// Smallest integer e with amax <= M * 2^e for M = 1.75 * 2^8 (E4M3) or 1.5 * 2^2 (E2M1),
// clamped to [-127, 127]; 0 for amax == 0.  Exact on the float32 bits: amax = 1.m * 2^(E-127).
template <int WF>
__device__ __forceinline__ int mx_scale_exponent(float amax) {
    const uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
    if (u == 0) return 0;
    const int E = (int)(u >> 23);
    if (E == 0) return -127;
    const uint32_t m = u & 0x7FFFFFu;
    const int e = WF == kWfmtE2M1 ? E - 129 + (m > 0x400000u ? 1 : 0) : E - 135 + (m > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Scaled matrix-core product with an E4M3 A operand and a B operand of format WF (the
// instruction's B-format field: 0 E4M3, 4 E2M1); one scale byte per lane and operand.
template <int WF>
__device__ __forceinline__ v4f mx_mfma(v8i a, v8i b, v4f acc, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, WF == kWfmtE2M1 ? 4 : 0, 0, sa, 0, sb);
}

}  // namespace moe
