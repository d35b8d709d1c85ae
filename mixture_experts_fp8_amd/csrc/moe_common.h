// Device helpers shared by the gfx950 kernels of the routed FP8 MoE step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 128;      // quantisation group / block edge
constexpr int kFragBytes = 2048; // one 16 x 128 E4M3 MFMA operand

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even float32 -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Scale exponent of a group: the smallest integer e with amax <= 448 * 2^e, clamped to
// [-127, 127]; 0 for amax == 0.  Exact integer logic on the float32 bits:
// amax = 1.m * 2^(E-127) and 448 = 1.75 * 2^8, so e = E - 135, plus one when the
// mantissa exceeds 1.75.  Subnormal amax (< 2^-126) needs e <= -135 and clamps to -127.
__device__ __forceinline__ int scale_exponent(float amax) {
    uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
    if (u == 0) return 0;
    int E = (int)(u >> 23);
    if (E == 0) return -127;
    int e = E - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two floats -> two E4M3FN bytes in the low 16 bits (round to nearest even; OCP format
// on gfx950; |v| <= 448 always holds after scaling).
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four floats -> four E4M3FN bytes.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Max over aligned groups of 16 lanes.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

// FP8 x FP8 16x16x128 matrix-core product with per-lane UE8M0 scales (byte 0 of sa / sb):
// lane l holds row (A) / column (B) l % 16 and K slots [32*(l/16), 32*(l/16)+32);
// acc lane l holds column l % 16, rows 4*(l/16) .. +3.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f acc, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
