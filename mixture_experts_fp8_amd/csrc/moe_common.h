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
    // branch-free: 0 for amax == 0, -127 for subnormal amax, else the clamped exponent
    const uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
    const int E = (int)(u >> 23);
    const int e = E - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    const int r = E == 0 ? (u == 0 ? 0 : -127) : e;
    return min(max(r, -127), 127);
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

// Lane exchange inside rows of 16 lanes by a DPP control word (a VALU operand modifier, no
// LDS round trip as with ds_bpermute): 0xB1 swaps neighbours, 0x4E swaps pairs within a
// quad, 0x124 / 0x128 rotate the row by 4 / 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Wave64 reductions (all 64 lanes active): a butterfly inside each row of 16 lanes by DPP
// (neighbours, pairs, rotations by 4 and 8), then the four row results read from lanes 0,
// 16, 32, 48 and combined as (r0 . r1) . (r2 . r3); the result is uniform.
template <typename Op>
__device__ __forceinline__ float wave_reduce_f32(float v, Op op) {
    v = op(v, dpp_f32<0xB1>(v));
    v = op(v, dpp_f32<0x4E>(v));
    v = op(v, dpp_f32<0x124>(v));
    v = op(v, dpp_f32<0x128>(v));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0)), r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32)), r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce_f32(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce_f32(v, [](float x, float y) { return x + y; });
}

// Max over aligned groups of 16 lanes (the hardware rows): within quads, then across the
// four quads by rotating the row by 4 and 8 lanes.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x124>(v));
    v = fmaxf(v, dpp_f32<0x128>(v));
    return v;
}

// FP8 x FP8 16x16x128 matrix-core product with per-lane UE8M0 scales (byte 0 of sa / sb):
// lane l holds row (A) / column (B) l % 16 and K slots [32*(l/16), 32*(l/16)+32);
// acc lane l holds column l % 16, rows 4*(l/16) .. +3.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f acc, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
}

// Quantise one 128-column bf16 group held by 16 consecutive lanes (lane `sub` owns
// elements 8*sub .. 8*sub+7, passed in v): E4M3 bytes to dq[8*sub ..], the UE8M0 scale
// byte to *ds (written by sub == 0).  All 16 lanes of the group must be active.
__device__ __forceinline__ void quant_group16_v(const uint4 v, uint8_t* __restrict__ dq, uint8_t* __restrict__ ds,
                                                int sub) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = max16(amax);
    const int e = scale_exponent(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = ldexpf(f[i], -e);
    uint2 q;
    q.x = cvt4_e4m3(f[0], f[1], f[2], f[3]);
    q.y = cvt4_e4m3(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<uint2*>(dq + sub * 8) = q;
    if (sub == 0) *ds = (uint8_t)(e + 127);
}

__device__ __forceinline__ void quant_group16(const uint16_t* __restrict__ src, uint8_t* __restrict__ dq,
                                              uint8_t* __restrict__ ds, int sub) {
    quant_group16_v(*reinterpret_cast<const uint4*>(src + sub * 8), dq, ds, sub);
}

// Raw buffer resource over [base, base + bytes): loads take one per-lane 32-bit offset
// (VGPR) plus a wave-uniform offset (SGPR); reads past `bytes` return zero.  A resource
// lives in scalar registers, so base and bytes must be wave-uniform; they are passed through
// readfirstlane so the compiler knows it and never wraps the loads in a waterfall loop.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Cache policy of the weight-stream loads: 2 = non-temporal (each weight byte is read once
// per step; keeping it out of the caches leaves them to the activations and router tensors).
#ifndef MOE_WLOAD_AUX
#define MOE_WLOAD_AUX 2
#endif

// One 2 KB matrix-core operand in packed order: lane l's 32 bytes are the 16 at
// soff + 16*l and the 16 at soff + 1024 + 16*l.
__device__ __forceinline__ v8i buf_frag(rsrc_t r, uint32_t lane16, uint32_t soff) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, lane16, soff, MOE_WLOAD_AUX);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, lane16, soff + 1024, MOE_WLOAD_AUX);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 32 contiguous bytes at voff + soff.
__device__ __forceinline__ v8i buf_a32(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16, 0);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Test output of the gate+up epilogues (kernels built with TAP): the float32 h of row `row` of
// an item whose rows start at sorted row `rowbase` (rows past nvalid are padding), column
// `col` of h, into htap [A, I].
template <bool TAP>
__device__ __forceinline__ void tap_h(float* htap, int I, int rowbase, int row, int nvalid, int col, float h) {
    if constexpr (TAP) {
        if (row < nvalid) htap[(int64_t)(rowbase + row) * I + col] = h;
    }
}

// Optional per-expert biases, float32, NULL for none: b13 [E, 2I] (gate columns, then up
// columns) is added to the gate and up sums before SwiGLU, b2 [E, H] to the down GEMM's output
// row.  Without biases the sums pass through unchanged (no +0 is added).
struct GuBias {
    float g, u;
};
__device__ __forceinline__ GuBias gu_bias(const float* b13, int e, int I, int col) {
    if (!b13) return GuBias{0.f, 0.f};
    const float* p = b13 + (int64_t)e * 2 * I + col;
    return GuBias{p[0], p[I]};
}
__device__ __forceinline__ float add_bias(const float* b, float v, float bv) { return b ? v + bv : v; }
__device__ __forceinline__ float out_bias(const float* b2, int e, int H, int col) {
    return b2 ? b2[(int64_t)e * H + col] : 0.f;
}

// Work order of the 128-row-tile GEMMs (items = tile x column block).  The workgroups of
// one XCD share its L2; all XCDs share the Infinity Cache.  Items come in super-tiles of
// 8 consecutive tiles x 4 column blocks (32 items, one per workgroup running on an XCD, so
// an XCD fetches 8 A tiles and 4 weight column blocks for 32 items).  Super-tiles go to the
// XCDs in windows of 8 consecutive tile groups: within a window XCD x takes tile group x, and
// all XCDs step through the column groups together, so at any time the 8 XCDs work on 64
// consecutive tiles (mostly one expert) and the same weight columns, which the Infinity
// Cache then serves from one HBM read.  Rank r of XCD x -> item (tile, col); false for the
// holes past the last tile or column.
#ifndef MOE_ORD_TILES
#define MOE_ORD_TILES 8
#endif
#ifndef MOE_ORD_COLS
#define MOE_ORD_COLS 4
#endif
constexpr int kOrdTiles = MOE_ORD_TILES, kOrdCols = MOE_ORD_COLS, kOrdXcds = 8, kOrdSlots = kOrdTiles * kOrdCols;
__host__ __device__ inline int ord_ranks(int ntiles, int ncol) {
    const int ngroups = (ntiles + kOrdTiles - 1) / kOrdTiles;
    const int nwin = (ngroups + kOrdXcds - 1) / kOrdXcds;
    return nwin * ((ncol + kOrdCols - 1) / kOrdCols) * kOrdSlots;
}
__host__ __device__ inline bool ord_item(int x, int r, int ntiles, int ncol, int& tile, int& col) {
    const int ncg = (ncol + kOrdCols - 1) / kOrdCols;
    const int s = r / kOrdSlots, j = r - s * kOrdSlots;
    const int win = s / ncg, cg = s - win * ncg;
    tile = (win * kOrdXcds + x) * kOrdTiles + j % kOrdTiles;
    col = cg * kOrdCols + j / kOrdTiles;
    return tile < ntiles && col < ncol;
}

}  // namespace moe
