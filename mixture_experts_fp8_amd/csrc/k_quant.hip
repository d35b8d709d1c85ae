// Quantisation and weight-layout kernels (gfx950).
//
// quant_act: E4M3 per (row, 128-column group) with a UE8M0 power-of-two scale, the
// activation scheme of the metrale "fp8_grouped_tc_w8a8.rs" page (module doc).  The
// same scale rule, applied per 128 x 128 block, quantises float32 expert weights.
#include "moe_common.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

// One 128-column group per 16 lanes; each lane owns 8 consecutive bf16 (16 bytes).
__global__ __launch_bounds__(256) void k_quant_act(const uint16_t* __restrict__ x, int rows, int cols,
                                                   int64_t ld, uint8_t* __restrict__ xq,
                                                   uint8_t* __restrict__ xs) {
    const int ngc = cols / kGroup;
    const int64_t ngroups = (int64_t)rows * ngc;
    const int sub = threadIdx.x & 15;
    const int64_t gstride = ((int64_t)gridDim.x * blockDim.x) >> 4;
    for (int64_t g = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4; g < ngroups; g += gstride) {
        const int64_t r = g / ngc;
        const int gc = (int)(g - r * ngc);
        quant_group16(x + r * ld + (int64_t)gc * kGroup, xq + r * cols + (int64_t)gc * kGroup, xs + r * ngc + gc, sub);
    }
}

// One 128 x 128 block of one expert per workgroup of 256 threads.  Thread t covers
// columns 4*(t%32) .. +3 of rows t/32 + 8*i, i < 16.
__global__ __launch_bounds__(256) void k_quant_weight_blocks(const float* __restrict__ w, int K, int N,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ s) {
    const int nbn = N / kGroup, nbk = K / kGroup;
    const int64_t blk = blockIdx.x;
    const int64_t e = blk / ((int64_t)nbk * nbn);
    const int kb = (int)((blk / nbn) % nbk);
    const int nb = (int)(blk % nbn);
    const int c4 = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const float* base = w + (e * K + (int64_t)kb * kGroup) * N + (int64_t)nb * kGroup + c4 * 4;
    float4 v[16];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = *reinterpret_cast<const float4*>(base + (int64_t)(r0 + 8 * i) * N);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    __shared__ float s_max[4];
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const int ex = scale_exponent(amax);
    uint8_t* qb = q + (e * K + (int64_t)kb * kGroup) * N + (int64_t)nb * kGroup + c4 * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t p = cvt4_e4m3(ldexpf(v[i].x, -ex), ldexpf(v[i].y, -ex), ldexpf(v[i].z, -ex),
                                     ldexpf(v[i].w, -ex));
        *reinterpret_cast<uint32_t*>(qb + (int64_t)(r0 + 8 * i) * N) = p;
    }
    if (threadIdx.x == 0) s[(e * nbk + kb) * nbn + nb] = (uint8_t)(ex + 127);
}

// Packed layout: 16-byte chunk id c = ((e*(N/16) + n16)*(K/128) + kb)*128 + h*64 + lane
// holds W[e][kb*128 + (lane/16)*32 + h*16 + b][n16*16 + lane%16], b < 16.
__global__ __launch_bounds__(256) void k_prepack(const uint8_t* __restrict__ w, int K, int N,
                                                 int64_t nchunks, uint8_t* __restrict__ out) {
    const int nkb = K / kGroup, nn16 = N / 16;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(c & 63);
        const int h = (int)((c >> 6) & 1);
        const int64_t blk = c >> 7;
        const int kb = (int)(blk % nkb);
        const int64_t en = blk / nkb;
        const int n16 = (int)(en % nn16);
        const int64_t e = en / nn16;
        const int k0 = kb * kGroup + (lane >> 4) * 32 + h * 16;
        const uint8_t* src = w + (e * K + k0) * N + n16 * 16 + (lane & 15);
        uint32_t d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[i] = (uint32_t)src[(int64_t)(4 * i) * N] | ((uint32_t)src[(int64_t)(4 * i + 1) * N] << 8) |
                   ((uint32_t)src[(int64_t)(4 * i + 2) * N] << 16) | ((uint32_t)src[(int64_t)(4 * i + 3) * N] << 24);
        }
        *reinterpret_cast<uint4*>(out + c * 16) = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                            hipStream_t st) {
    const int64_t threads = (int64_t)rows * (cols / kGroup) * 16;
    int blocks = (int)std::min<int64_t>(ceil_div(threads, 256), 16384);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_quant_act, dim3(blocks), dim3(256), 0, st, x, rows, cols, ld, xq, xs);
    return hipGetLastError();
}

hipError_t launch_quant_weight_blocks(const float* w, int E, int K, int N, uint8_t* q, uint8_t* s,
                                      hipStream_t st) {
    const int64_t blocks = (int64_t)E * (K / kGroup) * (N / kGroup);
    hipLaunchKernelGGL(k_quant_weight_blocks, dim3((unsigned)blocks), dim3(256), 0, st, w, K, N, q, s);
    return hipGetLastError();
}

hipError_t launch_prepack(const uint8_t* w, int E, int K, int N, uint8_t* out, hipStream_t st) {
    const int64_t nchunks = (int64_t)E * K * N / 16;
    const int blocks = (int)std::min<int64_t>(ceil_div(nchunks, 256), 65536);
    hipLaunchKernelGGL(k_prepack, dim3(blocks), dim3(256), 0, st, w, K, N, nchunks, out);
    return hipGetLastError();
}

}  // namespace moe
