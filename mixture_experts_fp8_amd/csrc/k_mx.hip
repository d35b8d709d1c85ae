// Micro-scaled variants of the expert step (gfx950): one UE8M0 scale per 32 elements.
//
//   MXFP8  E4M3 activations and weights (MindIE-SD "Fused MoE", section "MXFP8 dynamic
//          quant MoE": E4M3 weights with MX scales; the MATE Mega MoE recipe (1, 1, 32));
//   W4A8   the same activations with E2M1 (FP4) weights (the FP8 x FP4 Mega MoE path of the
//          DeepGEMM pull request, "weights switch from e2m1 to e4m3" for its W8A8 variant).
// Groups: activations and the re-quantised SwiGLU output per (row, 32 columns); weights per
// (32 rows of K, one column).  Scale rule as for the 128-element groups: the smallest power
// of two 2^e with amax <= M * 2^e (M = 448 for E4M3, 6 for E2M1), so nothing saturates.
//
// The matrix-core instruction v_mfma_scale_f32_16x16x128_f8f6f4 takes one scale byte per
// lane and operand: lane l's scale applies to row (column) l % 16 over K block
// [32 (l / 16), 32 (l / 16) + 32) of the instruction's K order, so MX is its native form.
// That K order (measured on the device with an in-bounds probe): an E4M3 operand lane of
// group G = l / 16 holds K 16 G .. 16 G + 15 in its first 16 bytes and K 64 + 16 G ..
// 64 + 16 G + 15 in its last 16; an E2M1 operand lane (16 bytes, two values per byte, the
// lower K in the low nibble) holds K 32 G .. 32 G + 31.  The 128-element path never depends
// on it (one scale per 128 K), but here every E4M3 operand is laid out in that order so a
// 32-element group is one scale block: the activation row is loaded as the 16 bytes at
// 16 G and the 16 at 64 + 16 G, the E4M3 weights are pre-packed the same way, and the
// re-quantised h is stored for the down GEMM in that order.
// The weight operand's format (E4M3 or E2M1) is the instruction's B-format field.
#include "moe_common.h"
#include "moe_internal.h"
#include "mx_common.h"

#include <algorithm>

namespace moe {

// E2M1 code of v / 2^ex (|v / 2^ex| <= 6): round to nearest, ties to the even code; the
// thresholds are the midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 of the magnitudes
// 0 0.5 1 1.5 2 3 4 6.  Sign of zero kept.
__device__ __forceinline__ uint32_t e2m1_code(float v, int ex) {
    const float a = fabsf(ldexpf(v, -ex));
    const uint32_t c = a <= 0.25f ? 0u
                     : a < 0.75f  ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f  ? 3u
                     : a <= 2.5f  ? 4u
                     : a < 3.5f   ? 5u
                     : a <= 5.0f  ? 6u
                                  : 7u;
    return c | (signbit(v) ? 8u : 0u);
}

// ---- activations: E4M3 per (row, 32 columns); 4 lanes per group, 8 bf16 per lane
__global__ __launch_bounds__(256) void k_quant_act_mx(const uint16_t* __restrict__ x, int rows, int cols, int64_t ld,
                                                      uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    const int ngc = cols / kMx;
    const int64_t ngroups = (int64_t)rows * ngc;
    const int sub = threadIdx.x & 3;
    const int64_t gstride = ((int64_t)gridDim.x * blockDim.x) >> 2;
    for (int64_t g = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2; g < ngroups; g += gstride) {
        const int64_t r = g / ngc;
        const int gc = (int)(g - r * ngc);
        const uint4 v = *reinterpret_cast<const uint4*>(x + r * ld + (int64_t)gc * kMx + sub * 8);
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
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const int e = mx_scale_exponent<kWfmtE4M3>(amax);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = ldexpf(f[i], -e);
        uint2 q;
        q.x = cvt4_e4m3(f[0], f[1], f[2], f[3]);
        q.y = cvt4_e4m3(f[4], f[5], f[6], f[7]);
        *reinterpret_cast<uint2*>(xq + r * cols + (int64_t)gc * kMx + sub * 8) = q;
        if (sub == 0) xs[r * ngc + gc] = (uint8_t)(e + 127);
    }
}

// ---- weights: float32 [E, K, N] -> codes + UE8M0 [E, K/32, N], one (32 x 1) group per
// column and thread.  E4M3 codes [E, K, N]; E2M1 codes [E, K, N/2] (column 2c in the low
// nibble of byte c), so an E2M1 thread takes the column pair (2c, 2c + 1).
template <int WF>
__global__ __launch_bounds__(256) void k_quant_weight_mx(const float* __restrict__ w, int E, int K, int N,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    constexpr int C = WF == kWfmtE2M1 ? 2 : 1;   // columns per thread
    const int ncol = N / C;
    const int64_t total = (int64_t)E * (K / kMx) * ncol;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(t % ncol);
        const int64_t ekg = t / ncol;
        const int kg = (int)(ekg % (K / kMx));
        const int64_t e = ekg / (K / kMx);
        const float* src = w + (e * K + (int64_t)kg * kMx) * N + (int64_t)c * C;
        float amax[C];
#pragma unroll
        for (int j = 0; j < C; ++j) amax[j] = 0.f;
        for (int i = 0; i < kMx; ++i)
#pragma unroll
            for (int j = 0; j < C; ++j) amax[j] = fmaxf(amax[j], fabsf(src[(int64_t)i * N + j]));
        int ex[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            ex[j] = mx_scale_exponent<WF>(amax[j]);
            s[(e * (K / kMx) + kg) * N + (int64_t)c * C + j] = (uint8_t)(ex[j] + 127);
        }
        if (WF == kWfmtE2M1) {
            uint8_t* dst = q + (e * K + (int64_t)kg * kMx) * (N / 2) + c;
            for (int i = 0; i < kMx; ++i)
                dst[(int64_t)i * (N / 2)] =
                    (uint8_t)(e2m1_code(src[(int64_t)i * N], ex[0]) | (e2m1_code(src[(int64_t)i * N + 1], ex[C - 1]) << 4));
        } else {
            uint8_t* dst = q + (e * K + (int64_t)kg * kMx) * N + c;
            for (int i = 0; i < kMx; ++i)
                dst[(int64_t)i * N] = (uint8_t)(cvt2_e4m3(ldexpf(src[(int64_t)i * N], -ex[0]), 0.f) & 0xFFu);
        }
    }
}

// ---- E2M1 prepack: logical [E, K, N/2] -> 1 KB blocks per (expert, 16 columns, 128 rows of
// K): byte ((e*(N/16) + n16)*(K/128) + kb)*1024 + lane*16 + b holds rows
// kb*128 + (lane/16)*32 + 2b (low nibble) and + 2b + 1 (high nibble) of column n16*16 + lane%16.
__global__ __launch_bounds__(256) void k_prepack_e2m1(const uint8_t* __restrict__ w, int K, int N, int64_t nchunks,
                                                      uint8_t* __restrict__ out) {
    const int nkb = K / kGroup, nn16 = N / 16;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(c & 63);
        const int64_t blk = c >> 6;
        const int kb = (int)(blk % nkb);
        const int64_t en = blk / nkb;
        const int n16 = (int)(en % nn16);
        const int64_t e = en / nn16;
        const int n = n16 * 16 + (lane & 15);
        const int k0 = kb * kGroup + (lane >> 4) * 32;
        const uint8_t* src = w + (e * K + k0) * (N / 2) + (n >> 1);
        const int sh = (n & 1) * 4;
        uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const uint32_t lo = (src[(int64_t)(2 * b) * (N / 2)] >> sh) & 15u;
            const uint32_t hi = (src[(int64_t)(2 * b + 1) * (N / 2)] >> sh) & 15u;
            d[b >> 2] |= (lo | (hi << 4)) << (8 * (b & 3));
        }
        *reinterpret_cast<uint4*>(out + c * 16) = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

// ---- E4M3 MX prepack: logical [E, K, N] -> 2 KB blocks in the instruction's K order:
// byte ((e*(N/16) + n16)*(K/128) + kb)*2048 + h*1024 + lane*16 + b holds row
// kb*128 + h*64 + (lane/16)*16 + b of column n16*16 + lane%16.
__global__ __launch_bounds__(256) void k_prepack_e4m3_mx(const uint8_t* __restrict__ w, int K, int N, int64_t nchunks,
                                                         uint8_t* __restrict__ out) {
    const int nkb = K / kGroup, nn16 = N / 16;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(c & 63);
        const int h = (int)((c >> 6) & 1);
        const int64_t blk = c >> 7;
        const int kb = (int)(blk % nkb);
        const int64_t en = blk / nkb;
        const int n16 = (int)(en % nn16);
        const int64_t e = en / nn16;
        const int k0 = kb * kGroup + h * 64 + (lane >> 4) * 16;
        const uint8_t* src = w + (e * K + k0) * N + n16 * 16 + (lane & 15);
        uint32_t d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[i] = (uint32_t)src[(int64_t)(4 * i) * N] | ((uint32_t)src[(int64_t)(4 * i + 1) * N] << 8) |
                   ((uint32_t)src[(int64_t)(4 * i + 2) * N] << 16) | ((uint32_t)src[(int64_t)(4 * i + 3) * N] << 24);
        *reinterpret_cast<uint4*>(out + c * 16) = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

// ---- MX scale prepack: logical [E, K/32, N] -> [E][N/16][K/128][64]: byte (e, n16, kb, l)
// is the scale of rows kb*128 + (l/16)*32 .. +31 of column n16*16 + l%16, the byte lane l of
// the matrix-core instruction takes for that operand.
__global__ __launch_bounds__(256) void k_prepack_mx_scales(const uint8_t* __restrict__ s, int K, int N, int64_t n,
                                                           uint8_t* __restrict__ out) {
    const int nkb = K / kGroup, nn16 = N / 16;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n; o += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(o & 63);
        const int64_t blk = o >> 6;
        const int kb = (int)(blk % nkb);
        const int64_t en = blk / nkb;
        const int n16 = (int)(en % nn16);
        const int64_t e = en / nn16;
        out[o] = s[(e * (K / kMx) + kb * 4 + (l >> 4)) * N + n16 * 16 + (l & 15)];
    }
}

// ---- grouped FFN, 16-row expert tiles (the tile list of the decode path).  As the FP8
// decode kernels (k_ffn.hip), with per-lane 32-element scales: the A operand of a lane is
// 32 bytes of its token row, whose scale is xs[tok][kb*4 + lane/16]; the weight operand of
// a lane is one packed fragment chunk with its own scale byte.
struct MxG1Args {
    const uint8_t* xq;
    const uint8_t* xs;          // [T, H/32]
    int T, k, H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w13p;        // packed fragments
    const uint8_t* w13sp;       // packed scales [E][2I/16][H/128][64]
    uint8_t* hq;                // [tile][I/128][2 KB]
    uint8_t* hs;                // [tile*16 + row][I/32]
    float* htap;                // test output: float32 h [A, I] (kernels built with TAP)
    const float* b13;           // optional gate/up bias [E, 2I]
};

template <int WF>
__device__ __forceinline__ v8i mx_wfrag(rsrc_t r, uint32_t lane16, uint32_t soff) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    if (WF == kWfmtE2M1) {
        const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, lane16, soff, MOE_WLOAD_AUX);
        return v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
    return buf_frag(r, lane16, soff);
}

// E4M3 activation operand in the instruction's K order: 16 bytes at K 16 G and 16 at 64 + 16 G.
__device__ __forceinline__ v8i mx_arow(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 64, 0);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}


template <int WF, int PF, bool TAP>
__global__ __launch_bounds__(512) void k_gemm1_mx(MxG1Args a) {
    constexpr int WN = 8;                     // wave wn: gate and up columns 16 wn .. +15 of the block
    constexpr uint32_t FB = WF == kWfmtE2M1 ? 1024u : 2048u;
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int ib = blockIdx.y;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup, KS = a.H / kMx;
    const int tid = threadIdx.x, lane = tid & 63, wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ float s_amax[WN][16];
    __shared__ __align__(16) uint8_t s_h[16 * 128];

    const int tok = a.sorted_assign[rowbase + min(lane & 15, nvalid - 1)] / a.k;
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    const uint32_t av = (uint32_t)tok * a.H + (lane >> 4) * 16;   // K 16 G .. and 64 + 16 G ..
    const uint8_t* sp = a.xs + (int64_t)tok * KS + (lane >> 4);
    const int NB16 = 2 * a.I / 16;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * FB, (uint32_t)NB16 * KB * FB);
    const rsrc_t rs = make_rsrc(a.w13sp + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    const int g16 = ib * 8 + wn, u16 = a.I / 16 + g16;
    const uint32_t l16 = lane * 16;

    v8i aq[PF], bg[PF], bu[PF];
    int sa[PF], sg[PF], su[PF];
    v4f accg = v4f{0.f, 0.f, 0.f, 0.f}, accu = accg;
    auto load = [&](int p, int kb) {
        aq[p] = mx_arow(ra, av, kb * kGroup);
        sa[p] = sp[kb * 4];
        bg[p] = mx_wfrag<WF>(rw, l16, (uint32_t)(g16 * KB + kb) * FB);
        bu[p] = mx_wfrag<WF>(rw, l16, (uint32_t)(u16 * KB + kb) * FB);
        sg[p] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane, (uint32_t)(g16 * KB + kb) * 64, 0);
        su[p] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane, (uint32_t)(u16 * KB + kb) * 64, 0);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) load(p, p);
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                accg = mx_mfma<WF>(aq[p], bg[p], accg, sa[p], sg[p]);
                accu = mx_mfma<WF>(aq[p], bu[p], accu, sa[p], su[p]);
                if (kb + PF < KB) load(p, kb + PF);
            }
        }
    }
    // SwiGLU, then E4M3 per (row, 32 columns): the pair of waves 2g, 2g+1 holds group g
    const GuBias bias = gu_bias(a.b13, e, a.I, ib * 128 + wn * 16 + (lane & 15));
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float g = add_bias(a.b13, accg[i], bias.g);
        hv[i] = g / (1.0f + expf(-g)) * add_bias(a.b13, accu[i], bias.u);
        tap_h<TAP>(a.htap, a.I, rowbase, 4 * (lane >> 4) + i, nvalid, ib * 128 + wn * 16 + (lane & 15), hv[i]);
        const float m = max16(fabsf(hv[i]));
        if ((lane & 15) == 0) s_amax[wn][4 * (lane >> 4) + i] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        const float am = fmaxf(s_amax[wn & ~1][row], s_amax[wn | 1][row]);
        const int ex = mx_scale_exponent<kWfmtE4M3>(am);
        s_h[row * 128 + wn * 16 + (lane & 15)] = (uint8_t)(cvt2_e4m3(ldexpf(hv[i], -ex), 0.f) & 0xFFu);
        if ((wn & 1) == 0 && (lane & 15) == 0)
            a.hs[((int64_t)tile * 16 + row) * (a.I / kMx) + ib * 4 + (wn >> 1)] = (uint8_t)(ex + 127);
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 128; q += 64 * WN) {
        const int hh = q >> 6, ln = q & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (ln & 15) * 128 + hh * 64 + (ln >> 4) * 16);
        *reinterpret_cast<uint4*>(a.hq + ((int64_t)tile * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

struct MxG2Args {
    const uint8_t* hq;
    const uint8_t* hs;
    int H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w2p;
    const uint8_t* w2sp;        // packed scales [E][H/16][I/128][64]
    void* out;
    int out_bf16;
    const float* b2;            // optional down bias [E, H]
};

// workgroup: one 16-row tile x 128 output columns, 4 waves of 2 fragments
template <int WF, int PF>
__global__ __launch_bounds__(256) void k_gemm2_mx(MxG2Args a) {
    constexpr int NFW = 2, WN = 4;
    constexpr uint32_t FB = WF == kWfmtE2M1 ? 1024u : 2048u;
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int lane = threadIdx.x & 63, wn = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * KB * kFragBytes, (uint32_t)KB * kFragBytes);
    const uint8_t* sp = a.hs + ((int64_t)tile * 16 + (lane & 15)) * (a.I / kMx) + (lane >> 4);
    const int NB16 = a.H / 16;
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * FB, (uint32_t)NB16 * KB * FB);
    const rsrc_t rs = make_rsrc(a.w2sp + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    const int n16 = blockIdx.y * (NFW * WN) + wn * NFW;
    const uint32_t l16 = lane * 16;

    v8i aq[PF], bq[PF][NFW];
    int sa[PF], sb[PF][NFW];
    v4f acc[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    auto load = [&](int p, int kb) {
        aq[p] = buf_frag(ra, l16, kb * kFragBytes);
        sa[p] = sp[kb * 4];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            bq[p][j] = mx_wfrag<WF>(rw, l16, (uint32_t)((n16 + j) * KB + kb) * FB);
            sb[p][j] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane, (uint32_t)((n16 + j) * KB + kb) * 64, 0);
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) load(p, p);
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
#pragma unroll
                for (int j = 0; j < NFW; ++j) acc[j] = mx_mfma<WF>(aq[p], bq[p][j], acc[j], sa[p], sb[p][j]);
                if (kb + PF < KB) load(p, kb + PF);
            }
        }
    }
    float bias[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) bias[j] = out_bias(a.b2, e, a.H, (n16 + j) * 16 + (lane & 15));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        if (row < nvalid) {
            const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const int col = (n16 + j) * 16 + (lane & 15);
                const float v = add_bias(a.b2, acc[j][i], bias[j]);
                if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(v);
                else reinterpret_cast<float*>(a.out)[o + col] = v;
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
hipError_t launch_quant_act_mx(const uint16_t* x, int rows, int cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                               hipStream_t st) {
    const int64_t threads = (int64_t)rows * (cols / kMx) * 4;
    const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(threads, 256), 16384));
    hipLaunchKernelGGL(k_quant_act_mx, dim3(blocks), dim3(256), 0, st, x, rows, cols, ld, xq, xs);
    return hipGetLastError();
}

hipError_t launch_quant_weight_mx(const float* w, int E, int K, int N, int wfmt, uint8_t* q, uint8_t* s,
                                  hipStream_t st) {
    const int64_t threads = (int64_t)E * (K / kMx) * (wfmt == kWfmtE2M1 ? N / 2 : N);
    const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(threads, 256), 65536));
    if (wfmt == kWfmtE2M1)
        hipLaunchKernelGGL(k_quant_weight_mx<kWfmtE2M1>, dim3(blocks), dim3(256), 0, st, w, E, K, N, q, s);
    else
        hipLaunchKernelGGL(k_quant_weight_mx<kWfmtE4M3>, dim3(blocks), dim3(256), 0, st, w, E, K, N, q, s);
    return hipGetLastError();
}

hipError_t launch_prepack_mx(const uint8_t* q, const uint8_t* s, int E, int K, int N, int wfmt, uint8_t* packed,
                             uint8_t* packed_s, hipStream_t st) {
    hipError_t e;
    if (wfmt == kWfmtE2M1) {
        const int64_t nchunks = (int64_t)E * K * N / 32;   // 16-byte chunks of 32 values
        const int blocks = (int)std::min<int64_t>(ceil_div(nchunks, 256), 65536);
        hipLaunchKernelGGL(k_prepack_e2m1, dim3(blocks), dim3(256), 0, st, q, K, N, nchunks, packed);
        e = hipGetLastError();
    } else {
        const int64_t nchunks = (int64_t)E * K * N / 16;
        const int blocks = (int)std::min<int64_t>(ceil_div(nchunks, 256), 65536);
        hipLaunchKernelGGL(k_prepack_e4m3_mx, dim3(blocks), dim3(256), 0, st, q, K, N, nchunks, packed);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)E * K * N / kMx;
    const int blocks = (int)std::min<int64_t>(ceil_div(n, 256), 65536);
    hipLaunchKernelGGL(k_prepack_mx_scales, dim3(blocks), dim3(256), 0, st, s, K, N, n, packed_s);
    return hipGetLastError();
}

template <int WF>
static hipError_t run_ffn_mx(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    MxG1Args g1{f.xq, f.xs, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles,
                f.w13p, f.w13s, w.hq, w.hs, f.debug_h, f.b13};
    if (f.debug_h) hipLaunchKernelGGL((k_gemm1_mx<WF, 2, true>), dim3(p.ntiles_max, f.I / kGroup), dim3(512), 0, st, g1);
    else hipLaunchKernelGGL((k_gemm1_mx<WF, 2, false>), dim3(p.ntiles_max, f.I / kGroup), dim3(512), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    MxG2Args g2{w.hq, w.hs, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16, f.b2};
    hipLaunchKernelGGL((k_gemm2_mx<WF, 2>), dim3(p.ntiles_max, f.H / 128), dim3(256), 0, st, g2);
    return hipGetLastError();
}

hipError_t launch_ffn_mx(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    return f.quant == kQuantW4A8 ? run_ffn_mx<kWfmtE2M1>(f, p, w, st, mid) : run_ffn_mx<kWfmtE4M3>(f, p, w, st, mid);
}

}  // namespace moe
