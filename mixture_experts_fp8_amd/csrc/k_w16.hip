// W8A16 expert FFN on 16-row tiles: E4M3 weights with UE8M0 128 x 128 block scales, bf16
// activations.  This is the weight-only expert step that the metrale grouped FP8 MoE page
// keeps as the decode default (FP8 weights, 16-bit activations; its W8A8 step differs from
// it only by the activation rounding).
//
// gfx950 has no matrix instruction taking bf16 against E4M3, so each weight fragment is
// decoded in registers: v_cvt_scalef32_pk_bf16_fp8 turns two E4M3 bytes into two bf16 values
// already multiplied by the block scale 2^(s - 127) (exact: three mantissa bits fit bf16's
// seven), and v_mfma_f32_16x16x32_bf16 contracts 32 K per instruction, four per 128-row K
// block.  The weights keep the packed FP8 layout (lane l's 32 bytes of a 2 KB block are K
// 32 (l / 16) .. + 31 of column l % 16), so the weight bytes streamed from HBM are those of
// the FP8 step.  The bf16 instruction pairs K slot 8 (l / 16) + i of A and B; a lane's four
// instructions per K block take its 32 weight K values in order, 8 at a time, so the A lane
// (row l % 16, group l / 16) reads the 32 activation values at K 32 (l / 16) .. + 31 of its
// row, 64 contiguous bytes, and instruction q takes the 8 at 8q.  The contraction is the
// same sum over K in another order.
//
// Gate+up: workgroup = one tile x one 128-column block of h (8 waves, one gate and one up
// fragment each); SiLU(g) * u in float32, rounded once to bf16 (RNE) into hb [tile][16][I].
// Down: workgroup = one tile x 128 output columns (2 waves x 4 fragments); A = the tile's hb
// rows; out = expert_out rows in sorted-slot order, float32 or bf16.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kW16MaxKB = 256;   // K blocks per GEMM (H, I up to 32768)

struct W16G1Args {
    const uint16_t* x;   // [T, H] bf16
    int T, k, H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w13p;   // packed E4M3 [E][2I/16][H/128][2 KB]
    const uint8_t* w13s;   // UE8M0 [E][H/128][2I/128]
    uint16_t* hb;          // [tile][16][I] bf16
    float* htap;           // test output: float32 h [A, I] before the bf16 rounding (kernels built with TAP)
    const float* b13;      // optional gate/up bias [E, 2I]
};

struct W16G2Args {
    const uint16_t* hb;
    int H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w2p;    // packed E4M3 [E][H/16][I/128][2 KB]
    const uint8_t* w2s;    // UE8M0 [E][I/128][H/128]
    void* out;
    int out_bf16;
    const float* b2;       // optional down bias [E, H]
};

// The 32 bf16 weights of one lane's fragment, scaled by 2^(s - 127) (sc carries s in its
// exponent field), as the four 8-element operands of the K block's instructions.
__device__ __forceinline__ void decode_frag(const v8i& q, float sc, v8bf (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * i], sc, false);
        const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * i], sc, true);
        const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * i + 1], sc, false);
        const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * i + 1], sc, true);
        b[i] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
}

// A lane's 32 activation values (64 bytes) as the four instruction operands.
__device__ __forceinline__ void act_ops(const uint4 (&v)[4], v8bf (&a)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(v8bf, v[i]);
}

__device__ __forceinline__ float ue8m0_as_scale(uint32_t s) { return __uint_as_float(s << 23); }

template <int PF, bool TAP>
__global__ __launch_bounds__(512) void k_gemm1_w16(W16G1Args a) {
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int ib = blockIdx.y;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ float s_sg[kW16MaxKB], s_su[kW16MaxKB];   // block scales of this column block
    __shared__ __align__(16) uint16_t s_h[16 * 128];

    const int tok = a.sorted_assign[rowbase + min(lane & 15, nvalid - 1)] / a.k;
    const uint4* xa = reinterpret_cast<const uint4*>(a.x + (int64_t)tok * a.H + (lane >> 4) * 32);
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    const int g16 = ib * 8 + wn, u16 = a.I / 16 + g16;
    const uint32_t l16 = lane * 16;
    for (int i = tid; i < KB; i += 512) {
        s_sg[i] = ue8m0_as_scale(sb[i * NBS + ib]);
        s_su[i] = ue8m0_as_scale(sb[i * NBS + a.I / kGroup + ib]);
    }
    __syncthreads();

    uint4 xv[PF][4];
    v8i bg[PF], bu[PF];
    v4f accg = v4f{0.f, 0.f, 0.f, 0.f}, accu = accg;
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[p][i] = xa[p * 16 + i];
            bg[p] = buf_frag(rw, l16, (g16 * KB + p) * kFragBytes);
            bu[p] = buf_frag(rw, l16, (u16 * KB + p) * kFragBytes);
        }
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                v8bf av[4], bgv[4], buv[4];
                act_ops(xv[p], av);
                decode_frag(bg[p], s_sg[kb], bgv);
                decode_frag(bu[p], s_su[kb], buv);
                const int kn = kb + PF;
                if (kn < KB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[p][i] = xa[kn * 16 + i];
                    bg[p] = buf_frag(rw, l16, (g16 * KB + kn) * kFragBytes);
                    bu[p] = buf_frag(rw, l16, (u16 * KB + kn) * kFragBytes);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], bgv[q], accg, 0, 0, 0);
                    accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], buv[q], accu, 0, 0, 0);
                }
            }
        }
    }
    // SwiGLU in float32, one bf16 rounding; lane holds rows 4 (lane / 16) + i of column
    // wn * 16 + lane % 16 of the block
    const GuBias bias = gu_bias(a.b13, e, a.I, ib * 128 + wn * 16 + (lane & 15));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float g = add_bias(a.b13, accg[i], bias.g);
        const float h = g / (1.0f + expf(-g)) * add_bias(a.b13, accu[i], bias.u);
        tap_h<TAP>(a.htap, a.I, rowbase, 4 * (lane >> 4) + i, nvalid, ib * 128 + wn * 16 + (lane & 15), h);
        s_h[(4 * (lane >> 4) + i) * 128 + wn * 16 + (lane & 15)] = f32_to_bf16(h);
    }
    __syncthreads();
    if (tid < 256) {   // 16 rows x 256 bytes
        const int r = tid >> 4, c = tid & 15;
        *reinterpret_cast<uint4*>(a.hb + ((int64_t)tile * 16 + r) * a.I + ib * 128 + c * 8) =
            *reinterpret_cast<const uint4*>(s_h + r * 128 + c * 8);
    }
}

template <int NFW, int WN, int PF>
__global__ __launch_bounds__(64 * WN) void k_gemm2_w16(W16G2Args a) {
    static_assert(NFW * WN == 8, "a workgroup covers one 128-column scale block");
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int lane = threadIdx.x & 63, wn = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint4* ha = reinterpret_cast<const uint4*>(a.hb + ((int64_t)tile * 16 + (lane & 15)) * a.I + (lane >> 4) * 32);
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    const int n16 = blockIdx.y * 8 + wn * NFW;
    const uint32_t l16 = lane * 16;
    __shared__ float s_sb[kW16MaxKB];
    for (int i = threadIdx.x; i < KB; i += 64 * WN) s_sb[i] = ue8m0_as_scale(sb[i * NBS + blockIdx.y]);
    __syncthreads();

    uint4 hv[PF][4];
    v8i bq[PF][NFW];
    v4f acc[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[p][i] = ha[p * 16 + i];
#pragma unroll
            for (int j = 0; j < NFW; ++j) bq[p][j] = buf_frag(rw, l16, ((n16 + j) * KB + p) * kFragBytes);
        }
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                v8bf av[4], bv[NFW][4];
                act_ops(hv[p], av);
#pragma unroll
                for (int j = 0; j < NFW; ++j) decode_frag(bq[p][j], s_sb[kb], bv[j]);
                const int kn = kb + PF;
                if (kn < KB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) hv[p][i] = ha[kn * 16 + i];
#pragma unroll
                    for (int j = 0; j < NFW; ++j) bq[p][j] = buf_frag(rw, l16, ((n16 + j) * KB + kn) * kFragBytes);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < NFW; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], bv[j][q], acc[j], 0, 0, 0);
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

// down-GEMM shape: fragments per wave, waves, K blocks in flight (NFW * WN = 8)
#ifndef MOE_W16_GEMM2
#define MOE_W16_GEMM2 4, 2, 2
#endif
#ifndef MOE_W16_PF1
#define MOE_W16_PF1 2
#endif

template <int NFW, int WN, int PF>
static void launch_gemm2_w16(const W16G2Args& g2, int ntiles_max, int H, hipStream_t st) {
    hipLaunchKernelGGL((k_gemm2_w16<NFW, WN, PF>), dim3(ntiles_max, H / kGroup), dim3(64 * WN), 0, st, g2);
}

hipError_t launch_ffn_w16(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    if (f.H / kGroup > kW16MaxKB || f.I / kGroup > kW16MaxKB) return hipErrorInvalidValue;
    uint16_t* hb = reinterpret_cast<uint16_t*>(w.hq);
    W16G1Args g1{f.x, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles, f.w13p, f.w13s, hb,
                 f.debug_h, f.b13};
    if (f.debug_h) hipLaunchKernelGGL((k_gemm1_w16<MOE_W16_PF1, true>), dim3(p.ntiles_max, f.I / kGroup), dim3(512), 0, st, g1);
    else hipLaunchKernelGGL((k_gemm1_w16<MOE_W16_PF1, false>), dim3(p.ntiles_max, f.I / kGroup), dim3(512), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    W16G2Args g2{hb, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16, f.b2};
    launch_gemm2_w16<MOE_W16_GEMM2>(g2, p.ntiles_max, f.H, st);
    return hipGetLastError();
}

}  // namespace moe
