// Grouped expert FFN and combine (gfx950).
//
// gate+up GEMM with the SwiGLU + E4M3 re-quantisation epilogue, then the down GEMM, as
// the two W8A8 launches of run_fp8_grouped_w8a8 (metrale "fp8_grouped_tc_w8a8.rs"),
// and the weighted combine of the MindIE-SD "Fused MoE" flow ("执行流程": combine).
//
// Both GEMMs run on the scaled FP8 matrix cores, v_mfma_scale_f32_16x16x128_f8f6f4: one
// instruction covers exactly one 128-deep K block, so the UE8M0 scale of the activation
// row and of the weight block enter as the instruction's own scale operands and the fp32
// accumulator sums already-scaled block products.
//
// Work decomposition: the expert-sorted rows are cut into tiles of BM rows that never
// straddle two experts (tile list built on the device from the expert counts).  A
// workgroup takes one tile and one 128-wide slice of the output columns.  A rows are
// staged in LDS (double buffered, gathered through sorted_assign for the gate+up GEMM)
// in the exact byte order the matrix cores read; B (weights, pre-packed) streams straight
// from memory into registers PF K-blocks ahead, 2 KB contiguous per operand.
#include "moe_common.h"
#include "moe_internal.h"

#include <algorithm>

// Decode-tile configurations (fragments per wave, waves per workgroup, K blocks in flight)
// of the gate+up and the down GEMM; fixed at build time.
#ifndef MOE_DEC_GEMM1
#define MOE_DEC_GEMM1 1, 8, 2
#endif
#ifndef MOE_DEC_GEMM2
#define MOE_DEC_GEMM2 2, 4, 2
#endif
// Prefill kernels (128 x 256 tiles): k_gemm{1,2}_pf8 (2x4 waves of 64x64, two waves per
// SIMD; 512 threads), k_gemm{1,2}_pfr (2x2 waves of 64x128; 256 threads), k_gemm{1,2}_pfn
// (waves split the columns) or k_gemm{1,2}_pf (LDS-DMA staging; 256 threads)
#ifndef MOE_PF_GEMM1
#define MOE_PF_GEMM1 k_gemm1_pf8<2>
#endif
#ifndef MOE_PF_GEMM2
#define MOE_PF_GEMM2 k_gemm2_pf8<2>
#endif
#ifndef MOE_PF_THREADS
#define MOE_PF_THREADS 512
#endif

namespace moe {

constexpr int kMaxKB = 256;   // K blocks (of 128) per GEMM: H and I up to 32768

// ----------------------------------------------------------------------------------------
// Tile list: tiles of BM rows per expert, in expert order.
__global__ __launch_bounds__(1024) void k_tiles(const int32_t* __restrict__ counts, int E, int BM,
                                                int2* __restrict__ tiles, int32_t* __restrict__ ntiles) {
    __shared__ int s_tmp[16];
    const int e = threadIdx.x;
    const int n = e < E ? (counts[e] + BM - 1) / BM : 0;
    // inclusive scan over the workgroup
    const int lane = e & 63, wv = e >> 6;
    int v = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_tmp[wv] = v;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wv; ++w) add += s_tmp[w];
    const int start = v + add - n;
    for (int i = 0; i < n; ++i) tiles[start + i] = make_int2(e, i * BM);
    if (e == 1023) *ntiles = v + add;
}

hipError_t launch_tiles(const int32_t* counts, int E, int BM, int2* tiles, int32_t* ntiles, hipStream_t st) {
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(1024), 0, st, counts, E, BM, tiles, ntiles);
    return hipGetLastError();
}

struct G1Args {
    const uint8_t* xq;
    const uint8_t* xs;
    int T, k, H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w13p;
    const uint8_t* w13s;
    uint8_t* hq;
    uint8_t* hs;
};

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int lane) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 1024 + lane * 16);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ v8i gmem_frag(const uint8_t* base, int lane) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 1024 + lane * 16);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// gate+up GEMM + SwiGLU + requant.  Wave (wm, wn) computes MFW m-frags x NFW gate frags and
// the NFW matching up frags; the workgroup covers BM rows x one 128-column block ib of h.
template <int MFW, int NFW, int WM, int WN, int PF>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm1(G1Args a) {
    constexpr int NT = 64 * WM * WN;
    constexpr int MF = MFW * WM;
    constexpr int BM = 16 * MF;
    constexpr int ACH = (BM * 8 + NT - 1) / NT;
    static_assert(NFW * WN == 8, "a workgroup covers 128 gate + 128 up columns");

    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int ib = blockIdx.y;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(BM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;

    __shared__ __align__(16) uint8_t s_a[2][MF][kFragBytes];
    __shared__ uint8_t s_sa[2][BM];
    __shared__ float s_amax[WN][BM];

    // A gather: chunk q = (row r = q/8, 16-byte column chunk c8 = q%8)
    int64_t a_src[ACH];
    int a_dst[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = tid + i * NT;
        a_dst[i] = -1;
        a_src[i] = 0;
        if (q < BM * 8) {
            const int r = q >> 3, c8 = q & 7;
            const int rr = min(r, nvalid - 1);
            const int tok = a.sorted_assign[rowbase + rr] / a.k;
            a_src[i] = (int64_t)tok * a.H + c8 * 16;
            a_dst[i] = (r >> 4) * kFragBytes + (c8 & 1) * 1024 + ((c8 >> 1) * 16 + (r & 15)) * 16;
        }
    }
    int64_t sa_src = -1;
    if (tid < BM) sa_src = (int64_t)(a.sorted_assign[rowbase + min(tid, nvalid - 1)] / a.k) * KB;

    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const uint8_t* wb = a.w13p + (int64_t)e * NB16 * KB * kFragBytes;
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    const int g16 = ib * 8 + wn * NFW;          // first gate n16 of this wave
    const int u16 = a.I / 16 + g16;             // first up n16

    v8i bq[PF][2 * NFW];
    v4f accg[MFW][NFW], accu[MFW][NFW];
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi)
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            accg[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};
            accu[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }

    uint4 areg[ACH];
    uint8_t sareg = 0;
    // prologue: A block 0 -> LDS stage 0; B blocks 0..PF-1 -> registers
#pragma unroll
    for (int i = 0; i < ACH; ++i)
        if (a_dst[i] >= 0) areg[i] = *reinterpret_cast<const uint4*>(a.xq + a_src[i]);
    if (sa_src >= 0) sareg = a.xs[sa_src];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                bq[p][j] = gmem_frag(wb + ((int64_t)(g16 + j) * KB + p) * kFragBytes, lane);
                bq[p][NFW + j] = gmem_frag(wb + ((int64_t)(u16 + j) * KB + p) * kFragBytes, lane);
            }
        }
#pragma unroll
    for (int i = 0; i < ACH; ++i)
        if (a_dst[i] >= 0) *reinterpret_cast<uint4*>(&s_a[0][0][0] + a_dst[i]) = areg[i];
    if (tid < BM) s_sa[0][tid] = sareg;
    __syncthreads();

    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                const int cur = kb & 1;
                if (kb + 1 < KB) {
#pragma unroll
                    for (int i = 0; i < ACH; ++i)
                        if (a_dst[i] >= 0)
                            areg[i] = *reinterpret_cast<const uint4*>(a.xq + a_src[i] + (int64_t)(kb + 1) * kGroup);
                    if (sa_src >= 0) sareg = a.xs[sa_src + kb + 1];
                }
                const int sg = sb[kb * NBS + ib];
                const int su = sb[kb * NBS + a.I / kGroup + ib];
#pragma unroll
                for (int mi = 0; mi < MFW; ++mi) {
                    const int mf = wm * MFW + mi;
                    const v8i af = lds_frag(&s_a[cur][mf][0], lane);
                    const int sa = s_sa[cur][mf * 16 + (lane & 15)];
#pragma unroll
                    for (int j = 0; j < NFW; ++j) {
                        accg[mi][j] = mfma_fp8(af, bq[p][j], accg[mi][j], sa, sg);
                        accu[mi][j] = mfma_fp8(af, bq[p][NFW + j], accu[mi][j], sa, su);
                    }
                }
                if (kb + PF < KB) {
#pragma unroll
                    for (int j = 0; j < NFW; ++j) {
                        bq[p][j] = gmem_frag(wb + ((int64_t)(g16 + j) * KB + kb + PF) * kFragBytes, lane);
                        bq[p][NFW + j] = gmem_frag(wb + ((int64_t)(u16 + j) * KB + kb + PF) * kFragBytes, lane);
                    }
                }
                if (kb + 1 < KB) {
#pragma unroll
                    for (int i = 0; i < ACH; ++i)
                        if (a_dst[i] >= 0) *reinterpret_cast<uint4*>(&s_a[cur ^ 1][0][0] + a_dst[i]) = areg[i];
                    if (tid < BM) s_sa[cur ^ 1][tid] = sareg;
                }
                __syncthreads();
            }
        }
    }

    // ---- epilogue: h = silu(g) * u; per-row amax over the 128 columns; E4M3 requant
    float hv[MFW][NFW][4];
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const float g = accg[mi][j][i];
                const float h = g / (1.0f + expf(-g)) * accu[mi][j][i];
                hv[mi][j][i] = h;
                m = fmaxf(m, fabsf(h));
            }
            m = max16(m);
            if ((lane & 15) == 0) s_amax[wn][(wm * MFW + mi) * 16 + 4 * (lane >> 4) + i] = m;
        }
    }
    __syncthreads();
    uint8_t* s_h = &s_a[0][0][0];   // [BM][128] bytes, reuses the A stages
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * MFW + mi) * 16 + 4 * (lane >> 4) + i;
            float am = s_amax[0][row];
#pragma unroll
            for (int w = 1; w < WN; ++w) am = fmaxf(am, s_amax[w][row]);
            const int ex = scale_exponent(am);
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const uint32_t q = cvt2_e4m3(ldexpf(hv[mi][j][i], -ex), 0.f) & 0xFFu;
                s_h[row * 128 + (wn * NFW + j) * 16 + (lane & 15)] = (uint8_t)q;
            }
            if (wn == 0 && (lane & 15) == 0)
                a.hs[((int64_t)tile * BM + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < MF * 128; q += NT) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (mf * 16 + (ln & 15)) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * MF + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

struct G2Args {
    const uint8_t* hq;
    const uint8_t* hs;
    int H, I;
    const int32_t* counts;
    const int32_t* offsets;
    const int2* tiles;
    const int32_t* ntiles;
    const uint8_t* w2p;
    const uint8_t* w2s;
    void* out;
    int out_bf16;
};

// down GEMM: wave (wm, wn) computes MFW m-frags x NFW column frags; the workgroup covers
// BM rows x 16*NFW*WN output columns.
template <int MFW, int NFW, int WM, int WN, int PF>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm2(G2Args a) {
    constexpr int NT = 64 * WM * WN;
    constexpr int MF = MFW * WM;
    constexpr int BM = 16 * MF;
    constexpr int ACH = (MF * 128 + NT - 1) / NT;

    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(BM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;

    __shared__ __align__(16) uint8_t s_a[2][MF][kFragBytes];
    __shared__ uint8_t s_sa[2][BM];

    const uint8_t* abase = a.hq + (int64_t)tile * MF * KB * kFragBytes;   // [mf][kb][2048]
    const uint8_t* sabase = a.hs + (int64_t)tile * BM * KB;               // [row][kb]
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const uint8_t* wb = a.w2p + (int64_t)e * NB16 * KB * kFragBytes;
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    const int n16 = blockIdx.y * (NFW * WN) + wn * NFW;

    v8i bq[PF][NFW];
    v4f acc[MFW][NFW];
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi)
#pragma unroll
        for (int j = 0; j < NFW; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // A copy: chunk q = (mf = q/128, 16-byte piece q%128) of the contiguous 2 KB operand
    uint4 areg[ACH];
    uint8_t sareg = 0;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = tid + i * NT;
        if (q < MF * 128)
            areg[i] = *reinterpret_cast<const uint4*>(abase + ((int64_t)(q >> 7) * KB) * kFragBytes + (q & 127) * 16);
    }
    if (tid < BM) sareg = sabase[tid * KB];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
#pragma unroll
            for (int j = 0; j < NFW; ++j) bq[p][j] = gmem_frag(wb + ((int64_t)(n16 + j) * KB + p) * kFragBytes, lane);
        }
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = tid + i * NT;
        if (q < MF * 128) *reinterpret_cast<uint4*>(&s_a[0][0][0] + q * 16) = areg[i];
    }
    if (tid < BM) s_sa[0][tid] = sareg;
    __syncthreads();

    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                const int cur = kb & 1;
                if (kb + 1 < KB) {
#pragma unroll
                    for (int i = 0; i < ACH; ++i) {
                        const int q = tid + i * NT;
                        if (q < MF * 128)
                            areg[i] = *reinterpret_cast<const uint4*>(
                                abase + ((int64_t)(q >> 7) * KB + kb + 1) * kFragBytes + (q & 127) * 16);
                    }
                    if (tid < BM) sareg = sabase[tid * KB + kb + 1];
                }
#pragma unroll
                for (int mi = 0; mi < MFW; ++mi) {
                    const int mf = wm * MFW + mi;
                    const v8i af = lds_frag(&s_a[cur][mf][0], lane);
                    const int sa = s_sa[cur][mf * 16 + (lane & 15)];
#pragma unroll
                    for (int j = 0; j < NFW; ++j) {
                        const int sbv = sb[kb * NBS + ((n16 + j) * 16) / kGroup];
                        acc[mi][j] = mfma_fp8(af, bq[p][j], acc[mi][j], sa, sbv);
                    }
                }
                if (kb + PF < KB) {
#pragma unroll
                    for (int j = 0; j < NFW; ++j)
                        bq[p][j] = gmem_frag(wb + ((int64_t)(n16 + j) * KB + kb + PF) * kFragBytes, lane);
                }
                if (kb + 1 < KB) {
#pragma unroll
                    for (int i = 0; i < ACH; ++i) {
                        const int q = tid + i * NT;
                        if (q < MF * 128) *reinterpret_cast<uint4*>(&s_a[cur ^ 1][0][0] + q * 16) = areg[i];
                    }
                    if (tid < BM) s_sa[cur ^ 1][tid] = sareg;
                }
                __syncthreads();
            }
        }
    }

    // ---- epilogue: rows in expert-sorted slot order
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * MFW + mi) * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < NFW; ++j) {
                    const int col = (n16 + j) * 16 + (lane & 15);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[mi][j][i]);
                    else reinterpret_cast<float*>(a.out)[o + col] = acc[mi][j][i];
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Decode variants: a tile is one 16-row matrix-core fragment, so there is nothing to share
// between waves on the A side.  Each wave loads its A fragment (the 16 gathered token rows'
// 32-byte K slices, L2-resident) and its B fragments (straight from HBM) PF K-blocks ahead
// into registers; no LDS and no barrier inside the K loop.

__device__ __forceinline__ v8i gmem_a32(const uint8_t* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

template <int NFW, int WN, int PF>
__global__ __launch_bounds__(64 * WN) void k_gemm1_dec(G1Args a) {
    static_assert(NFW * WN == 8, "a workgroup covers 128 gate + 128 up columns");
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int ib = blockIdx.y;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ float s_amax[WN][16];
    __shared__ __align__(16) uint8_t s_h[16 * 128];
    __shared__ uint8_t s_sg[kMaxKB], s_su[kMaxKB];   // weight-block scales of this column block

    const int tok = a.sorted_assign[rowbase + min(lane & 15, nvalid - 1)] / a.k;
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    const uint32_t av = (uint32_t)tok * a.H + (lane >> 4) * 32;
    const uint8_t* sp = a.xs + (int64_t)tok * KB;
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    const int g16 = ib * 8 + wn * NFW;
    const int u16 = a.I / 16 + g16;
    const uint32_t l16 = lane * 16;
    for (int i = tid; i < KB; i += 64 * WN) {
        s_sg[i] = sb[i * NBS + ib];
        s_su[i] = sb[i * NBS + a.I / kGroup + ib];
    }
    __syncthreads();

    v8i aq[PF], bq[PF][2 * NFW];
    int sa[PF];
    v4f accg[NFW], accu[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) accg[j] = accu[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
            aq[p] = buf_a32(ra, av, p * kGroup);
            sa[p] = sp[p];
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                bq[p][j] = buf_frag(rw, l16, ((g16 + j) * KB + p) * kFragBytes);
                bq[p][NFW + j] = buf_frag(rw, l16, ((u16 + j) * KB + p) * kFragBytes);
            }
        }
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                const int sg = s_sg[kb];
                const int su = s_su[kb];
#pragma unroll
                for (int j = 0; j < NFW; ++j) {
                    accg[j] = mfma_fp8(aq[p], bq[p][j], accg[j], sa[p], sg);
                    accu[j] = mfma_fp8(aq[p], bq[p][NFW + j], accu[j], sa[p], su);
                }
                const int kn = kb + PF;
                if (kn < KB) {
                    aq[p] = buf_a32(ra, av, kn * kGroup);
                    sa[p] = sp[kn];
#pragma unroll
                    for (int j = 0; j < NFW; ++j) {
                        bq[p][j] = buf_frag(rw, l16, ((g16 + j) * KB + kn) * kFragBytes);
                        bq[p][NFW + j] = buf_frag(rw, l16, ((u16 + j) * KB + kn) * kFragBytes);
                    }
                }
            }
        }
    }
    // epilogue: SwiGLU, row amax over the 128 columns (across the WN waves), requant
    float hv[NFW][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            const float g = accg[j][i];
            const float h = g / (1.0f + expf(-g)) * accu[j][i];
            hv[j][i] = h;
            m = fmaxf(m, fabsf(h));
        }
        m = max16(m);
        if ((lane & 15) == 0) s_amax[wn][4 * (lane >> 4) + i] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        float am = s_amax[0][row];
#pragma unroll
        for (int w = 1; w < WN; ++w) am = fmaxf(am, s_amax[w][row]);
        const int ex = scale_exponent(am);
#pragma unroll
        for (int j = 0; j < NFW; ++j)
            s_h[row * 128 + (wn * NFW + j) * 16 + (lane & 15)] =
                (uint8_t)(cvt2_e4m3(ldexpf(hv[j][i], -ex), 0.f) & 0xFFu);
        if (wn == 0 && (lane & 15) == 0)
            a.hs[((int64_t)tile * 16 + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 128; q += 64 * WN) {
        const int hh = q >> 6, ln = q & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (ln & 15) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + ((int64_t)tile * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int NFW, int WN, int PF>
__global__ __launch_bounds__(64 * WN) void k_gemm2_dec(G2Args a) {
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int lane = threadIdx.x & 63, wn = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * KB * kFragBytes, (uint32_t)KB * kFragBytes);
    const uint8_t* sp = a.hs + ((int64_t)tile * 16 + (lane & 15)) * KB;
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    const int n16 = blockIdx.y * (NFW * WN) + wn * NFW;
    const uint32_t l16 = lane * 16;
    static_assert(NFW * WN == 8, "a workgroup covers one 128-column scale block");
    __shared__ uint8_t s_sb[kMaxKB];
    for (int i = threadIdx.x; i < KB; i += 64 * WN) s_sb[i] = sb[i * NBS + blockIdx.y];
    __syncthreads();

    v8i aq[PF], bq[PF][NFW];
    int sa[PF];
    v4f acc[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < KB) {
            aq[p] = buf_frag(ra, l16, p * kFragBytes);
            sa[p] = sp[p];
#pragma unroll
            for (int j = 0; j < NFW; ++j) bq[p][j] = buf_frag(rw, l16, ((n16 + j) * KB + p) * kFragBytes);
        }
    for (int kb0 = 0; kb0 < KB; kb0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kb = kb0 + p;
            if (kb < KB) {
                const int sbv = s_sb[kb];
#pragma unroll
                for (int j = 0; j < NFW; ++j) acc[j] = mfma_fp8(aq[p], bq[p][j], acc[j], sa[p], sbv);
                const int kn = kb + PF;
                if (kn < KB) {
                    aq[p] = buf_frag(ra, l16, kn * kFragBytes);
                    sa[p] = sp[kn];
#pragma unroll
                    for (int j = 0; j < NFW; ++j) bq[p][j] = buf_frag(rw, l16, ((n16 + j) * KB + kn) * kFragBytes);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        if (row < nvalid) {
            const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const int col = (n16 + j) * 16 + (lane & 15);
                if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[j][i]);
                else reinterpret_cast<float*>(a.out)[o + col] = acc[j][i];
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Prefill variants: workgroup tile 128 rows x 256 columns, 4 waves as 2 (rows) x 2
// (columns), wave tile 64 x 128 (4 x 8 matrix-core fragments).  A and B fragments travel
// global -> LDS by the LDS-DMA form of the buffer load (no staging registers) through a
// 3-stage ring; each stage is its own LDS array so the compiler tracks the DMA writes per
// stage.  Per K block: wait until this wave's DMA for the block has landed, barrier, issue
// the DMA two blocks ahead, then read fragments from LDS and run 32 MFMAs per wave.  The A
// row scales of all K blocks are loaded into LDS once per tile.

constexpr int kPfBM = 128, kPfStageA = 8 * kFragBytes, kPfStage = kPfStageA + 16 * kFragBytes;  // 48 KB
constexpr int kPfMaxKB = 64;     // K blocks whose A scales fit the LDS table

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
// vmcnt <= n (n < 16), other counters untouched
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8))

__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 16, voff, soff, 0, 0);
}

// gate+up prefill GEMM; grid (I/128 column blocks, tiles)
__global__ __launch_bounds__(256, 1) void k_gemm1_pf(G1Args a) {
    const int ib = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    __shared__ __align__(16) uint8_t st0[kPfStage], st1[kPfStage], st2[kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sg[kPfMaxKB], s_su[kPfMaxKB];
    __shared__ float s_amax[2][kPfBM];

    // A scales of every K block: thread pair (row, half) copies half of the row's KB bytes
    {
        const int r = tid >> 1, half = tid & 1;
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        const uint8_t* src = a.xs + (int64_t)tok * KB;
        for (int kb = half; kb < KB; kb += 2) s_sa[r * KB + kb] = src[kb];
    }
    // this wave's DMA sources: A fragments 2wv, 2wv+1 (rows gathered), B fragments 4wv..4wv+3
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    uint32_t aoff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = (2 * wv + q) * 16 + (lane & 15);
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        aoff[q] = (uint32_t)tok * a.H + (lane >> 4) * 32;
    }
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    for (int i = tid; i < KB; i += 256) {
        s_sg[i] = sb[i * NBS + ib];
        s_su[i] = sb[i * NBS + a.I / kGroup + ib];
    }
    int bn16[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = 4 * wv + j;
        bn16[j] = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
    }
    const uint32_t l16 = lane * 16;
    auto issue = [&](int kb, uint8_t* st) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) dma16(ra, st + (2 * wv + q) * kFragBytes + h * 1024, aoff[q] + h * 16, kb * kGroup);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                dma16(rw, st + kPfStageA + (4 * wv + j) * kFragBytes + h * 1024, l16,
                      (uint32_t)(bn16[j] * KB + kb) * kFragBytes + h * 1024);
    };

    v4f accg[4][4], accu[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) accg[mi][j] = accu[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    __builtin_amdgcn_s_waitcnt(0);   // scale copies done before the DMA count starts
    issue(0, st0);
    issue(min(1, KB - 1), st1);

    // Every step issues the DMA of block kb + 2 (clamped to the last block: the duplicate
    // lands in a stage nobody reads again), so exactly 12 DMA loads per wave follow the
    // ones of block kb and vmcnt(12) means "block kb has landed".
    auto step = [&](int kb, const uint8_t* cur, uint8_t* nxt) {
        WAIT_VMCNT(12);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads and writes done
        __builtin_amdgcn_s_barrier();
        issue(min(kb + 2, KB - 1), nxt);
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
        const int sg = s_sg[kb];
        const int su = s_su[kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v8i bg = lds_frag(cur + kPfStageA + (wn * 4 + j) * kFragBytes, lane);
            const v8i bu = lds_frag(cur + kPfStageA + (8 + wn * 4 + j) * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                accg[mi][j] = mfma_fp8(af[mi], bg, accg[mi][j], sa[mi], sg);
                accu[mi][j] = mfma_fp8(af[mi], bu, accu[mi][j], sa[mi], su);
            }
        }
    };
    int kb0 = 0;
    for (; kb0 + 3 <= KB; kb0 += 3) {
        step(kb0, st0, st2);
        step(kb0 + 1, st1, st0);
        step(kb0 + 2, st2, st1);
    }
    if (kb0 < KB) step(kb0, st0, st2);
    if (kb0 + 1 < KB) step(kb0 + 1, st1, st0);
    __builtin_amdgcn_s_waitcnt(0);   // the trailing duplicate DMA must land before LDS is reused

    // ---- epilogue: SwiGLU, row amax over the 128 columns (two waves), requant
    float hv[4][4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float g = accg[mi][j][i];
                const float h = g / (1.0f + expf(-g)) * accu[mi][j][i];
                hv[mi][j][i] = h;
                m = fmaxf(m, fabsf(h));
            }
            m = max16(m);
            if ((lane & 15) == 0) s_amax[wn][(wm * 4 + mi) * 16 + 4 * (lane >> 4) + i] = m;
        }
    }
    __syncthreads();
    uint8_t* s_h = st0;   // [128][128] bytes
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            const int ex = scale_exponent(fmaxf(s_amax[0][row], s_amax[1][row]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_h[row * 128 + (wn * 4 + j) * 16 + (lane & 15)] =
                    (uint8_t)(cvt2_e4m3(ldexpf(hv[mi][j][i], -ex), 0.f) & 0xFFu);
            if (wn == 0 && (lane & 15) == 0)
                a.hs[((int64_t)tile * kPfBM + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 8 * 128; q += 256) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (mf * 16 + (ln & 15)) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

// down prefill GEMM; grid (H/256 column blocks, tiles)
__global__ __launch_bounds__(256, 1) void k_gemm2_pf(G2Args a) {
    const int nb = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    __shared__ __align__(16) uint8_t st0[kPfStage], st1[kPfStage], st2[kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sb[2][kPfMaxKB];   // the two 128-column scale blocks of this workgroup

    {
        const uint8_t* src = a.hs + (int64_t)tile * kPfBM * KB;   // [row][kb], contiguous for the tile
        for (int i = tid; i < kPfBM * KB; i += 256) s_sa[i] = src[i];
    }
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    for (int i = tid; i < 2 * KB; i += 256) s_sb[i & 1][i >> 1] = sb[(i >> 1) * NBS + nb * 2 + (i & 1)];
    const uint32_t l16 = lane * 16;
    auto issue = [&](int kb, uint8_t* st) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                dma16(ra, st + (2 * wv + q) * kFragBytes + h * 1024, l16,
                      (uint32_t)((2 * wv + q) * KB + kb) * kFragBytes + h * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                dma16(rw, st + kPfStageA + (4 * wv + j) * kFragBytes + h * 1024, l16,
                      (uint32_t)((nb * 16 + 4 * wv + j) * KB + kb) * kFragBytes + h * 1024);
    };

    v4f acc[4][8];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    __builtin_amdgcn_s_waitcnt(0);
    issue(0, st0);
    issue(min(1, KB - 1), st1);

    auto step = [&](int kb, const uint8_t* cur, uint8_t* nxt) {
        WAIT_VMCNT(12);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        issue(min(kb + 2, KB - 1), nxt);
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = wn * 8 + j;
            const v8i b = lds_frag(cur + kPfStageA + f * kFragBytes, lane);
            const int sbv = s_sb[wn][kb];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mfma_fp8(af[mi], b, acc[mi][j], sa[mi], sbv);
        }
    };
    int kb0 = 0;
    for (; kb0 + 3 <= KB; kb0 += 3) {
        step(kb0, st0, st2);
        step(kb0 + 1, st1, st0);
        step(kb0 + 2, st2, st1);
    }
    if (kb0 < KB) step(kb0, st0, st2);
    if (kb0 + 1 < KB) step(kb0 + 1, st1, st0);
    __builtin_amdgcn_s_waitcnt(0);   // the trailing duplicate DMA must land before LDS is reused

#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int col = nb * 256 + (wn * 8 + j) * 16 + (lane & 15);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[mi][j][i]);
                    else reinterpret_cast<float*>(a.out)[o + col] = acc[mi][j][i];
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Register-staged prefill variants: the same tiles, but each wave loads its 12 16-byte
// pieces of a K block into registers (buffer loads) and writes them to LDS itself.  Two LDS
// buffers and two register sets: at step kb the wave issues the loads of block kb+2 into
// one register set, computes block kb from LDS, then stores the other register set (block
// kb+1, loaded a step earlier) into the free LDS buffer; one barrier per step.  Plain loads
// into registers keep the compiler's vmcnt accounting exact.

struct PfLoads {
    uint4 v[12];
};

__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff, int aux) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i x = aux ? __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2)
                      : __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
}

template <int NR>
__global__ __launch_bounds__(256, 1) void k_gemm1_pfr(G1Args a) {
    const int ib = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    __shared__ __align__(16) uint8_t buf[2][kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sg[kPfMaxKB], s_su[kPfMaxKB];
    __shared__ float s_amax[2][kPfBM];

    {
        const int r = tid >> 1, half = tid & 1;
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        const uint8_t* src = a.xs + (int64_t)tok * KB;
        for (int kb = half; kb < KB; kb += 2) s_sa[r * KB + kb] = src[kb];
    }
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    uint32_t aoff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = (2 * wv + q) * 16 + (lane & 15);
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        aoff[q] = (uint32_t)tok * a.H + (lane >> 4) * 32;
    }
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    for (int i = tid; i < KB; i += 256) {
        s_sg[i] = sb[i * NBS + ib];
        s_su[i] = sb[i * NBS + a.I / kGroup + ib];
    }
    int bn16[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = 4 * wv + j;
        bn16[j] = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
    }
    const uint32_t l16 = lane * 16;
    auto load = [&](int kb, PfLoads& L) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) L.v[q * 2 + h] = bload16(ra, aoff[q] + h * 16, kb * kGroup, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                L.v[4 + j * 2 + h] = bload16(rw, l16, (uint32_t)(bn16[j] * KB + kb) * kFragBytes + h * 1024, 0);
    };
    auto store = [&](const PfLoads& L, uint8_t* st) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint4*>(st + (2 * wv + q) * kFragBytes + h * 1024 + l16) = L.v[q * 2 + h];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint4*>(st + kPfStageA + (4 * wv + j) * kFragBytes + h * 1024 + l16) = L.v[4 + j * 2 + h];
    };

    v4f accg[4][4], accu[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) accg[mi][j] = accu[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    PfLoads R[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) load(min(r, KB - 1), R[r]);
    store(R[0], buf[0]);
    __syncthreads();

    auto compute = [&](int kb, const uint8_t* cur) {
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
        const int sg = s_sg[kb];
        const int su = s_su[kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v8i bg = lds_frag(cur + kPfStageA + (wn * 4 + j) * kFragBytes, lane);
            const v8i bu = lds_frag(cur + kPfStageA + (8 + wn * 4 + j) * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                accg[mi][j] = mfma_fp8(af[mi], bg, accg[mi][j], sa[mi], sg);
                accu[mi][j] = mfma_fp8(af[mi], bu, accu[mi][j], sa[mi], su);
            }
        }
    };
    // step kb: LDS buffer kb%2 holds block kb; register set kb%NR is free (its block was
    // stored a step ago) and takes block kb+NR; after the MMAs, register set (kb+1)%NR
    // (block kb+1, loaded NR-1 steps ago) goes to LDS buffer (kb+1)%2.
    // Loads and stores are unconditional (block indices clamped to the last block; the
    // duplicates land in buffers nobody reads) so the number of loads in flight is the same
    // on every path and the compiler's vmcnt waits stay exact.
    auto step = [&](int kb, const int ri, const int bi) {
        load(min(kb + NR, KB - 1), R[ri]);
        compute(kb, buf[bi]);
        store(R[(ri + 1) % NR], buf[bi ^ 1]);
        __syncthreads();
    };
    constexpr int U = NR == 3 ? 6 : (NR == 4 ? 4 : 2);
    int kb = 0;
    for (; kb + U <= KB; kb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(kb + u, u % NR, u & 1);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb + u < KB) step(kb + u, u % NR, u & 1);

    float hv[4][4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float g = accg[mi][j][i];
                const float h = g / (1.0f + expf(-g)) * accu[mi][j][i];
                hv[mi][j][i] = h;
                m = fmaxf(m, fabsf(h));
            }
            m = max16(m);
            if ((lane & 15) == 0) s_amax[wn][(wm * 4 + mi) * 16 + 4 * (lane >> 4) + i] = m;
        }
    }
    __syncthreads();
    uint8_t* s_h = buf[0];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            const int ex = scale_exponent(fmaxf(s_amax[0][row], s_amax[1][row]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_h[row * 128 + (wn * 4 + j) * 16 + (lane & 15)] =
                    (uint8_t)(cvt2_e4m3(ldexpf(hv[mi][j][i], -ex), 0.f) & 0xFFu);
            if (wn == 0 && (lane & 15) == 0)
                a.hs[((int64_t)tile * kPfBM + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 8 * 128; q += 256) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (mf * 16 + (ln & 15)) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int NR>
__global__ __launch_bounds__(256, 1) void k_gemm2_pfr(G2Args a) {
    const int nb = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    __shared__ __align__(16) uint8_t buf[2][kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sb[2][kPfMaxKB];
    {
        const uint8_t* src = a.hs + (int64_t)tile * kPfBM * KB;
        for (int i = tid; i < kPfBM * KB; i += 256) s_sa[i] = src[i];
    }
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    for (int i = tid; i < 2 * KB; i += 256) s_sb[i & 1][i >> 1] = sb[(i >> 1) * NBS + nb * 2 + (i & 1)];
    const uint32_t l16 = lane * 16;
    auto load = [&](int kb, PfLoads& L) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                L.v[q * 2 + h] = bload16(ra, l16, (uint32_t)((2 * wv + q) * KB + kb) * kFragBytes + h * 1024, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                L.v[4 + j * 2 + h] = bload16(rw, l16, (uint32_t)((nb * 16 + 4 * wv + j) * KB + kb) * kFragBytes + h * 1024, 0);
    };
    auto store = [&](const PfLoads& L, uint8_t* st) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint4*>(st + (2 * wv + q) * kFragBytes + h * 1024 + l16) = L.v[q * 2 + h];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint4*>(st + kPfStageA + (4 * wv + j) * kFragBytes + h * 1024 + l16) = L.v[4 + j * 2 + h];
    };

    v4f acc[4][8];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    PfLoads R[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) load(min(r, KB - 1), R[r]);
    store(R[0], buf[0]);
    __syncthreads();

    auto compute = [&](int kb, const uint8_t* cur) {
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
        const int sbv = s_sb[wn][kb];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const v8i b = lds_frag(cur + kPfStageA + (wn * 8 + j) * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mfma_fp8(af[mi], b, acc[mi][j], sa[mi], sbv);
        }
    };
    // step kb: LDS buffer kb%2 holds block kb; register set kb%NR is free (its block was
    // stored a step ago) and takes block kb+NR; after the MMAs, register set (kb+1)%NR
    // (block kb+1, loaded NR-1 steps ago) goes to LDS buffer (kb+1)%2.
    // Loads and stores are unconditional (block indices clamped to the last block; the
    // duplicates land in buffers nobody reads) so the number of loads in flight is the same
    // on every path and the compiler's vmcnt waits stay exact.
    auto step = [&](int kb, const int ri, const int bi) {
        load(min(kb + NR, KB - 1), R[ri]);
        compute(kb, buf[bi]);
        store(R[(ri + 1) % NR], buf[bi ^ 1]);
        __syncthreads();
    };
    constexpr int U = NR == 3 ? 6 : (NR == 4 ? 4 : 2);
    int kb = 0;
    for (; kb + U <= KB; kb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(kb + u, u % NR, u & 1);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb + u < KB) step(kb + u, u % NR, u & 1);

#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int col = nb * 256 + (wn * 8 + j) * 16 + (lane & 15);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[mi][j][i]);
                    else reinterpret_cast<float*>(a.out)[o + col] = acc[mi][j][i];
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Column-split prefill variants: wave w owns all 8 row fragments of the 128-row tile and 4
// column fragments, so no B fragment is shared between waves.  A (the 8 row fragments of a
// K block, 16 KB) is staged once in LDS for all four waves, register-staged and double
// buffered (thread t owns the 16-byte pieces t, t+256, t+512, t+768; piece p sits at byte
// 16p of the LDS block, i.e. fragment p/128 in matrix-core order).  B fragments stream from
// memory straight into each wave's registers PFB K blocks ahead.  LDS traffic per K block
// and workgroup: 16 KB written + 64 KB read.

template <bool kG1, int PFB>
struct PfnCore {
    // one K block: 8 row fragments x 4 column fragments of MFMAs for this wave
    static __device__ __forceinline__ void mma(v4f (&acc)[8][4], const uint8_t* ab, const v8i (&b)[4],
                                               const uint8_t* s_sa, int KB, int kb, int lane, const int (&sbv)[4]) {
#pragma unroll
        for (int mf = 0; mf < 8; ++mf) {
            const v8i af = lds_frag(ab + mf * kFragBytes, lane);
            const int sa = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mf][j] = mfma_fp8(af, b[j], acc[mf][j], sa, sbv[j]);
        }
    }
};

template <int PFB>
__global__ __launch_bounds__(256, 1) void k_gemm1_pfn(G1Args a) {
    const int ib = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);

    __shared__ __align__(16) uint8_t abuf[2][8 * kFragBytes];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sg[kPfMaxKB], s_su[kPfMaxKB];
    __shared__ float s_amax[4][kPfBM];

    {
        const int r = tid >> 1, half = tid & 1;
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        const uint8_t* src = a.xs + (int64_t)tok * KB;
        for (int kb = half; kb < KB; kb += 2) s_sa[r * KB + kb] = src[kb];
    }
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    for (int i = tid; i < KB; i += 256) {
        s_sg[i] = sb[i * NBS + ib];
        s_su[i] = sb[i * NBS + a.I / kGroup + ib];
    }
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, mf = p >> 7, hh = (p >> 6) & 1, ln = p & 63;
        const int r = mf * 16 + (ln & 15);
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        aoff[i] = (uint32_t)tok * a.H + (ln >> 4) * 32 + hh * 16;
    }
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const int g16 = ib * 8 + 2 * wv, u16 = a.I / 16 + g16;
    const int bn16[4] = {g16, g16 + 1, u16, u16 + 1};
    const uint32_t l16 = lane * 16;

    v4f acc[8][4];
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mf][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 R[2][4];
    v8i bq[PFB][4];
    auto loadA = [&](int kb, uint4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = bload16(ra, aoff[i], kb * kGroup, 0);
    };
    auto storeA = [&](const uint4 (&r)[4], uint8_t* ab) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(ab + (tid + 256 * i) * 16) = r[i];
    };
    auto loadB = [&](int kb, v8i (&b)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = buf_frag(rw, l16, (uint32_t)(bn16[j] * KB + kb) * kFragBytes);
    };
    loadA(0, R[0]);
    if (KB > 1) loadA(1, R[1]);
#pragma unroll
    for (int p = 0; p < PFB; ++p)
        if (p < KB) loadB(p, bq[p]);
    storeA(R[0], abuf[0]);
    __syncthreads();

    auto step = [&](int kb, const int p, const int ab) {
        if (kb + 2 < KB) loadA(kb + 2, R[ab]);
        const int sg = s_sg[kb], su = s_su[kb];
        const int sbv[4] = {sg, sg, su, su};
        PfnCore<true, PFB>::mma(acc, abuf[ab], bq[p], s_sa, KB, kb, lane, sbv);
        if (kb + PFB < KB) loadB(kb + PFB, bq[p]);
        if (kb + 1 < KB) storeA(R[ab ^ 1], abuf[ab ^ 1]);
        __syncthreads();
    };
    static_assert(PFB == 2 || PFB == 4, "the K loop is unrolled by 4");
    for (int kb = 0; kb < KB; kb += 4) {
        step(kb, 0, 0);
        if (kb + 1 < KB) step(kb + 1, 1 % PFB, 1);
        if (kb + 2 < KB) step(kb + 2, 2 % PFB, 0);
        if (kb + 3 < KB) step(kb + 3, 3 % PFB, 1);
    }

    // ---- epilogue: SwiGLU on this wave's 32 columns, row amax over the four waves, requant
    float hv[8][2][4];
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const float g = acc[mf][jj][i];
                const float h = g / (1.0f + expf(-g)) * acc[mf][2 + jj][i];
                hv[mf][jj][i] = h;
                m = fmaxf(m, fabsf(h));
            }
            m = max16(m);
            if ((lane & 15) == 0) s_amax[wv][mf * 16 + 4 * (lane >> 4) + i] = m;
        }
    }
    __syncthreads();
    uint8_t* s_h = abuf[0];   // [128][128] bytes
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mf * 16 + 4 * (lane >> 4) + i;
            const float am = fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row]));
            const int ex = scale_exponent(am);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                s_h[row * 128 + (2 * wv + jj) * 16 + (lane & 15)] =
                    (uint8_t)(cvt2_e4m3(ldexpf(hv[mf][jj][i], -ex), 0.f) & 0xFFu);
            if (wv == 0 && (lane & 15) == 0)
                a.hs[((int64_t)tile * kPfBM + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 8 * 128; q += 256) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (mf * 16 + (ln & 15)) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int PFB>
__global__ __launch_bounds__(256, 1) void k_gemm2_pfn(G2Args a) {
    const int nb = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);

    __shared__ __align__(16) uint8_t abuf[2][8 * kFragBytes];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sb[2][kPfMaxKB];   // the workgroup's two 128-column scale blocks
    {
        const uint8_t* src = a.hs + (int64_t)tile * kPfBM * KB;
        for (int i = tid; i < kPfBM * KB; i += 256) s_sa[i] = src[i];
    }
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    for (int i = tid; i < 2 * KB; i += 256) s_sb[i & 1][i >> 1] = sb[(i >> 1) * NBS + nb * 2 + (i & 1)];
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const int n16 = nb * 16 + 4 * wv;
    const int sblk = wv >> 1;   // this wave's 64 columns lie in scale block nb*2 + wv/2
    const uint32_t l16 = lane * 16;

    v4f acc[8][4];
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mf][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 R[2][4];
    v8i bq[PFB][4];
    auto loadA = [&](int kb, uint4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i;
            r[i] = bload16(ra, (p & 127) * 16, (uint32_t)((p >> 7) * KB + kb) * kFragBytes, 0);
        }
    };
    auto storeA = [&](const uint4 (&r)[4], uint8_t* ab) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(ab + (tid + 256 * i) * 16) = r[i];
    };
    auto loadB = [&](int kb, v8i (&b)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = buf_frag(rw, l16, (uint32_t)((n16 + j) * KB + kb) * kFragBytes);
    };
    loadA(0, R[0]);
    if (KB > 1) loadA(1, R[1]);
#pragma unroll
    for (int p = 0; p < PFB; ++p)
        if (p < KB) loadB(p, bq[p]);
    storeA(R[0], abuf[0]);
    __syncthreads();

    auto step = [&](int kb, const int p, const int ab) {
        if (kb + 2 < KB) loadA(kb + 2, R[ab]);
        const int s = s_sb[sblk][kb];
        const int sbv[4] = {s, s, s, s};
        PfnCore<false, PFB>::mma(acc, abuf[ab], bq[p], s_sa, KB, kb, lane, sbv);
        if (kb + PFB < KB) loadB(kb + PFB, bq[p]);
        if (kb + 1 < KB) storeA(R[ab ^ 1], abuf[ab ^ 1]);
        __syncthreads();
    };
    static_assert(PFB == 2 || PFB == 4, "the K loop is unrolled by 4");
    for (int kb = 0; kb < KB; kb += 4) {
        step(kb, 0, 0);
        if (kb + 1 < KB) step(kb + 1, 1 % PFB, 1);
        if (kb + 2 < KB) step(kb + 2, 2 % PFB, 0);
        if (kb + 3 < KB) step(kb + 3, 3 % PFB, 1);
    }

#pragma unroll
    for (int mf = 0; mf < 8; ++mf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mf * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = (n16 + j) * 16 + (lane & 15);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[mf][j][i]);
                    else reinterpret_cast<float*>(a.out)[o + col] = acc[mf][j][i];
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// 8-wave prefill variants: the 128 x 256 tile split over 2 (rows) x 4 (columns) waves of
// 64 x 64 (4 x 4 fragments), two waves per SIMD so one wave's LDS and load waits overlap the
// other's matrix-core work.  Operands are register-staged through two LDS buffers as in the
// 4-wave variant; each of the 512 threads moves 6 16-byte pieces per K block (2 of A, 4 of B).
// Piece p of a stage sits at byte 16 p: fragment p / 128, half (p / 64) % 2, lane p % 64.

struct Pf8Loads {
    uint4 v[6];
};

template <int NR>
__global__ __launch_bounds__(512, 1) void k_gemm1_pf8(G1Args a) {
    const int ib = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2][kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sg[kPfMaxKB], s_su[kPfMaxKB];
    __shared__ float s_amax[4][kPfBM];

    if (tid < 2 * kPfBM) {
        const int r = tid >> 1, half = tid & 1;
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        const uint8_t* src = a.xs + (int64_t)tok * KB;
        for (int kb = half; kb < KB; kb += 2) s_sa[r * KB + kb] = src[kb];
    }
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    for (int i = tid; i < KB; i += 512) {
        s_sg[i] = sb[i * NBS + ib];
        s_su[i] = sb[i * NBS + a.I / kGroup + ib];
    }
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + 512 * i, mf = p >> 7, hh = (p >> 6) & 1, ln = p & 63;
        const int r = mf * 16 + (ln & 15);
        const int tok = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
        aoff[i] = (uint32_t)tok * a.H + (ln >> 4) * 32 + hh * 16;
    }
    int bsoff[4];   // wave-uniform byte offset of the piece's fragment row and half
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = wv * 64 + 512 * i, f = q >> 7, hh = (q >> 6) & 1;
        const int n16 = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
        bsoff[i] = __builtin_amdgcn_readfirstlane(n16 * KB * kFragBytes + hh * 1024);
    }
    const uint32_t l16 = lane * 16;
    auto load = [&](int kb, Pf8Loads& L) {
#pragma unroll
        for (int i = 0; i < 2; ++i) L.v[i] = bload16(ra, aoff[i], kb * kGroup, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) L.v[2 + i] = bload16(rw, l16, (uint32_t)(bsoff[i] + kb * kFragBytes), 0);
    };
    auto store = [&](const Pf8Loads& L, uint8_t* st) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(st + (tid + 512 * i) * 16) = L.v[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(st + kPfStageA + (tid + 512 * i) * 16) = L.v[2 + i];
    };

    v4f acc[4][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    Pf8Loads R[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) load(min(r, KB - 1), R[r]);
    store(R[0], buf[0]);
    __syncthreads();

    auto compute = [&](int kb, const uint8_t* cur) {
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
        const int sg = s_sg[kb], su = s_su[kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = j < 2 ? 2 * wn + j : 8 + 2 * wn + (j - 2);
            const v8i b = lds_frag(cur + kPfStageA + f * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mfma_fp8(af[mi], b, acc[mi][j], sa[mi], j < 2 ? sg : su);
        }
    };
    // Same step order as the 4-wave kernel: load block kb+NR, compute block kb, store block kb+1.
    auto step = [&](int kb, const int ri, const int bi) {
        load(min(kb + NR, KB - 1), R[ri]);
        compute(kb, buf[bi]);
        store(R[(ri + 1) % NR], buf[bi ^ 1]);
        __syncthreads();
    };
    constexpr int U = NR == 3 ? 6 : (NR == 4 ? 4 : 2);
    int kb = 0;
    for (; kb + U <= KB; kb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(kb + u, u % NR, u & 1);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb + u < KB) step(kb + u, u % NR, u & 1);

    float hv[4][2][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const float g = acc[mi][jj][i];
                const float h = g / (1.0f + expf(-g)) * acc[mi][2 + jj][i];
                hv[mi][jj][i] = h;
                m = fmaxf(m, fabsf(h));
            }
            m = max16(m);
            if ((lane & 15) == 0) s_amax[wn][(wm * 4 + mi) * 16 + 4 * (lane >> 4) + i] = m;
        }
    }
    __syncthreads();
    uint8_t* s_h = buf[0];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            const float am = fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row]));
            const int ex = scale_exponent(am);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                s_h[row * 128 + (2 * wn + jj) * 16 + (lane & 15)] =
                    (uint8_t)(cvt2_e4m3(ldexpf(hv[mi][jj][i], -ex), 0.f) & 0xFFu);
            if (wn == 0 && (lane & 15) == 0)
                a.hs[((int64_t)tile * kPfBM + row) * (a.I / kGroup) + ib] = (uint8_t)(ex + 127);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 8 * 128; q += 512) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + (mf * 16 + (ln & 15)) * 128 + (ln >> 4) * 32 + hh * 16);
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int NR>
__global__ __launch_bounds__(512, 1) void k_gemm2_pf8(G2Args a) {
    const int nb = blockIdx.x;
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2][kPfStage];
    __shared__ uint8_t s_sa[kPfBM * kPfMaxKB];
    __shared__ uint8_t s_sb[2][kPfMaxKB];
    {
        const uint8_t* src = a.hs + (int64_t)tile * kPfBM * KB;
        for (int i = tid; i < kPfBM * KB; i += 512) s_sa[i] = src[i];
    }
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
    for (int i = tid; i < 2 * KB; i += 512) s_sb[i & 1][i >> 1] = sb[(i >> 1) * NBS + nb * 2 + (i & 1)];
    const rsrc_t ra = make_rsrc(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const rsrc_t rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint32_t l16 = lane * 16;
    int asoff[2], bsoff[4];   // wave-uniform byte offsets of the pieces' fragment rows and halves
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = wv * 64 + 512 * i, mf = p >> 7, hh = (p >> 6) & 1;
        asoff[i] = __builtin_amdgcn_readfirstlane(mf * KB * kFragBytes + hh * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = wv * 64 + 512 * i, f = q >> 7, hh = (q >> 6) & 1;
        bsoff[i] = __builtin_amdgcn_readfirstlane((nb * 16 + f) * KB * kFragBytes + hh * 1024);
    }
    auto load = [&](int kb, Pf8Loads& L) {
#pragma unroll
        for (int i = 0; i < 2; ++i) L.v[i] = bload16(ra, l16, (uint32_t)(asoff[i] + kb * kFragBytes), 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) L.v[2 + i] = bload16(rw, l16, (uint32_t)(bsoff[i] + kb * kFragBytes), 0);
    };
    auto store = [&](const Pf8Loads& L, uint8_t* st) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(st + (tid + 512 * i) * 16) = L.v[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(st + kPfStageA + (tid + 512 * i) * 16) = L.v[2 + i];
    };

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    Pf8Loads R[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) load(min(r, KB - 1), R[r]);
    store(R[0], buf[0]);
    __syncthreads();

    auto compute = [&](int kb, const uint8_t* cur) {
        v8i af[4];
        int sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            af[mi] = lds_frag(cur + mf * kFragBytes, lane);
            sa[mi] = s_sa[(mf * 16 + (lane & 15)) * KB + kb];
        }
        const int sbv = s_sb[wn >> 1][kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v8i b = lds_frag(cur + kPfStageA + (wn * 4 + j) * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mfma_fp8(af[mi], b, acc[mi][j], sa[mi], sbv);
        }
    };
    auto step = [&](int kb, const int ri, const int bi) {
        load(min(kb + NR, KB - 1), R[ri]);
        compute(kb, buf[bi]);
        store(R[(ri + 1) % NR], buf[bi ^ 1]);
        __syncthreads();
    };
    constexpr int U = NR == 3 ? 6 : (NR == 4 ? 4 : 2);
    int kb = 0;
    for (; kb + U <= KB; kb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(kb + u, u % NR, u & 1);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb + u < KB) step(kb + u, u % NR, u & 1);

#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = nb * 256 + (wn * 4 + j) * 16 + (lane & 15);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(acc[mi][j][i]);
                    else reinterpret_cast<float*>(a.out)[o + col] = acc[mi][j][i];
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Decode tiles (16 rows) while experts average at most this many rows; 128-row tiles above.
#ifndef MOE_DEC_MAX_AVG_ROWS
#define MOE_DEC_MAX_AVG_ROWS 24
#endif

FfnPlan ffn_plan(int T, int k, int E) {
    const int64_t A = (int64_t)T * k;
    const int64_t avg = A / E;
    FfnPlan p;
    p.BM = avg <= MOE_DEC_MAX_AVG_ROWS ? 16 : 128;
    p.ntiles_max = (int)(ceil_div(A, p.BM) + std::min<int64_t>(E, A));
    return p;
}

// workspace: tiles [ntiles_max] int2 | ntiles int | hq [ntiles_max*BM, I] | hs [ntiles_max*BM, I/128]
size_t ffn_workspace_bytes(int T, int H, int I, int E, int k) {
    (void)H;
    const FfnPlan p = ffn_plan(T, k, E);
    const size_t rows = (size_t)p.ntiles_max * p.BM;
    return align256((size_t)p.ntiles_max * 8) + align256(4) + align256(rows * I) + align256(rows * (I / kGroup));
}

template <int MFW, int NFW1, int NFW2, int WM, int WN, int PF1, int PF2>
static hipError_t run_ffn(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    G1Args g1{f.xq, f.xs, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles, f.w13p, f.w13s,
              w.hq, w.hs};
    hipLaunchKernelGGL((k_gemm1<MFW, NFW1, WM, WN, PF1>), dim3(p.ntiles_max, f.I / kGroup), dim3(64 * WM * WN), 0,
                       st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    G2Args g2{w.hq, w.hs, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16};
    const int ncols = 16 * NFW2 * WN;
    hipLaunchKernelGGL((k_gemm2<MFW, NFW2, WM, WN, PF2>), dim3(p.ntiles_max, f.H / ncols), dim3(64 * WM * WN), 0,
                       st, g2);
    return hipGetLastError();
}

template <int NFW1, int WN1, int PF1, int NFW2, int WN2, int PF2>
static hipError_t run_ffn_dec(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    G1Args g1{f.xq, f.xs, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles, f.w13p, f.w13s,
              w.hq, w.hs};
    hipLaunchKernelGGL((k_gemm1_dec<NFW1, WN1, PF1>), dim3(p.ntiles_max, f.I / kGroup), dim3(64 * WN1), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    G2Args g2{w.hq, w.hs, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16};
    hipLaunchKernelGGL((k_gemm2_dec<NFW2, WN2, PF2>), dim3(p.ntiles_max, f.H / (16 * NFW2 * WN2)), dim3(64 * WN2), 0,
                       st, g2);
    return hipGetLastError();
}

static hipError_t run_ffn_pf(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    G1Args g1{f.xq, f.xs, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles, f.w13p, f.w13s,
              w.hq, w.hs};
    hipLaunchKernelGGL((MOE_PF_GEMM1), dim3(f.I / kGroup, p.ntiles_max), dim3(MOE_PF_THREADS), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    G2Args g2{w.hq, w.hs, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16};
    hipLaunchKernelGGL((MOE_PF_GEMM2), dim3(f.H / 256, p.ntiles_max), dim3(MOE_PF_THREADS), 0, st, g2);
    return hipGetLastError();
}

FfnWs carve_ffn_ws(const FfnArgs& f, void* ws) {
    const FfnPlan p = ffn_plan(f.T, f.k, f.E);
    const size_t rows = (size_t)p.ntiles_max * p.BM;
    uint8_t* w = static_cast<uint8_t*>(ws);
    FfnWs r;
    r.tiles = reinterpret_cast<int2*>(w);
    w += align256((size_t)p.ntiles_max * 8);
    r.ntiles = reinterpret_cast<int32_t*>(w);
    w += align256(4);
    r.hq = w;
    w += align256(rows * f.I);
    r.hs = w;
    return r;
}

hipError_t launch_grouped_ffn(const FfnArgs& f, void* ws, hipStream_t st, hipEvent_t mid, bool tiles_ready) {
    const FfnPlan p = ffn_plan(f.T, f.k, f.E);
    const FfnWs w = carve_ffn_ws(f, ws);
    if (!tiles_ready) {
        const hipError_t e = launch_tiles(f.counts, f.E, p.BM, w.tiles, w.ntiles, st);
        if (e != hipSuccess) return e;
    }
    // output columns per workgroup of the down GEMM = 128, a divisor of H
    if (p.BM == 16) return run_ffn_dec<MOE_DEC_GEMM1, MOE_DEC_GEMM2>(f, p, w, st, mid);
    // 128-row tiles: the staged kernels need the tile's A scales in LDS and 256-column
    // down-GEMM blocks; other shapes take the plain 128-row kernels
    if (f.H / kGroup <= kPfMaxKB && f.I / kGroup <= kPfMaxKB && f.H % 256 == 0)
        return run_ffn_pf(f, p, w, st, mid);
    return run_ffn<4, 4, 4, 2, 2, 2, 2>(f, p, w, st, mid);
}

// ----------------------------------------------------------------------------------------
// Combine: workgroup (token, 1024-column slice); each thread owns 4 consecutive columns and
// issues the loads of up to 8 expert rows before summing them in slot order j = 0, 1, ...
template <bool BF16>
__device__ __forceinline__ float4 load4(const void* eo, int64_t idx) {
    if (BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(eo) + idx);
        return make_float4(bf16_to_f32(u.x & 0xFFFFu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFFu),
                           bf16_to_f32(u.y >> 16));
    }
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(eo) + idx);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ eo, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int k, int H,
                                                 uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int c4 = blockIdx.y * 256 + threadIdx.x;
    if (c4 * 4 >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 v[8];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int p = j < k ? pos[(int64_t)t * k + j] : -1;
            wj[u] = p >= 0 ? w[(int64_t)t * k + j] : 0.f;
            v[u] = p >= 0 ? load4<BF16>(eo, (int64_t)p * H + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                acc.x = fmaf(wj[u], v[u].x, acc.x);
                acc.y = fmaf(wj[u], v[u].y, acc.y);
                acc.z = fmaf(wj[u], v[u].z, acc.z);
                acc.w = fmaf(wj[u], v[u].w, acc.w);
            }
        }
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + (int64_t)t * H + c4 * 4) = o;
}

hipError_t launch_combine(const void* eo, int bf16, const int32_t* pos, const float* w, int T, int k, int H,
                          uint16_t* y, hipStream_t st) {
    const dim3 grid(T, (unsigned)ceil_div(H / 4, 256));
    if (bf16) hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, st, eo, pos, w, k, H, y);
    else hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, st, eo, pos, w, k, H, y);
    return hipGetLastError();
}

}  // namespace moe
