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
#include "mx_common.h"
#include "work_items.h"

#include <algorithm>
#include <type_traits>

// Decode-tile configurations (fragments per wave, waves per workgroup, K blocks in flight)
// of the gate+up and the down GEMM; fixed at build time.
#ifndef MOE_DEC_GEMM1
#define MOE_DEC_GEMM1 1, 8, 2
#endif
#ifndef MOE_DEC_GEMM2
#define MOE_DEC_GEMM2 2, 4, 2
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
    int ord;    // work order of the 128-row-tile kernels: 1 super-tiles (ord_item), 0 column blocks
    const int4* pairs;       // 256-row items: {first tile, expert, first sorted row, valid rows}
    const int32_t* npairs;   // and the pair count
    float* htap;             // test output: float32 h [A, I] in sorted order (kernels built with TAP)
    const float* b13;        // optional gate/up bias [E, 2I]
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
template <int MFW, int NFW, int WM, int WN, int PF, bool TAP>
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
    GuBias bias[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) bias[j] = gu_bias(a.b13, e, a.I, ib * 128 + (wn * NFW + j) * 16 + (lane & 15));
    float hv[MFW][NFW][4];
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const float g = add_bias(a.b13, accg[mi][j][i], bias[j].g);
                const float h = g / (1.0f + expf(-g)) * add_bias(a.b13, accu[mi][j][i], bias[j].u);
                hv[mi][j][i] = h;
                m = fmaxf(m, fabsf(h));
                tap_h<TAP>(a.htap, a.I, rowbase, (wm * MFW + mi) * 16 + 4 * (lane >> 4) + i, nvalid,
                           ib * 128 + (wn * NFW + j) * 16 + (lane & 15), h);
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
    int ord;
    const int4* pairs;
    const int32_t* npairs;
    const float* b2;         // optional down bias [E, H]
    int wnt = 0;             // 256-row down items: weights by non-temporal loads (each read by one item)
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
    float bias[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) bias[j] = out_bias(a.b2, e, a.H, (n16 + j) * 16 + (lane & 15));
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
                    const float v = add_bias(a.b2, acc[mi][j][i], bias[j]);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(v);
                    else reinterpret_cast<float*>(a.out)[o + col] = v;
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

template <int NFW, int WN, int PF, bool TAP>
__global__ __launch_bounds__(64 * WN) void k_gemm1_dec(G1Args a) {
    static_assert(NFW * WN == 8, "a workgroup covers 128 gate + 128 up columns");
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int ib = blockIdx.y;
    const int2 te = a.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ float s_amax[WN][16];
    __shared__ __align__(16) uint8_t s_h[16 * 128];
    __shared__ uint8_t s_sg[kMaxKB], s_su[kMaxKB];   // weight-block scales of this column block

    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const rsrc_t rw = make_rsrc(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint8_t* sb = a.w13s + (int64_t)e * KB * NBS;
    const int g16 = ib * 8 + wn * NFW;
    const int u16 = a.I / 16 + g16;
    const uint32_t l16 = lane * 16;
    // request order: the token id (oldest, so waiting for it waits for nothing else), the
    // block scales, the first PF weight blocks, then the activations that need the id; the
    // weight stream starts with the workgroup instead of after a round trip for the scales
    static_assert(64 * WN >= kMaxKB, "one scale pair per thread");
    const int nvalid = min(16, a.counts[e] - m0);
    const int rowbase = a.offsets[e] + m0;
    const int f0 = a.sorted_assign[rowbase + min(lane & 15, nvalid - 1)];   // used after the weight requests
    const int si = min(tid, KB - 1);   // every thread loads (no branch: the wait for the id stays exact)
    const uint8_t sg8 = sb[si * NBS + ib], su8 = sb[si * NBS + a.I / kGroup + ib];
    v8i aq[PF], bq[PF][2 * NFW];
    int sa[PF];
    // unconditional (blocks p >= KB are never used; the buffer loads stay inside their
    // descriptors' ranges or read zero), so no branch blurs the waits
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            bq[p][j] = buf_frag(rw, l16, ((g16 + j) * KB + p) * kFragBytes);
            bq[p][NFW + j] = buf_frag(rw, l16, ((u16 + j) * KB + p) * kFragBytes);
        }
    __builtin_amdgcn_sched_barrier(0);
    const int tok = f0 / a.k;
    const rsrc_t ra = make_rsrc(a.xq, (uint32_t)a.T * a.H);
    const uint32_t av = (uint32_t)tok * a.H + (lane >> 4) * 32;
    const uint8_t* sp = a.xs + (int64_t)tok * KB;
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        aq[p] = buf_a32(ra, av, p * kGroup);
        sa[p] = sp[min(p, KB - 1)];
    }
    if (tid < KB) {
        s_sg[tid] = sg8;
        s_su[tid] = su8;
    }
    __syncthreads();

    v4f accg[NFW], accu[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) accg[j] = accu[j] = v4f{0.f, 0.f, 0.f, 0.f};
    // The refills are unconditional: past the last block their offsets point outside the
    // descriptors' ranges (bit 31 set), so they read zero without touching memory.  With no
    // branch around them the loaded registers need no merge copies, and the waits stay at
    // "the block about to be used" instead of draining the whole pipeline.
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
            }
            const int kn = kb + PF;
            const bool more = kn < KB;
            const int kc = more ? kn : 0;
            const uint32_t off_ok = more ? 0u : 0x80000000u;
            aq[p] = buf_a32(ra, av | off_ok, kc * kGroup);
            sa[p] = sp[min(kn, KB - 1)];
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                bq[p][j] = buf_frag(rw, l16 | off_ok, ((g16 + j) * KB + kc) * kFragBytes);
                bq[p][NFW + j] = buf_frag(rw, l16 | off_ok, ((u16 + j) * KB + kc) * kFragBytes);
            }
        }
    }
    // epilogue: SwiGLU, row amax over the 128 columns (across the WN waves), requant
    GuBias bias[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) bias[j] = gu_bias(a.b13, e, a.I, ib * 128 + (wn * NFW + j) * 16 + (lane & 15));
    float hv[NFW][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            const float g = add_bias(a.b13, accg[j][i], bias[j].g);
            const float h = g / (1.0f + expf(-g)) * add_bias(a.b13, accu[j][i], bias[j].u);
            hv[j][i] = h;
            m = fmaxf(m, fabsf(h));
            tap_h<TAP>(a.htap, a.I, rowbase, 4 * (lane >> 4) + i, nvalid, ib * 128 + (wn * NFW + j) * 16 + (lane & 15), h);
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
    static_assert(64 * WN >= kMaxKB, "one scale per thread");
    __shared__ uint8_t s_sb[kMaxKB];
    // the block scale, the first PF weight and h blocks, then the row scales, all requested
    // before the one barrier (the loads are unconditional: no branch blurs the waits; blocks
    // p >= KB read inside their descriptors' ranges or zero and are never used)
    const uint8_t sb8 = sb[min((int)threadIdx.x, KB - 1) * NBS + blockIdx.y];
    int sa[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) sa[p] = sp[min(p, KB - 1)];
    __builtin_amdgcn_sched_barrier(0);
    v8i aq[PF], bq[PF][NFW];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
        for (int j = 0; j < NFW; ++j) bq[p][j] = buf_frag(rw, l16, ((n16 + j) * KB + p) * kFragBytes);
        aq[p] = buf_frag(ra, l16, p * kFragBytes);
    }
    if ((int)threadIdx.x < KB) s_sb[threadIdx.x] = sb8;
    __syncthreads();

    v4f acc[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
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
// Prefill kernels: workgroup tile 128 rows x 256 columns, 8 waves as 2 (rows) x 4 (columns)
// of 64 x 64 (4 x 4 matrix-core fragments), two waves per SIMD so one wave's LDS waits
// overlap the other's matrix-core work.  Operands travel global -> LDS by the LDS-DMA form
// of the buffer load (no staging registers, no LDS store instructions) through a 3-stage
// ring of 48 KB stages, so two K blocks (96 KB per CU) are in flight while the waves compute
// the third.  Each of the 512 threads moves 6 16-byte pieces per K block (2 of A, 4 of B);
// piece p of a stage sits at byte 16 p: fragment p / 128, half (p / 64) % 2, lane p % 64.
// The A row scales of all K blocks and the weight block scales of the workgroup's columns
// sit in LDS.

constexpr int kPfBM = 128, kPfStageA = 8 * kFragBytes, kPfStage = kPfStageA + 16 * kFragBytes;  // 48 KB
constexpr int kPfMaxKB = 64;     // K blocks whose A scales fit the LDS table

// Work order of the prefill grids (one dimension, ncol * tiles workgroups rounded up to a
// multiple of kXcds).  Workgroup L runs on XCD L % kXcds (the dispatcher deals workgroups to
// the XCDs in turn), so XCD x takes the contiguous share x of the work list; the list walks
// super-blocks of kPfGroupTiles consecutive tiles (mostly one expert), and inside a
// super-block the column block is the outer index.  The workgroups that run together on one
// XCD then share both their A tiles and their weight column blocks through that XCD's L2.
constexpr int kXcds = 8;
#ifndef MOE_PF_GROUP_TILES
#define MOE_PF_GROUP_TILES 4
#endif
constexpr int kPfGroupTiles = MOE_PF_GROUP_TILES;

__device__ __forceinline__ bool pf_work_item(int ord, int ncol, int ntiles, int& tile, int& col) {
    const int L = blockIdx.x;
    if (ord) return ord_item(L % kXcds, L / kXcds, ntiles, ncol, tile, col);
    const int total = ntiles * ncol;
    const int per = (total + kXcds - 1) / kXcds;
    const int w = (L % kXcds) * per + L / kXcds;
    if (L / kXcds >= per || w >= total) return false;
    const int sb = w / (kPfGroupTiles * ncol), r = w - sb * kPfGroupTiles * ncol;
    const int t0 = sb * kPfGroupTiles;
    const int g = min(kPfGroupTiles, ntiles - t0);
    col = r / g;
    tile = t0 + r - col * g;
    return true;
}

// ----------------------------------------------------------------------------------------
// The DMA is issued from inline asm: the compiler does not track it, so it inserts no wait
// before the LDS reads of the other stages (it cannot tell which stage a DMA writes and
// would wait for all of them); completion of a stage is awaited explicitly (each thread's
// own DMAs by vmcnt, then a barrier for everyone's).  No register receives data from these
// loads.  A scales are kept per K block ([kb][row]) so that the 16 rows a wave reads sit in
// consecutive bytes (no LDS bank conflicts).

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
constexpr int kPfdStages = 3;

// Buffer descriptor in scalar registers (the base and size are wave-uniform).
__device__ __forceinline__ v4i_t make_srd(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    v4i_t r;
    r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)b);
    r[1] = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu);   // stride 0
    r[2] = (int)__builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p);
}

// 16 bytes per lane from the buffer at voff + soff into LDS at m0base + 16 * lane.
__device__ __forceinline__ void dma16_async(const v4i_t& srd, uint32_t m0base, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0base), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

// dma16_async with the non-temporal cache policy (data read once).
__device__ __forceinline__ void dma16_async_nt(const v4i_t& srd, uint32_t m0base, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(m0base), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

// Wait until at most N of this thread's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Scaled FP8 matrix-core product taking the A scale from byte ba of sa and the B scale from
// byte bb of sb (the instruction's scale byte selects; ba, bb are constants after unrolling).
__device__ __forceinline__ v4f mfma_fp8_sel(int ba, int bb, v8i a, v8i b, v4f acc, int sa, int sb) {
#define MOE_SEL(A, B) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, A, sa, B, sb)
    switch (ba * 2 + bb) {
        case 0: MOE_SEL(0, 0);
        case 1: MOE_SEL(0, 1);
        case 2: MOE_SEL(1, 0);
        case 3: MOE_SEL(1, 1);
        case 4: MOE_SEL(2, 0);
        case 5: MOE_SEL(2, 1);
        case 6: MOE_SEL(3, 0);
        default: MOE_SEL(3, 1);
    }
#undef MOE_SEL
}

// ---- epilogue helpers of the gate/up kernels
// Max over each aligned group of 16 lanes for four values at once: the four DPP chains are
// interleaved, so no step waits on its own predecessor.
__device__ __forceinline__ void max16x4(float (&m)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], dpp_f32<0xB1>(m[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], dpp_f32<0x4E>(m[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], dpp_f32<0x124>(m[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], dpp_f32<0x128>(m[i]));
}

// SwiGLU of one 16-row fragment: gate columns acc[jj], up columns acc[2 + jj] (jj = 0, 1),
// plus the lane's column biases when b13 is set -> h[jj][i]; m[i] = max |h| of row
// 4 (lane / 16) + i over the 32 columns of the two fragments (in every lane of the 16-lane group).
template <bool BIAS>
__device__ __forceinline__ void swiglu_frag_b(const v4f* acc, const GuBias (&bias)[2], float (&h)[2][4],
                                              float (&m)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m[i] = 0.f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float g = BIAS ? acc[jj][i] + bias[jj].g : acc[jj][i];
            const float u = BIAS ? acc[2 + jj][i] + bias[jj].u : acc[2 + jj][i];
            h[jj][i] = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504f)) * u;
            m[i] = fmaxf(m[i], fabsf(h[jj][i]));
        }
    }
    max16x4(m);
}
// (the bias test is uniform: one branch per fragment instead of a select per value)
__device__ __forceinline__ void swiglu_frag(const v4f* acc, const float* b13, const GuBias (&bias)[2],
                                            float (&h)[2][4], float (&m)[4]) {
    if (b13) swiglu_frag_b<true>(acc, bias, h, m);
    else swiglu_frag_b<false>(acc, bias, h, m);
}

// E4M3 bytes of a lane quad's 4 x 4 block (lane 4Q + q of a 16-lane group holds column
// 4Q + q of rows 0..3, scaled by 2^-ex[i]), transposed within the quad (two DPP exchanges
// and a byte select): the result holds row q, columns 4Q .. 4Q + 3 (byte k = column 4Q + k).
__device__ __forceinline__ uint32_t e4m3_quad_rows(const float (&h)[4], const int (&ex)[4], int q) {
    const int x = (int)cvt4_e4m3(ldexpf(h[0], -ex[0]), ldexpf(h[1], -ex[1]), ldexpf(h[2], -ex[2]), ldexpf(h[3], -ex[3]));
    const int z = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // lane q ^ 2
    const int x1 = q < 2 ? (int)(((uint32_t)x & 0xFFFFu) | ((uint32_t)z << 16))
                         : (int)(((uint32_t)z >> 16) | ((uint32_t)x & 0xFFFF0000u));
    const int w = __builtin_amdgcn_update_dpp(0, x1, 0xB1, 0xF, 0xF, false);  // lane q ^ 1
    return __builtin_amdgcn_perm((uint32_t)w, (uint32_t)x1, (q & 1) ? 0x03070105u : 0x06020400u);
}

// Test output of a 16-row fragment's SwiGLU (swiglu_frag): lane l holds rows row0 + 4 (l / 16)
// + i of columns col0 + 16 jj + l % 16.
template <bool TAP>
__device__ __forceinline__ void tap_frag(float* htap, int I, int rowbase, int row0, int nvalid, int col0,
                                         const float (&h)[2][4]) {
    if constexpr (TAP) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tap_h<true>(htap, I, rowbase, row0 + 4 * (lane >> 4) + i, nvalid, col0 + 16 * jj + (lane & 15), h[jj][i]);
    }
}

// One thread per row r < nrows: the row's E4M3 scale exponent (from the four column waves'
// maxima) as the biased byte, in row order (s_ex) and in the order of the hs blocks,
// [tile of the item][row % 16][row / 16] (s_exT), which a few 16-byte stores then copy out.
__device__ __forceinline__ void row_exponents(const float (*s_amax)[4], uint8_t* s_ex, uint8_t* s_exT, int nrows) {
    const int r = threadIdx.x;
    if (r < nrows) {
        const float4 am4 = *reinterpret_cast<const float4*>(s_amax[r]);
        const uint8_t b = (uint8_t)(scale_exponent(fmaxf(fmaxf(am4.x, am4.y), fmaxf(am4.z, am4.w))) + 127);
        s_ex[r] = b;
        s_exT[(r >> 7) * 128 + (r & 15) * 8 + ((r >> 4) & 7)] = b;
    }
}

// The exponents of rows row0 .. row0 + 3 (row0 % 4 == 0) from s_ex.
__device__ __forceinline__ void load_exponents4(const uint8_t* s_ex, int row0, int (&ex)[4]) {
    const uint32_t b4 = *reinterpret_cast<const uint32_t*>(s_ex + row0);
#pragma unroll
    for (int i = 0; i < 4; ++i) ex[i] = (int)((b4 >> (8 * i)) & 0xFFu) - 127;
}

// A rows in LDS (k_gemm1_pf, k_gemm1_pp, k_gemm1_p2): a 128-byte line per row, its 16-byte
// K chunks in slot order P = 0 2 4 6 1 3 5 7 (chunk c at slot c / 2 for even c, 4 + c / 2 for
// odd c), then XOR-swizzled by row % 8.  A lane of group G = lane / 16 needs K chunks 2 G and
// 2 G + 1 (the weights' packing), which sit at slots G and G + 4: with that placement the 16
// lanes that the LDS serves together read distinct banks, where slots 2 G and 2 G + 1 left
// two-way conflicts (the slot order of the MX kernels, whose operands use this K order
// natively, measured conflict-free; a compute probe of the fragment reads ran 5% faster).
__device__ __forceinline__ int a_chunk_of_slot(int s) { return s < 4 ? 2 * s : 2 * s - 7; }
__device__ __forceinline__ int a_slot_lo(int lane) { return lane >> 4; }

template <bool TAP>
__global__ __launch_bounds__(512, 1) void k_gemm1_pf(G1Args a) {
    int ib, tile;
    if (!pf_work_item(a.ord, a.I / kGroup, __builtin_amdgcn_readfirstlane(*a.ntiles), tile, ib)) return;
    const int2 te = a.tiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = __builtin_amdgcn_readfirstlane(a.offsets[e] + m0);
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[kPfdStages * kPfStage];
    __shared__ __align__(16) uint8_t s_sa[kPfMaxKB * kPfBM];   // [kb][wm][row % 16][fragment of wm]
    __shared__ uint16_t s_sgu[kPfMaxKB];                      // gate scale | up scale << 8
    __shared__ __align__(16) float s_amax[kPfBM][4];   // [row][column wave]
    __shared__ __align__(16) uint8_t s_ex[kPfBM], s_exT[kPfBM];

    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const v4i_t ra = make_srd(a.xq, (uint32_t)a.T * a.H);
    const v4i_t rw = make_srd(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    // A pieces: wave instruction i moves rows 8 (wv + 8 i) .. +7, whole 128-byte lines; lane l
    // brings 16-byte chunk (l % 8) ^ (l / 8) of row 8 (wv + 8 i) + l / 8 to slot l % 8 of
    // that row in LDS, i.e. chunk c of row r sits at r * 128 + 16 (c ^ (r % 8)).
    const int rs = tid >> 2;   // the row whose A scales this thread stages
    int tok[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int r = i < 2 ? 8 * (wv + 8 * i) + (lane >> 3) : rs;
        tok[i] = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
    }
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i] = (uint32_t)tok[i] * a.H + (a_chunk_of_slot((lane & 7) ^ (lane >> 3)) << 4);
    uint32_t bsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = wv * 64 + 512 * i, f = q >> 7, hh = (q >> 6) & 1;
        const int n16 = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
        bsoff[i] = __builtin_amdgcn_readfirstlane(n16 * KB * kFragBytes + hh * 1024);
    }
    const uint32_t l16 = lane * 16;
    const uint32_t lds_w = lds_addr(buf) + wv * 64 * 16;   // this wave's 1 KB piece row of stage 0
    auto issue = [&](int kb, int s) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * kPfStage);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(ra, st + i * 512 * 16, aoff[i], kb * kGroup);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(rw, st + kPfStageA + i * 512 * 16, l16, bsoff[i] + kb * kFragBytes);
    };
    // Scales are loaded before the first DMAs are issued and stored after: the wait for them
    // then also covers those DMAs, which the first K block needs anyway.  Thread tid stages
    // the scales of row tid / 4 for K blocks tid % 4 + 4 t.
    uint32_t sv[kPfMaxKB / 4];
    {
        const uint8_t* src = a.xs + (int64_t)tok[2] * KB;
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 4; ++t) {
            const int kb = (tid & 3) + 4 * t;
            sv[t] = kb < KB ? src[kb] : 0u;
        }
    }
    uint32_t sgu = 0;
    if (tid < KB) {
        const uint8_t* sb = a.w13s + ((int64_t)e * KB + tid) * NBS;
        sgu = (uint32_t)sb[ib] | (uint32_t)sb[a.I / kGroup + ib] << 8;
    }
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);
    {
        const int sa_pos = (rs >> 6) * 64 + (rs & 15) * 4 + ((rs >> 4) & 3);
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 4; ++t) {
            const int kb = (tid & 3) + 4 * t;
            if (kb < KB) s_sa[kb * kPfBM + sa_pos] = (uint8_t)sv[t];
        }
        if (tid < KB) s_sgu[tid] = (uint16_t)sgu;
    }

    v4f acc[4][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Fragments of one K block in registers: read from LDS one step before the MFMAs use
    // them, so the reads of block kb+1 overlap the matrix-core work on block kb.
    // F.sa byte mi: the scale of row 16 (4 wm + mi) + lane % 16; F.sgu byte 0 gate, byte 1 up.
    struct Frags {
        v8i a[4], b[4];
        int sa, sgu;
    };
    const int r16 = lane & 15, x8 = r16 & 7;
    // row fragments of this wave holding valid rows (the rest are skipped: wave-uniform)
    const int nact = __builtin_amdgcn_readfirstlane(min(4, max(0, (nvalid - wm * 64 + 15) >> 4)));
    auto read = [&](int kb, int st, Frags& F) {
        const uint8_t* cur = buf + st * kPfStage;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            // row 16 mf + r16, K chunks 2 (lane / 16) and 2 (lane / 16) + 1 of the swizzled rows
            const uint8_t* rowp = cur + ((wm * 4 + mi) * 16 + r16) * kGroup;
            const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((a_slot_lo(lane) ^ x8) << 4));
            const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((a_slot_lo(lane) + 4) ^ x8) << 4));
            F.a[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        F.sa = *reinterpret_cast<const int*>(s_sa + kb * kPfBM + wm * 64 + r16 * 4);
        F.sgu = s_sgu[kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) F.b[j] = lds_frag(cur + kPfStageA + (j < 2 ? 2 * wn + j : 6 + 2 * wn + j) * kFragBytes, lane);
    };
    // step kb (stage st holds block kb, whose fragments F already hold or are receiving):
    // wait until block kb+1 has landed everywhere (the barrier also finds every wave done
    // reading stage st), refill stage st with block kb+3, read block kb+1 into G, then the
    // 16 MFMAs of block kb.
    auto step = [&](int kb, int st, Frags& F, Frags& G) __attribute__((always_inline)) {
        if (kb + 2 < KB) wait_vm<6>(); else wait_vm<0>();
        __syncthreads();
        if (kb + 3 < KB) issue(kb + 3, st);
        if (kb + 1 < KB) read(kb + 1, st == 2 ? 0 : st + 1, G);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                if (mi < nact) acc[mi][j] = mfma_fp8_sel(mi, j >> 1, F.a[mi], F.b[j], acc[mi][j], F.sa, F.sgu);
    };
    if (KB > 2) wait_vm<12>(); else if (KB > 1) wait_vm<6>(); else wait_vm<0>();
    __syncthreads();
    Frags F0, F1;
    read(0, 0, F0);
    int st = 0;
    for (int kb = 0; kb < KB; kb += 2) {
        step(kb, st, F0, F1);
        st = st == 2 ? 0 : st + 1;
        if (kb + 1 < KB) {
            step(kb + 1, st, F1, F0);
            st = st == 2 ? 0 : st + 1;
        }
    }

    // SwiGLU and per-row amax over the tile's 128 h columns (4 waves x 2 fragments)
    GuBias bias[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) bias[jj] = gu_bias(a.b13, e, a.I, ib * 128 + (2 * wn + jj) * 16 + r16);
    float hv[4][2][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < nact) {
            float m[4];
            swiglu_frag(acc[mi], a.b13, bias, hv[mi], m);
            tap_frag<TAP>(a.htap, a.I, rowbase, (wm * 4 + mi) * 16, nvalid, ib * 128 + 2 * wn * 16, hv[mi]);
            if (r16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s_amax[(wm * 4 + mi) * 16 + 4 * (lane >> 4) + i][wn] = m[i];
            }
        }
    }
    __syncthreads();   // also: every wave is done reading the stages before buf is reused
    row_exponents(s_amax, s_ex, s_exT, kPfBM);
    __syncthreads();
    // E4M3 requantisation; h staged as [128 rows][128] bytes, 16-byte chunks XOR-swizzled by
    // row % 8, one dword (4 columns of one row) per lane and fragment
    uint8_t* s_h = buf;
    const int q = lane & 3, g4 = 4 * (lane >> 4);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < nact) {
            int ex[4];
            load_exponents4(s_ex, (wm * 4 + mi) * 16 + g4, ex);
            const int row = (wm * 4 + mi) * 16 + g4 + q;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<uint32_t*>(s_h + row * 128 + (((2 * wn + jj) ^ (row & 7)) << 4) + 4 * (r16 >> 2)) =
                    e4m3_quad_rows(hv[mi][jj], ex, q);
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup;
    for (int q = tid; q < 8 * 128; q += 512) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const int R = mf * 16 + (ln & 15);
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + R * 128 + (((2 * (ln >> 4) + hh) ^ (R & 7)) << 4));
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
    if (tid < 8)   // the tile's hs block for this column block: [row % 16][row / 16]
        *reinterpret_cast<uint4*>(a.hs + ((int64_t)tile * KB2 + ib) * 128 + tid * 16) =
            *reinterpret_cast<const uint4*>(s_exT + tid * 16);
}

// ----------------------------------------------------------------------------------------
// Persistent gate/up GEMM on 128-row tiles (the tile shape, operand layouts and epilogue of
// k_gemm1_pf).  One workgroup per CU walks its item list (tile, I column block) as one
// stream of K blocks through three 48 KB LDS stages (two blocks in flight), so no item starts
// from an empty pipeline:
//   * the sorted assignment ids of item n + 2's rows reach LDS by a dword LDS-DMA issued at
//     item n's first K block;
//   * item n + 1's first two K blocks are issued at item n's last two blocks;
//   * its A row scales (gathered through those ids) and gate/up weight scales are loaded at the
//     start of item n's epilogue and stored to the other half of a double table at its end.
// Waits: before computing block g, every vector-memory op older than block g + 1's DMA must be
// done (vmcnt <= 6: that DMA is 6 ops per thread), so the ids DMA is issued before a step's
// block DMA.  The compiler does not see the DMAs, so its own wait for a load it issued also
// waits for every DMA issued before: the loads it sees (the scales) are issued and used within
// the epilogue only.  Needs 2 <= KB <= 32 and KB <= 4 SVN.
constexpr int kPpMaxItems = 128, kPpMaxKB = 32, kPpStages = 3;

// 4 bytes per lane from the buffer at voff + soff into LDS at m0base + 4 * lane.
__device__ __forceinline__ void dma4_async(const v4i_t& srd, uint32_t m0base, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(m0base), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

template <int SVN, bool TAP>   // scale bytes a thread stages per item: KB <= 4 SVN
__global__ __launch_bounds__(512, 1) void k_gemm1_pp(G1Args a) {
    __shared__ __align__(16) uint8_t buf[kPpStages * kPfStage];
    __shared__ __align__(16) uint8_t s_sa[2][kPpMaxKB * kPfBM];   // [item parity][kb][wm][row % 16][fragment of wm]
    __shared__ uint16_t s_sgu[2][kPpMaxKB + 1];                  // gate scale | up scale << 8 (+ a dummy slot)
    __shared__ __align__(16) int s_tok[2][kPfBM];                // sorted assignment ids of the item's rows
    __shared__ __align__(16) float s_amax[kPfBM][4];
    __shared__ __align__(16) uint8_t s_ex[kPfBM], s_exT[kPfBM];
    __shared__ int4 s_it[kPpMaxItems];                           // tile, column block, expert, first sorted row
    __shared__ int s_nv[kPpMaxItems];
    __shared__ int s_cnt[kItWaves];

    const int ncol = a.I / kGroup, KB = a.H / kGroup;
    // (uniform: the loops below run on scalar counters)
    const int cnt = __builtin_amdgcn_readfirstlane(it_fill_items<1>(
        a.ord, ncol, __builtin_amdgcn_readfirstlane(*a.ntiles), a.tiles, a.counts, a.offsets, s_it, s_nv, kPpMaxItems, s_cnt));
    if (cnt <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;
    const int r16 = lane & 15, x8 = r16 & 7;
    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const v4i_t ra = make_srd(a.xq, (uint32_t)a.T * a.H);
    const v4i_t rtok = make_srd(a.sorted_assign, (uint32_t)a.T * a.k * 4);
    const uint32_t lds_w = lds_addr(buf) + wv * 1024, l16 = lane * 16;
    const int rs = tid >> 2;   // the row whose A scales this thread stages

    // ---- per-item helpers (n: item index; all reads of the item table are uniform)
    auto tok_dma = [&](int n) __attribute__((always_inline)) {   // ids of item n's 128 rows
        if (wv < 2) {
            const int rowbase = __builtin_amdgcn_readfirstlane(s_it[n].w);
            dma4_async(rtok, __builtin_amdgcn_readfirstlane(lds_addr(s_tok[n & 1]) + wv * 256), lane * 4,
                       (uint32_t)(rowbase + wv * 64) * 4);
        }
    };
    // Every thread loads and stores on every path (sources clamped into range; the bytes of
    // blocks kb >= KB land in table slots no one reads, kb < 4 SVN <= kPpMaxKB, and the gate/up
    // scales of threads tid >= KB in a dummy slot): a load that one path skipped, or left
    // unused, would make the compiler wait for it at the next write of its register, which
    // falls inside the next item's DMA stream (see the epilogue).
    uint32_t sv[SVN], sgu_g, sgu_u;   // combined only where stored (see below)
    auto scale_loads = [&](int n) __attribute__((always_inline)) {
        const int4 it = s_it[n];
        const int ib = __builtin_amdgcn_readfirstlane(it.y), e = __builtin_amdgcn_readfirstlane(it.z);
        const int nv = __builtin_amdgcn_readfirstlane(s_nv[n]);
        const uint8_t* src = a.xs + (int64_t)(s_tok[n & 1][min(rs, nv - 1)] / a.k) * KB;
#pragma unroll
        for (int t = 0; t < SVN; ++t) sv[t] = src[min((tid & 3) + 4 * t, KB - 1)];
        const uint8_t* sb = a.w13s + ((int64_t)e * KB + min(tid, KB - 1)) * NBS;
        sgu_g = sb[ib];
        sgu_u = sb[ncol + ib];
    };
    auto scale_stores = [&](int n) __attribute__((always_inline)) {
        const int sa_pos = (rs >> 6) * 64 + (rs & 15) * 4 + ((rs >> 4) & 3);
#pragma unroll
        for (int t = 0; t < SVN; ++t) s_sa[n & 1][((tid & 3) + 4 * t) * kPfBM + sa_pos] = (uint8_t)sv[t];
        s_sgu[n & 1][min(tid, kPpMaxKB)] = (uint16_t)(sgu_g | sgu_u << 8);
    };
    // DMA stream state: the item whose blocks are being issued
    uint32_t aoff[2], bsoff[4];
    v4i_t rw;
    auto dma_item = [&](int n) __attribute__((always_inline)) {
        const int4 it = s_it[n];
        const int ib = __builtin_amdgcn_readfirstlane(it.y), e = __builtin_amdgcn_readfirstlane(it.z);
        const int nv = __builtin_amdgcn_readfirstlane(s_nv[n]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {   // rows 8 (wv + 8 i) + lane / 8, whole lines, swizzled chunks
            const int r = 8 * (wv + 8 * i) + (lane >> 3);
            aoff[i] = (uint32_t)(s_tok[n & 1][min(r, nv - 1)] / a.k) * a.H + (a_chunk_of_slot((lane & 7) ^ (lane >> 3)) << 4);
        }
        rw = make_srd(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = wv * 64 + 512 * i, f = q >> 7, hh = (q >> 6) & 1;
            const int n16 = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
            bsoff[i] = __builtin_amdgcn_readfirstlane(n16 * KB * kFragBytes + hh * 1024);
        }
    };
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * kPfStage);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(ra, st + i * 8192, aoff[i], __builtin_amdgcn_readfirstlane(kb * kGroup));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16_async(rw, st + kPfStageA + i * 8192, l16, __builtin_amdgcn_readfirstlane(bsoff[i] + kb * kFragBytes));
    };

    // ---- first item: ids (and the second item's), scales, first two blocks
    tok_dma(0);
    if (cnt > 1) tok_dma(1);
    wait_vm<0>();
    __syncthreads();
    scale_loads(0);
    const int G = cnt * KB;   // K blocks of the whole stream
    dma_item(0);
    issue(0, 0);
    int dn = 0, dkb = 1;      // the next block to issue: item dn, K block dkb
    if (1 < G) {
        if (dkb == KB) {
            dn = 1;
            dkb = 0;
            dma_item(1);
        }
        issue(dkb, 1);
    }
    scale_stores(0);

    v4f acc[4][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    int g = 0, sg3 = 0;   // global K-block step and its stage (g % 3)
    for (int n = 0; n < cnt; ++n) {
        const int4 it = s_it[n];
        const int tile = __builtin_amdgcn_readfirstlane(it.x), ib = __builtin_amdgcn_readfirstlane(it.y);
        const int nvalid = __builtin_amdgcn_readfirstlane(s_nv[n]);
        const int nact = min(4, max(0, (nvalid - wm * 64 + 15) >> 4));
        const bool more = n + 1 < cnt;
        for (int kb = 0; kb < KB; ++kb, ++g) {
            if (g + 1 < G) wait_vm<6>();   // block g landed (block g + 1's 6 DMAs may be in flight) ...
            else wait_vm<0>();
            __syncthreads();               // ... everywhere; every wave is done with block g - 1's stage
            // the ids DMA goes before this step's block DMA (see the waits above)
            if (kb == 0 && n + 2 < cnt) tok_dma(n + 2);
            if (g + 2 < G) {   // block g + 2 into the stage of block g - 1
                if (++dkb == KB) {
                    dkb = 0;
                    dma_item(++dn);
                }
                issue(dkb, sg3 == 0 ? 2 : sg3 - 1);
            }

            const uint8_t* cur = buf + sg3 * kPfStage;
            sg3 = sg3 == 2 ? 0 : sg3 + 1;
            const int sa = *reinterpret_cast<const int*>(s_sa[n & 1] + kb * kPfBM + wm * 64 + r16 * 4);
            const int sg = s_sgu[n & 1][kb];
            v8i bf[4], af[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = lds_frag(cur + kPfStageA + (j < 2 ? 2 * wn + j : 6 + 2 * wn + j) * kFragBytes, lane);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const uint8_t* rowp = cur + ((wm * 4 + mi) * 16 + r16) * kGroup;
                const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((a_slot_lo(lane) ^ x8) << 4));
                const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((a_slot_lo(lane) + 4) ^ x8) << 4));
                af[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                if (mi < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[mi][j] = mfma_fp8_sel(mi, j >> 1, af[mi], bf[j], acc[mi][j], sa, sg);
                }
        }

        // ---- epilogue of item n (the next item's first blocks are in flight in the other stages)
        // The compiler does not see the DMAs, so its wait for any load it issued (vmcnt counts
        // in issue order) also waits for every DMA issued before; such waits must come only
        // after those blocks have landed, late in the epilogue.  Hence: the next item's
        // scales are loaded here and stored at the end (after the last item the current
        // item's are reloaded into its own table, so that no load is left unused on any path
        // through the loop), and the bias loads and their SwiGLU form a branch of their own,
        // so that without biases no load is pending at the SwiGLU's register writes.
        const int sn = more ? n + 1 : n;
        scale_loads(sn);
        float hv[4][2][4];
        auto swiglu_all = [&](auto HASB) __attribute__((always_inline)) {
            GuBias bias[2] = {};
            if constexpr (decltype(HASB)::value) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) bias[jj] = gu_bias(a.b13, it.z, a.I, ib * 128 + (2 * wn + jj) * 16 + r16);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if (mi < nact) {
                    float m[4];
                    swiglu_frag_b<decltype(HASB)::value>(acc[mi], bias, hv[mi], m);
                    tap_frag<TAP>(a.htap, a.I, it.w, (wm * 4 + mi) * 16, nvalid, ib * 128 + 2 * wn * 16, hv[mi]);
                    if (r16 == 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) s_amax[(wm * 4 + mi) * 16 + 4 * (lane >> 4) + i][wn] = m[i];
                    }
                }
            }
        };
        if (a.b13) swiglu_all(std::true_type{});
        else swiglu_all(std::false_type{});
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};
        __syncthreads();   // also: every wave is done reading the stage of block g - 1
        row_exponents(s_amax, s_ex, s_exT, kPfBM);
        __syncthreads();
        // h staged in the stage of the item's last block (the next two blocks are in the others)
        uint8_t* s_h = buf + (sg3 == 0 ? 2 : sg3 - 1) * kPfStage;   // [128 rows][128], chunks swizzled by row % 8
        const int q = lane & 3, g4 = 4 * (lane >> 4);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi < nact) {
                int ex[4];
                load_exponents4(s_ex, (wm * 4 + mi) * 16 + g4, ex);
                const int row = (wm * 4 + mi) * 16 + g4 + q;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    *reinterpret_cast<uint32_t*>(s_h + row * 128 + (((2 * wn + jj) ^ (row & 7)) << 4) + 4 * (r16 >> 2)) =
                        e4m3_quad_rows(hv[mi][jj], ex, q);
            }
        }
        __syncthreads();
        for (int qq = tid; qq < 8 * 128; qq += 512) {
            const int mf = qq >> 7, w = qq & 127, hh = w >> 6, ln = w & 63;
            const int R = mf * 16 + (ln & 15);
            const uint4 v = *reinterpret_cast<const uint4*>(s_h + R * 128 + (((2 * (ln >> 4) + hh) ^ (R & 7)) << 4));
            *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * ncol + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
        }
        if (tid < 8)   // the tile's hs block for this column block: [row % 16][row / 16]
            *reinterpret_cast<uint4*>(a.hs + ((int64_t)tile * ncol + ib) * 128 + tid * 16) =
                *reinterpret_cast<const uint4*>(s_exT + tid * 16);
        scale_stores(sn);   // read after the next item's first barrier
    }
    wait_vm<0>();
}

__global__ __launch_bounds__(512, 1) void k_gemm2_pf(G2Args a) {
    int nb, tile;
    if (!pf_work_item(a.ord, a.H / 256, __builtin_amdgcn_readfirstlane(*a.ntiles), tile, nb)) return;
    const int2 te = a.tiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = __builtin_amdgcn_readfirstlane(a.offsets[e] + m0);
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[kPfdStages * kPfStage];
    __shared__ __align__(16) uint8_t s_sa[kPfMaxKB * kPfBM];   // [kb][row]
    __shared__ uint8_t s_sb[2][kPfMaxKB];

    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const v4i_t ra = make_srd(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const v4i_t rw = make_srd(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint32_t l16 = lane * 16;
    uint32_t asoff[2], bsoff[4];
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
    const uint32_t lds_w = lds_addr(buf) + wv * 64 * 16;
    auto issue = [&](int kb, int s) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * kPfStage);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(ra, st + i * 512 * 16, l16, asoff[i] + kb * kFragBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(rw, st + kPfStageA + i * 512 * 16, l16, bsoff[i] + kb * kFragBytes);
    };
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);
    {
        const uint8_t* src = a.hs + (int64_t)tile * kPfBM * KB;   // [kb][row % 16][row / 16]
        for (int i = tid; i < kPfBM * KB; i += 512) {
            const int kb = i >> 7, w = i & 127;
            s_sa[kb * kPfBM + (w & 7) * 16 + (w >> 3)] = src[i];
        }
        const uint8_t* sb = a.w2s + (int64_t)e * KB * NBS;
        for (int i = tid; i < 2 * KB; i += 512) s_sb[i & 1][i >> 1] = sb[(i >> 1) * NBS + nb * 2 + (i & 1)];
    }


    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Frags {
        v8i a[4], b[4];
        int sa[4], sb;
    };
    auto read = [&](int kb, int st, Frags& F) {
        const uint8_t* cur = buf + st * kPfStage;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            F.a[mi] = lds_frag(cur + mf * kFragBytes, lane);
            F.sa[mi] = s_sa[kb * kPfBM + mf * 16 + (lane & 15)];
        }
        F.sb = s_sb[wn >> 1][kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) F.b[j] = lds_frag(cur + kPfStageA + (wn * 4 + j) * kFragBytes, lane);
    };
    auto step = [&](int kb, int st, Frags& F, Frags& G) {
        if (kb + 2 < KB) wait_vm<6>(); else wait_vm<0>();
        __syncthreads();
        if (kb + 3 < KB) issue(kb + 3, st);
        if (kb + 1 < KB) read(kb + 1, st == 2 ? 0 : st + 1, G);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mfma_fp8(F.a[mi], F.b[j], acc[mi][j], F.sa[mi], F.sb);
    };
    if (KB > 2) wait_vm<12>(); else if (KB > 1) wait_vm<6>(); else wait_vm<0>();
    __syncthreads();
    Frags F0, F1;
    read(0, 0, F0);
    int st = 0;
    for (int kb = 0; kb < KB; kb += 2) {
        step(kb, st, F0, F1);
        st = st == 2 ? 0 : st + 1;
        if (kb + 1 < KB) {
            step(kb + 1, st, F1, F0);
            st = st == 2 ? 0 : st + 1;
        }
    }

    float bias[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bias[j] = out_bias(a.b2, e, a.H, nb * 256 + (wn * 4 + j) * 16 + (lane & 15));
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
                    const float v = add_bias(a.b2, acc[mi][j][i], bias[j]);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(v);
                    else reinterpret_cast<float*>(a.out)[o + col] = v;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Micro-scaled gate/up and down GEMMs on 128-row tiles (MXFP8: E4M3 weights; W4A8: E2M1
// weights): the tile shape, work order and three-stage LDS ring of k_gemm1_pf / k_gemm2_pf
// with one UE8M0 scale per 32 elements.  Per K block a stage holds the A operand (128 rows of
// 128 bytes), the 16 weight fragments (2 KB E4M3 or 1 KB E2M1, packed as for the 16-row MX
// kernels), the A rows' four scale bytes (one dword per row) and the fragments' 64 per-lane
// scale bytes; the scales ride LDS-DMA copies beside the operands, so one wait covers a
// block.  Every E4M3 operand is in the matrix instruction's K order (lane group G = lane / 16
// holds K 16 G .. +15 and 64 + 16 G .. +15 of its row), so each lane's scale byte covers one
// 32-element group: the activation fragment reads take 16-byte chunks G and G + 4 of the
// swizzled row, the re-quantised h is stored for the down GEMM in that order, and its scales
// as [tile row][I / 32].
template <int WF>
struct MxPf {
    static constexpr int FB = WF == kWfmtE2M1 ? 1024 : 2048;   // bytes per weight fragment
    static constexpr int NBI = 16 * FB / 8192;                 // weight copies per thread and block
    static constexpr int SA = kPfStageA + 16 * FB;             // A-row scales: one dword per row
    static constexpr int SB = SA + kPfBM * 4;                  // weight scales: [fragment][lane]
    static constexpr int Stage = SB + 16 * 64;
    static constexpr int Ops = 2 + NBI + 1;                    // copies per thread and block
};

// The stage's weight fragment f as an operand (E2M1: the lane's 16 bytes, upper half unused).
template <int WF>
__device__ __forceinline__ v8i mx_lds_wfrag(const uint8_t* stage, int f, int lane) {
    if constexpr (WF == kWfmtE2M1) {
        const uint4 v = *reinterpret_cast<const uint4*>(stage + kPfStageA + f * 1024 + lane * 16);
        return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    } else {
        return lds_frag(stage + kPfStageA + f * 2048, lane);
    }
}

// Scale byte of lane group G from a stage's A-row scale dword of row `row`.
template <int WF>
__device__ __forceinline__ int mx_lds_ascale(const uint8_t* stage, int row, int G) {
    return (int)((*reinterpret_cast<const uint32_t*>(stage + MxPf<WF>::SA + row * 4) >> (8 * G)) & 0xFFu);
}

template <int WF, bool TAP>
__global__ __launch_bounds__(512, 1) void k_gemm1_mxpf(G1Args a) {
    using C = MxPf<WF>;
    int ib, tile;
    if (!pf_work_item(a.ord, a.I / kGroup, __builtin_amdgcn_readfirstlane(*a.ntiles), tile, ib)) return;
    const int2 te = a.tiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = __builtin_amdgcn_readfirstlane(a.offsets[e] + m0);
    const int KB = a.H / kGroup, KS = a.H / kMx;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[kPfdStages * C::Stage];

    const int NB16 = 2 * a.I / 16;
    const v4i_t ra = make_srd(a.xq, (uint32_t)a.T * a.H);
    const v4i_t rw = make_srd(a.w13p + (int64_t)e * NB16 * KB * C::FB, (uint32_t)NB16 * KB * C::FB);
    const v4i_t rxs = make_srd(a.xs, (uint32_t)a.T * KS);
    const v4i_t rws = make_srd(a.w13s + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    auto n16_of = [&](int f) { return f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8); };
    // A pieces as in k_gemm1_pf: rows 8 (wv + 8 i) + lane / 8, whole lines, chunk c of row r at
    // r * 128 + 16 (c ^ (r % 8)).  Scale copies, one dword per lane: waves 0, 1 (and, as
    // duplicates of the same bytes, 6, 7) bring row (wv % 2) * 64 + lane's four A scales of the
    // block; waves 2..5 bring the 16 fragments' per-lane weight scales.
    const bool sc_a = wv < 2 || wv >= 6;
    const int sr = (wv & 1) * 64 + lane;
    int tok[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int r = i < 2 ? 8 * (wv + 8 * i) + (lane >> 3) : sr;
        tok[i] = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
    }
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i] = (uint32_t)tok[i] * a.H + (((lane & 7) ^ (lane >> 3)) << 4);
    uint32_t bsoff[C::NBI];
#pragma unroll
    for (int i = 0; i < C::NBI; ++i) {
        const int b = (wv * 64 + 512 * i) * 16;   // this wave's byte of the stage's fragments
        bsoff[i] = __builtin_amdgcn_readfirstlane(n16_of(b / C::FB) * KB * C::FB + b % C::FB);
    }
    uint32_t scoff;
    if (sc_a) {
        scoff = (uint32_t)tok[2] * KS;
    } else {
        const int t = (wv - 2) * 64 + lane;
        scoff = (uint32_t)n16_of(t >> 4) * KB * 64 + (t & 15) * 4;
    }
    const uint32_t l16 = lane * 16;
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    const uint32_t lds_s = lds_addr(buf) + (sc_a ? C::SA + (wv & 1) * 256 : C::SB + (wv - 2) * 256);
    auto issue = [&](int kb, int s) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * C::Stage);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(ra, st + i * 8192, aoff[i], kb * kGroup);
#pragma unroll
        for (int i = 0; i < C::NBI; ++i) dma16_async(rw, st + kPfStageA + i * 8192, l16, bsoff[i] + kb * C::FB);
        const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_s + s * C::Stage);
        if (sc_a) dma4_async(rxs, ss, scoff, kb * 4);
        else dma4_async(rws, ss, scoff, kb * 64);
    };
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);

    v4f acc[4][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Frags {
        v8i a[4], b[4];
        int sa[4], sb[4];
    };
    const int r16 = lane & 15, x8 = r16 & 7, G = lane >> 4;
    const int nact = __builtin_amdgcn_readfirstlane(min(4, max(0, (nvalid - wm * 64 + 15) >> 4)));
    auto read = [&](int st, Frags& F) {
        const uint8_t* cur = buf + st * C::Stage;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int row = (wm * 4 + mi) * 16 + r16;
            const uint8_t* rowp = cur + row * kGroup;
            const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((G ^ x8) << 4));
            const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((G + 4) ^ x8) << 4));
            F.a[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            F.sa[mi] = mx_lds_ascale<WF>(cur, row, G);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = j < 2 ? 2 * wn + j : 6 + 2 * wn + j;
            F.b[j] = mx_lds_wfrag<WF>(cur, f, lane);
            F.sb[j] = cur[C::SB + f * 64 + lane];
        }
    };
    // as k_gemm1_pf: wait for block kb + 1 everywhere, refill stage st with block kb + 3, read
    // block kb + 1, then block kb's 16 instructions
    auto step = [&](int kb, int st, Frags& F, Frags& N) __attribute__((always_inline)) {
        if (kb + 2 < KB) wait_vm<C::Ops>();
        else wait_vm<0>();
        __syncthreads();
        if (kb + 3 < KB) issue(kb + 3, st);
        if (kb + 1 < KB) read(st == 2 ? 0 : st + 1, N);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                if (mi < nact) acc[mi][j] = mx_mfma<WF>(F.a[mi], F.b[j], acc[mi][j], F.sa[mi], F.sb[j]);
    };
    if (KB > 2) wait_vm<2 * C::Ops>();
    else if (KB > 1) wait_vm<C::Ops>();
    else wait_vm<0>();
    __syncthreads();
    Frags F0, F1;
    read(0, F0);
    int st = 0;
    for (int kb = 0; kb < KB; kb += 2) {
        step(kb, st, F0, F1);
        st = st == 2 ? 0 : st + 1;
        if (kb + 1 < KB) {
            step(kb + 1, st, F1, F0);
            st = st == 2 ? 0 : st + 1;
        }
    }

    // SwiGLU; a wave's two fragments are the 32 h columns 32 wn .. of the block, one MX group,
    // so each row's amax is the swiglu_frag maximum and the scale needs no other wave
    GuBias bias[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) bias[jj] = gu_bias(a.b13, e, a.I, ib * 128 + (2 * wn + jj) * 16 + r16);
    float hv[4][2][4];
    int ex[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < nact) {
            float m[4];
            swiglu_frag(acc[mi], a.b13, bias, hv[mi], m);
            tap_frag<TAP>(a.htap, a.I, rowbase, (wm * 4 + mi) * 16, nvalid, ib * 128 + 2 * wn * 16, hv[mi]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ex[mi][i] = mx_scale_exponent<kWfmtE4M3>(m[i]);
        }
    }
    __syncthreads();   // every wave is done reading the stages before buf is reused
    // E4M3 bytes staged as [128 rows][128] (16-byte chunks XOR-swizzled by row % 8), one dword
    // (4 columns of one row) per lane and fragment; the scales straight to hs
    uint8_t* s_h = buf;
    const int q = lane & 3, g4 = 4 * (lane >> 4), KS2 = a.I / kMx;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < nact) {
            const int row = (wm * 4 + mi) * 16 + g4 + q;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<uint32_t*>(s_h + row * 128 + (((2 * wn + jj) ^ (row & 7)) << 4) + 4 * (r16 >> 2)) =
                    e4m3_quad_rows(hv[mi][jj], ex[mi], q);
            if (r16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.hs[((int64_t)tile * kPfBM + (wm * 4 + mi) * 16 + g4 + i) * KS2 + ib * 4 + wn] =
                        (uint8_t)(ex[mi][i] + 127);
            }
        }
    }
    __syncthreads();
    // out in the down GEMM's operand order: fragment (row fragment mf, half hh), lane ln holds
    // row mf * 16 + ln % 16, columns 64 hh + 16 (ln / 16) .. +15 (chunk 4 hh + ln / 16)
    const int KB2 = a.I / kGroup;
    for (int q2 = tid; q2 < 8 * 128; q2 += 512) {
        const int mf = q2 >> 7, w = q2 & 127, hh = w >> 6, ln = w & 63;
        const int R = mf * 16 + (ln & 15), c = 4 * hh + (ln >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + R * 128 + ((c ^ (R & 7)) << 4));
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)tile * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int WF>
__global__ __launch_bounds__(512, 1) void k_gemm2_mxpf(G2Args a) {
    using C = MxPf<WF>;
    int nb, tile;
    if (!pf_work_item(a.ord, a.H / 256, __builtin_amdgcn_readfirstlane(*a.ntiles), tile, nb)) return;
    const int2 te = a.tiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
    const int nvalid = min(kPfBM, a.counts[e] - m0);
    const int rowbase = __builtin_amdgcn_readfirstlane(a.offsets[e] + m0);
    const int KB = a.I / kGroup, KS2 = a.I / kMx;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[kPfdStages * C::Stage];

    const int NB16 = a.H / 16;
    const v4i_t ra = make_srd(a.hq + (int64_t)tile * 8 * KB * kFragBytes, (uint32_t)8 * KB * kFragBytes);
    const v4i_t rw = make_srd(a.w2p + (int64_t)e * NB16 * KB * C::FB, (uint32_t)NB16 * KB * C::FB);
    const v4i_t rhs = make_srd(a.hs + (int64_t)tile * kPfBM * KS2, (uint32_t)kPfBM * KS2);
    const v4i_t rws = make_srd(a.w2s + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    const uint32_t l16 = lane * 16;
    uint32_t asoff[2], bsoff[C::NBI];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = wv * 64 + 512 * i, mf = p >> 7, hh = (p >> 6) & 1;
        asoff[i] = __builtin_amdgcn_readfirstlane(mf * KB * kFragBytes + hh * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::NBI; ++i) {
        const int b = (wv * 64 + 512 * i) * 16;
        bsoff[i] = __builtin_amdgcn_readfirstlane((nb * 16 + b / C::FB) * KB * C::FB + b % C::FB);
    }
    // scale copies as in k_gemm1_mxpf: A-row scales of the tile's hs rows, weight scales of
    // the item's 16 fragments
    const bool sc_a = wv < 2 || wv >= 6;
    uint32_t scoff;
    if (sc_a) {
        scoff = (uint32_t)((wv & 1) * 64 + lane) * KS2;
    } else {
        const int t = (wv - 2) * 64 + lane;
        scoff = (uint32_t)(nb * 16 + (t >> 4)) * KB * 64 + (t & 15) * 4;
    }
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    const uint32_t lds_s = lds_addr(buf) + (sc_a ? C::SA + (wv & 1) * 256 : C::SB + (wv - 2) * 256);
    auto issue = [&](int kb, int s) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * C::Stage);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_async(ra, st + i * 8192, l16, asoff[i] + kb * kFragBytes);
#pragma unroll
        for (int i = 0; i < C::NBI; ++i) dma16_async(rw, st + kPfStageA + i * 8192, l16, bsoff[i] + kb * C::FB);
        const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_s + s * C::Stage);
        if (sc_a) dma4_async(rhs, ss, scoff, kb * 4);
        else dma4_async(rws, ss, scoff, kb * 64);
    };
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Frags {
        v8i a[4], b[4];
        int sa[4], sb[4];
    };
    const int G = lane >> 4, r16 = lane & 15;
    auto read = [&](int st, Frags& F) {
        const uint8_t* cur = buf + st * C::Stage;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int mf = wm * 4 + mi;
            F.a[mi] = lds_frag(cur + mf * kFragBytes, lane);
            F.sa[mi] = mx_lds_ascale<WF>(cur, mf * 16 + r16, G);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            F.b[j] = mx_lds_wfrag<WF>(cur, wn * 4 + j, lane);
            F.sb[j] = cur[C::SB + (wn * 4 + j) * 64 + lane];
        }
    };
    auto step = [&](int kb, int st, Frags& F, Frags& N) __attribute__((always_inline)) {
        if (kb + 2 < KB) wait_vm<C::Ops>();
        else wait_vm<0>();
        __syncthreads();
        if (kb + 3 < KB) issue(kb + 3, st);
        if (kb + 1 < KB) read(st == 2 ? 0 : st + 1, N);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][j] = mx_mfma<WF>(F.a[mi], F.b[j], acc[mi][j], F.sa[mi], F.sb[j]);
    };
    if (KB > 2) wait_vm<2 * C::Ops>();
    else if (KB > 1) wait_vm<C::Ops>();
    else wait_vm<0>();
    __syncthreads();
    Frags F0, F1;
    read(0, F0);
    int st = 0;
    for (int kb = 0; kb < KB; kb += 2) {
        step(kb, st, F0, F1);
        st = st == 2 ? 0 : st + 1;
        if (kb + 1 < KB) {
            step(kb + 1, st, F1, F0);
            st = st == 2 ? 0 : st + 1;
        }
    }

    float bias[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bias[j] = out_bias(a.b2, e, a.H, nb * 256 + (wn * 4 + j) * 16 + r16);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (wm * 4 + mi) * 16 + 4 * (lane >> 4) + i;
            if (row < nvalid) {
                const int64_t o = (int64_t)(rowbase + row) * a.H;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = nb * 256 + (wn * 4 + j) * 16 + r16;
                    const float v = add_bias(a.b2, acc[mi][j][i], bias[j]);
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + col] = f32_to_bf16(v);
                    else reinterpret_cast<float*>(a.out)[o + col] = v;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// 256-row items for experts with many rows: an item is a pair of consecutive 128-row tiles
// of one expert (the second may be absent) and 256 columns, so each K block moves 64 KB
// (A 32 KB + B 32 KB) per 256 x 256 x 128 product instead of 48 KB per 128 x 256 x 128:
// a third fewer bytes from L2 per flop, and the per-item fill and epilogue spread over twice
// the work.  8 waves as 2 (rows) x 4 (columns), each 128 x 64 (8 x 4 fragments, 128
// accumulator registers per lane), two waves per SIMD.  Two 64 KB LDS stages: block kb + 1
// loads while the waves compute block kb.  The tile list and the hq / hs layouts are those
// of the 128-row tiles.
constexpr int kP2Rows = 256, kP2StageA = 16 * kFragBytes, kP2Stage = kP2StageA + 16 * kFragBytes;   // 64 KB

// Pair list: for each expert, one entry per 256-row item (ceil(count / 256) of them) holding
// the index of its first tile (tiles of 128 rows in expert order, as k_tiles writes them),
// the expert, the item's first row in the sorted order and its valid rows, so that a GEMM
// workgroup finds its rows with one load.
__global__ __launch_bounds__(1024) void k_pairs(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                                                int E, int4* __restrict__ pairs, int32_t* __restrict__ npairs) {
    __shared__ int s_t[16], s_p[16];
    const int e = threadIdx.x;
    const int c = e < E ? counts[e] : 0;
    const int nt = (c + kPfBM - 1) / kPfBM, np = (c + kP2Rows - 1) / kP2Rows;
    const int lane = e & 63, wv = e >> 6;
    int vt = nt, vp = np;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int ut = __shfl_up(vt, o), up = __shfl_up(vp, o);
        if (lane >= o) {
            vt += ut;
            vp += up;
        }
    }
    if (lane == 63) {
        s_t[wv] = vt;
        s_p[wv] = vp;
    }
    __syncthreads();
    int at = 0, ap = 0;
    for (int w = 0; w < wv; ++w) {
        at += s_t[w];
        ap += s_p[w];
    }
    const int t0 = vt + at - nt, p0 = vp + ap - np;
    const int off = e < E ? offsets[e] : 0;
    for (int i = 0; i < np; ++i) pairs[p0 + i] = make_int4(t0 + 2 * i, e, off + kP2Rows * i, min(kP2Rows, c - kP2Rows * i));
    if (e == 1023) *npairs = vp + ap;
}

template <bool TAP>
__global__ __launch_bounds__(512, 1) void k_gemm1_p2(G1Args a) {
    int ib, pair;
    if (!pf_work_item(a.ord, a.I / kGroup, __builtin_amdgcn_readfirstlane(*a.npairs), pair, ib)) return;
    const int4 pi = a.pairs[pair];
    const int t0 = __builtin_amdgcn_readfirstlane(pi.x), e = __builtin_amdgcn_readfirstlane(pi.y);
    const int rowbase = __builtin_amdgcn_readfirstlane(pi.z), nvalid = __builtin_amdgcn_readfirstlane(pi.w);
    const bool second = nvalid > kPfBM;
    const int KB = a.H / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2 * kP2Stage];
    __shared__ __align__(16) uint8_t s_sa[kPfMaxKB * kP2Rows];   // [kb][wm][row % 16][fragment of wm]
    __shared__ uint16_t s_sgu[kPfMaxKB];                        // gate scale | up scale << 8
    __shared__ __align__(16) float s_amax[kP2Rows][4];   // [row][column wave]
    __shared__ __align__(16) uint8_t s_ex[kP2Rows], s_exT[kP2Rows];

    const int NB16 = 2 * a.I / 16, NBS = 2 * a.I / kGroup;
    const v4i_t ra = make_srd(a.xq, (uint32_t)a.T * a.H);
    const v4i_t rw = make_srd(a.w13p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    // A: wave instruction i moves rows 8 (wv + 8 i) .. +7 as whole lines into the XOR-swizzled
    // row layout (chunk c of row r at r * 128 + 16 (c ^ (r % 8))), as the 128-row kernel does
    const int rs = tid >> 1;   // the row whose A scales this thread stages (with its neighbour)
    int tok[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int r = i < 4 ? 8 * (wv + 8 * i) + (lane >> 3) : rs;
        tok[i] = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
    }
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)tok[i] * a.H + (a_chunk_of_slot((lane & 7) ^ (lane >> 3)) << 4);
    uint32_t bsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = wv * 64 + 512 * i, f = q >> 7, hh = (q >> 6) & 1;
        const int n16 = f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8);
        bsoff[i] = __builtin_amdgcn_readfirstlane(n16 * KB * kFragBytes + hh * 1024);
    }
    const uint32_t l16 = lane * 16;
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * kP2Stage);
#pragma unroll
        for (int i = 0; i < 4; ++i)   // rows 128.. only for a pair with a second tile (uniform)
            if (i < 2 || second) dma16_async(ra, st + i * 8192, aoff[i], kb * kGroup);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(rw, st + kP2StageA + i * 8192, l16, bsoff[i] + kb * kFragBytes);
    };
    // scales: loaded before the first DMAs, stored after (their wait also covers block 0)
    uint32_t sv[kPfMaxKB / 2];
    {
        const uint8_t* src = a.xs + (int64_t)tok[4] * KB;
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 2; ++t) {
            const int kb = (tid & 1) + 2 * t;
            sv[t] = kb < KB ? src[kb] : 0u;
        }
    }
    uint32_t sgu = 0;
    if (tid < KB) {
        const uint8_t* sb = a.w13s + ((int64_t)e * KB + tid) * NBS;
        sgu = (uint32_t)sb[ib] | (uint32_t)sb[a.I / kGroup + ib] << 8;
    }
    issue(0, 0);
    {
        const int sa_pos = (rs >> 7) * 128 + (rs & 15) * 8 + ((rs >> 4) & 7);
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 2; ++t) {
            const int kb = (tid & 1) + 2 * t;
            if (kb < KB) s_sa[kb * kP2Rows + sa_pos] = (uint8_t)sv[t];
        }
        if (tid < KB) s_sgu[tid] = (uint16_t)sgu;
    }

    v4f acc[8][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15, x8 = r16 & 7;
    // row fragments of this wave holding valid rows (the rest are skipped: wave-uniform)
    const int nact = __builtin_amdgcn_readfirstlane(min(8, max(0, (nvalid - wm * kPfBM + 15) >> 4)));
    auto loop = [&](auto FULL) __attribute__((always_inline)) {
        for (int kb = 0; kb < KB; ++kb) {
            wait_vm<0>();      // block kb landed (this thread's pieces) ...
            __syncthreads();   // ... and everyone's; every wave is done with block kb - 1's stage
            if (kb + 1 < KB) issue(kb + 1, (kb + 1) & 1);
            if (nact > 0) {
                const uint8_t* cur = buf + (kb & 1) * kP2Stage;
                const v2i_t sa = *reinterpret_cast<const v2i_t*>(s_sa + kb * kP2Rows + wm * 128 + r16 * 8);
                const int sg = s_sgu[kb];
                v8i bf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[j] = lds_frag(cur + kP2StageA + (j < 2 ? 2 * wn + j : 6 + 2 * wn + j) * kFragBytes, lane);
                auto afrag = [&](int mi) __attribute__((always_inline)) {
                    const uint8_t* rowp = cur + ((wm * 8 + mi) * 16 + r16) * kGroup;
                    const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((a_slot_lo(lane) ^ x8) << 4));
                    const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((a_slot_lo(lane) + 4) ^ x8) << 4));
                    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                };
                // row fragments in pairs, the next pair's LDS reads in flight during this
                // pair's 8 matrix-core instructions (the scheduling barrier keeps that order)
                v8i a0 = afrag(0), a1 = afrag(1);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    v8i n0 = a0, n1 = a1;
                    if (p < 3) {
                        n0 = afrag(2 * p + 2);
                        n1 = afrag(2 * p + 3);
                    }
                    if (decltype(FULL)::value || 2 * p < nact) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[2 * p][j] = mfma_fp8_sel(2 * p & 3, j >> 1, a0, bf[j], acc[2 * p][j], sa[p >> 1], sg);
                    }
                    if (decltype(FULL)::value || 2 * p + 1 < nact) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[2 * p + 1][j] =
                                mfma_fp8_sel((2 * p + 1) & 3, j >> 1, a1, bf[j], acc[2 * p + 1][j], sa[p >> 1], sg);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    a0 = n0;
                    a1 = n1;
                }
            }
        }
    };
    if (nact == 8) loop(std::true_type{});
    else loop(std::false_type{});

    // SwiGLU, per-row amax over the item's 128 h columns (4 waves x 2 fragments)
    GuBias bias[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) bias[jj] = gu_bias(a.b13, e, a.I, ib * 128 + (2 * wn + jj) * 16 + r16);
    float hv[8][2][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi < nact) {
            float m[4];
            swiglu_frag(acc[mi], a.b13, bias, hv[mi], m);
            tap_frag<TAP>(a.htap, a.I, rowbase, (wm * 8 + mi) * 16, nvalid, ib * 128 + 2 * wn * 16, hv[mi]);
            if (r16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s_amax[(wm * 8 + mi) * 16 + 4 * (lane >> 4) + i][wn] = m[i];
            }
        }
    }
    __syncthreads();   // also: every wave is done reading the stages before buf is reused
    row_exponents(s_amax, s_ex, s_exT, second ? kP2Rows : kPfBM);
    __syncthreads();
    // E4M3 requantisation; h staged as [256 rows][128] bytes, 16-byte chunks XOR-swizzled by
    // row % 8, one dword (4 columns of one row) per lane and fragment
    uint8_t* s_h = buf;
    const int KB2 = a.I / kGroup;
    const int q = lane & 3, g4 = 4 * (lane >> 4);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi < nact) {
            int ex[4];
            load_exponents4(s_ex, (wm * 8 + mi) * 16 + g4, ex);
            const int row = (wm * 8 + mi) * 16 + g4 + q;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<uint32_t*>(s_h + row * 128 + (((2 * wn + jj) ^ (row & 7)) << 4) + 4 * (r16 >> 2)) =
                    e4m3_quad_rows(hv[mi][jj], ex, q);
        }
    }
    __syncthreads();
    const int nf = second ? 16 : 8;
    for (int q = tid; q < nf * 128; q += 512) {
        const int mf = q >> 7, w = q & 127, hh = w >> 6, ln = w & 63;
        const int R = mf * 16 + (ln & 15);
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + R * 128 + (((2 * (ln >> 4) + hh) ^ (R & 7)) << 4));
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)t0 * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
    if (tid < (second ? 16 : 8))   // the pair's hs blocks for this column block: [row % 16][row / 16]
        *reinterpret_cast<uint4*>(a.hs + ((int64_t)(t0 + (tid >> 3)) * KB2 + ib) * 128 + (tid & 7) * 16) =
            *reinterpret_cast<const uint4*>(s_exT + tid * 16);
}

// Two float32 values as packed bf16 (round to nearest even), a in the low half: one
// conversion instruction on gfx950.
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{a, b}, bf16x2_t));
}

// Output of a 256-row down item through an LDS staging buffer of BUF bytes (free after the K
// loop), as whole 16-byte pieces of full rows, in passes of RP rows: bf16 RP = 256 if the
// buffer holds them (512 bytes a row), else 128; float32 RP = 128 or 64 (1 KB a row).  A lane
// holds rows wm * 128 + 16 mi + 4 (lane / 16) + i of columns wn * 64 + 16 j + lane % 16;
// staged rows are swizzled by 16 columns times (row / 4) % 4, which for a lane's rows is
// lane / 16, so the lane's offsets per j are formed once; a row-parity term keeps the two rows a
// lane pair writes together in different banks (odd rows: the 16-column index also XOR 2 for
// bf16, XOR 1 for float32).  The two lanes of a column pair
// swap one value of each row pair, so that the even lane holds rows 0 and 2 and the odd lane
// rows 1 and 3 of both columns; each lane then writes both columns of each of its two rows
// (bf16: one conversion of the pair into a dword; float32: 8 bytes).  The bf16 read-out walks
// 16 rows a step with offsets fixed per thread.  The caller has synchronised the workgroup
// after its last read of the buffer.
template <int BUF>
__device__ __forceinline__ void p2_store_output(const G2Args& a, v4f (&acc)[8][4], uint8_t* buf, int rowbase,
                                                int nvalid, int nb, int nact) {
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3, r16 = lane & 15, r0 = 4 * (lane >> 4), q4 = lane >> 4;
    const int odd = lane & 1;
    if (a.out_bf16) {
        constexpr int RP = BUF >= 256 * 512 ? 256 : 128;
        static_assert(BUF >= RP * 512, "staging buffer too small");
#pragma unroll
        for (int q = 0; q < 256 / RP; ++q) {
            const int nr = min(RP, nvalid - q * RP);
            if (nr <= 0) break;
            if (q) __syncthreads();   // the previous pass has left the LDS
            uint32_t ob[4];           // bytes: row r0 + odd of the pass, swizzled column pair of fragment j
#pragma unroll
            for (int j = 0; j < 4; ++j) ob[j] = (r0 + odd) * 512 + 2 * (wn * 64 + 16 * (j ^ q4 ^ (2 * odd)) + (r16 & 14));
#pragma unroll
            for (int mi = 0; mi < 8; ++mi) {
                const int R0 = wm * kPfBM + mi * 16 - q * RP;   // wave-uniform
                if (mi < nact && R0 >= 0 && R0 < RP) {
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float lo = acc[mi][j][2 * ip], hi = acc[mi][j][2 * ip + 1];
                            const float got = dpp_f32<0xB1>(odd ? lo : hi);   // from lane ^ 1
                            // even lane: row 2 ip, columns (own, neighbour's); odd: row 2 ip + 1
                            const uint32_t v = bf16x2_bits(odd ? got : lo, odd ? hi : got);
                            *reinterpret_cast<uint32_t*>(buf + ob[j] + (R0 + 2 * ip) * 512) = v;
                        }
                }
            }
            __syncthreads();
            // thread t moves 16 bytes (8 columns) of rows t / 32 + 16 s: its LDS swizzle and
            // column stay fixed
            const int m = tid & 31, R1 = tid >> 5;
            const uint8_t* src = buf + (R1 * 256 + ((8 * m) ^ (16 * (((R1 >> 2) & 3) ^ (2 * (R1 & 1)))))) * 2;
            uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) + ((int64_t)(rowbase + q * RP + R1) * a.H + nb * 256 + 8 * m) * 2;
            const int64_t rstep = (int64_t)16 * a.H * 2;
            // non-temporal: the expert outputs are read once, by the combine, and do not fit the
            // caches; streaming them past the L2 and Infinity Cache leaves those to the weights
            // and hq tiles that other items still read
            for (int R = R1; R < nr; R += 16, src += 16 * 512, dst += rstep) {
                typedef unsigned v4 __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(*reinterpret_cast<const v4*>(src), reinterpret_cast<v4*>(dst));
            }
        }
    } else {
        constexpr int RP = BUF >= 128 * 1024 ? 128 : 64;
        static_assert(BUF >= RP * 1024, "staging buffer too small");
        float* out = reinterpret_cast<float*>(a.out);
#pragma unroll
        for (int q = 0; q < 256 / RP; ++q) {
            const int nr = min(RP, nvalid - q * RP);
            if (nr <= 0) break;
            if (q) __syncthreads();
            uint32_t ob[4];   // bytes: row r0 + odd, swizzled column pair of fragment j
#pragma unroll
            for (int j = 0; j < 4; ++j) ob[j] = (r0 + odd) * 1024 + 4 * (wn * 64 + 16 * (j ^ q4 ^ odd) + (r16 & 14));
#pragma unroll
            for (int mi = 0; mi < 8; ++mi) {
                const int R0 = wm * kPfBM + mi * 16 - q * RP;
                if (mi < nact && R0 >= 0 && R0 < RP) {
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {   // the column-pair exchange of the bf16 path
                            const float lo = acc[mi][j][2 * ip], hi = acc[mi][j][2 * ip + 1];
                            const float got = dpp_f32<0xB1>(odd ? lo : hi);
                            *reinterpret_cast<v2f_t*>(buf + ob[j] + (R0 + 2 * ip) * 1024) =
                                v2f_t{odd ? got : lo, odd ? hi : got};
                        }
                }
            }
            __syncthreads();
            const float* s_o = reinterpret_cast<const float*>(buf);
            for (int t = tid; t < nr * 64; t += 512) {
                const int R = t >> 6, m = t & 63;
                typedef float v4 __attribute__((ext_vector_type(4)));   // non-temporal as above
                const v4 v = *reinterpret_cast<const v4*>(s_o + R * 256 + ((4 * m) ^ (16 * (((R >> 2) & 3) ^ (R & 1)))));
                __builtin_nontemporal_store(v, reinterpret_cast<v4*>(out + (int64_t)(rowbase + q * RP + R) * a.H + nb * 256 + 4 * m));
            }
        }
    }
}

__global__ __launch_bounds__(512, 1) void k_gemm2_p2(G2Args a) {
    int nb, pair;
    if (!pf_work_item(a.ord, a.H / 256, __builtin_amdgcn_readfirstlane(*a.npairs), pair, nb)) return;
    const int4 pi = a.pairs[pair];
    const int t0 = __builtin_amdgcn_readfirstlane(pi.x), e = __builtin_amdgcn_readfirstlane(pi.y);
    const int rowbase = __builtin_amdgcn_readfirstlane(pi.z), nvalid = __builtin_amdgcn_readfirstlane(pi.w);
    const bool second = nvalid > kPfBM;
    const int KB = a.I / kGroup;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2 * kP2Stage];
    __shared__ __align__(16) uint8_t s_hs[2 * kPfMaxKB * kPfBM];   // [tile of the pair][kb][row % 16][row / 16]
    __shared__ uint16_t s_sb[kPfMaxKB];                            // scales of column blocks 2 nb, 2 nb + 1

    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    const int nt = second ? 2 : 1;
    // a missing second tile reads as zeros (outside the descriptor's range)
    const v4i_t ra = make_srd(a.hq + (int64_t)t0 * 8 * KB * kFragBytes, (uint32_t)nt * 8 * KB * kFragBytes);
    const v4i_t rw = make_srd(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
    const uint32_t l16 = lane * 16;
    // piece group g = wv + 8 i: fragment g / 2, half g % 2 (A: of the pair's 16 row
    // fragments; B: of the item's 16 column fragments)
    uint32_t asoff[4], bsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = wv + 8 * i;
        asoff[i] = __builtin_amdgcn_readfirstlane((g >> 1) * KB * kFragBytes + (g & 1) * 1024);
        bsoff[i] = __builtin_amdgcn_readfirstlane((nb * 16 + (g >> 1)) * KB * kFragBytes + (g & 1) * 1024);
    }
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * kP2Stage);
#pragma unroll
        for (int i = 0; i < 4; ++i)   // fragments 8.. only for a pair with a second tile (uniform)
            if (i < 2 || second) dma16_async(ra, st + i * 8192, l16, asoff[i] + kb * kFragBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (a.wnt) dma16_async_nt(rw, st + kP2StageA + i * 8192, l16, bsoff[i] + kb * kFragBytes);
            else dma16_async(rw, st + kP2StageA + i * 8192, l16, bsoff[i] + kb * kFragBytes);
        }
    };
    // scales (loaded before the first DMAs, stored after): the pair's hs blocks as dwords
    // (same layout in LDS), the two weight-block scales per K block
    const int nsd = nt * KB * 32;   // dwords
    uint32_t sv[kPfMaxKB / 4];
    {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.hs + (int64_t)t0 * KB * kPfBM);
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 4; ++t) {
            const int i = tid + 512 * t;
            sv[t] = i < nsd ? src[i] : 0u;
        }
    }
    uint32_t sbv = 0;
    if (tid < KB) {
        const uint8_t* sb = a.w2s + ((int64_t)e * KB + tid) * NBS + nb * 2;
        sbv = (uint32_t)sb[0] | (uint32_t)sb[1] << 8;
    }
    issue(0, 0);
    {
#pragma unroll
        for (int t = 0; t < kPfMaxKB / 4; ++t) {
            const int i = tid + 512 * t;
            if (i < nsd) reinterpret_cast<uint32_t*>(s_hs)[i] = sv[t];
        }
        if (tid < KB) s_sb[tid] = (uint16_t)sbv;
    }

    v4f acc[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int nact = __builtin_amdgcn_readfirstlane(min(8, max(0, (nvalid - wm * kPfBM + 15) >> 4)));
    const bool active = nact > 0;
    for (int kb = 0; kb < KB; ++kb) {
        wait_vm<0>();
        __syncthreads();
        if (kb + 1 < KB) issue(kb + 1, (kb + 1) & 1);
        if (active) {
            const uint8_t* cur = buf + (kb & 1) * kP2Stage;
            const v2i_t sa = *reinterpret_cast<const v2i_t*>(s_hs + ((wm * KB + kb) * 16 + r16) * 8);
            const int sb = (s_sb[kb] >> (8 * (wn >> 1))) & 0xFF;
            v8i bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = lds_frag(cur + kP2StageA + (wn * 4 + j) * kFragBytes, lane);
            v8i a0 = lds_frag(cur + (wm * 8) * kFragBytes, lane), a1 = lds_frag(cur + (wm * 8 + 1) * kFragBytes, lane);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                v8i n0 = a0, n1 = a1;
                if (p < 3) {
                    n0 = lds_frag(cur + (wm * 8 + 2 * p + 2) * kFragBytes, lane);
                    n1 = lds_frag(cur + (wm * 8 + 2 * p + 3) * kFragBytes, lane);
                }
                if (2 * p < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[2 * p][j] = mfma_fp8_sel(2 * p & 3, 0, a0, bf[j], acc[2 * p][j], sa[p >> 1], sb);
                }
                if (2 * p + 1 < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[2 * p + 1][j] = mfma_fp8_sel((2 * p + 1) & 3, 0, a1, bf[j], acc[2 * p + 1][j], sa[p >> 1], sb);
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
            }
        }
    }

    if (a.b2) {   // down bias of the lane's columns
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float bv = a.b2[(int64_t)e * a.H + nb * 256 + wn * 64 + 16 * j + r16];
#pragma unroll
            for (int mi = 0; mi < 8; ++mi)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mi][j][i] += bv;
        }
    }

    __syncthreads();   // every wave is done reading the stages
    p2_store_output<2 * kP2Stage>(a, acc, buf, rowbase, nvalid, nb, nact);
}

// ----------------------------------------------------------------------------------------
// Micro-scaled gate/up and down GEMMs on 256-row items (tile pairs), for experts averaging
// >= 128 rows: the item list, waves (2 x 4 of 128 x 64), two LDS stages and output paths of
// k_gemm1_p2 / k_gemm2_p2, with the per-stage scale copies of the 128-row MX kernels.  Stage:
// A 256 rows (32 KB), 16 weight fragments, 256 A-row scale dwords, 16 x 64 weight-scale bytes.
template <int WF>
struct MxP2 {
    static constexpr int FB = WF == kWfmtE2M1 ? 1024 : 2048;
    static constexpr int NBI = 16 * FB / 8192;
    static constexpr int SA = kP2StageA + 16 * FB;
    static constexpr int SB = SA + kP2Rows * 4;
    static constexpr int Stage = SB + 16 * 64;
};

template <int WF>
__device__ __forceinline__ v8i mx_lds_wfrag_at(const uint8_t* wbase, int f, int lane) {
    if constexpr (WF == kWfmtE2M1) {
        const uint4 v = *reinterpret_cast<const uint4*>(wbase + f * 1024 + lane * 16);
        return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    } else {
        return lds_frag(wbase + f * 2048, lane);
    }
}

template <int WF, bool TAP>
__global__ __launch_bounds__(512, 1) void k_gemm1_mxp2(G1Args a) {
    using C = MxP2<WF>;
    int ib, pair;
    if (!pf_work_item(a.ord, a.I / kGroup, __builtin_amdgcn_readfirstlane(*a.npairs), pair, ib)) return;
    const int4 pi = a.pairs[pair];
    const int t0 = __builtin_amdgcn_readfirstlane(pi.x), e = __builtin_amdgcn_readfirstlane(pi.y);
    const int rowbase = __builtin_amdgcn_readfirstlane(pi.z), nvalid = __builtin_amdgcn_readfirstlane(pi.w);
    const bool second = nvalid > kPfBM;
    const int KB = a.H / kGroup, KS = a.H / kMx;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2 * C::Stage];

    const int NB16 = 2 * a.I / 16;
    const v4i_t ra = make_srd(a.xq, (uint32_t)a.T * a.H);
    const v4i_t rw = make_srd(a.w13p + (int64_t)e * NB16 * KB * C::FB, (uint32_t)NB16 * KB * C::FB);
    const v4i_t rxs = make_srd(a.xs, (uint32_t)a.T * KS);
    const v4i_t rws = make_srd(a.w13s + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    auto n16_of = [&](int f) { return f < 8 ? ib * 8 + f : a.I / 16 + ib * 8 + (f - 8); };
    // A: wave instruction i moves rows 8 (wv + 8 i) .. +7 as whole lines (chunk c of row r at
    // r * 128 + 16 (c ^ (r % 8))).  Scale copies, one dword per lane: waves 0..3 the four A
    // scales of row wv * 64 + lane, waves 4..7 the per-lane weight scales of the 16 fragments.
    const bool sc_a = wv < 4;
    int tok[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int r = i < 4 ? 8 * (wv + 8 * i) + (lane >> 3) : (wv & 3) * 64 + lane;
        tok[i] = a.sorted_assign[rowbase + min(r, nvalid - 1)] / a.k;
    }
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)tok[i] * a.H + (((lane & 7) ^ (lane >> 3)) << 4);
    uint32_t bsoff[C::NBI];
#pragma unroll
    for (int i = 0; i < C::NBI; ++i) {
        const int b = (wv * 64 + 512 * i) * 16;
        bsoff[i] = __builtin_amdgcn_readfirstlane(n16_of(b / C::FB) * KB * C::FB + b % C::FB);
    }
    uint32_t scoff;
    if (sc_a) {
        scoff = (uint32_t)tok[4] * KS;
    } else {
        const int t = (wv - 4) * 64 + lane;
        scoff = (uint32_t)n16_of(t >> 4) * KB * 64 + (t & 15) * 4;
    }
    const uint32_t l16 = lane * 16;
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    const uint32_t lds_s = lds_addr(buf) + (sc_a ? C::SA + wv * 256 : C::SB + (wv - 4) * 256);
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * C::Stage);
#pragma unroll
        for (int i = 0; i < 4; ++i)   // rows 128.. only for a pair with a second tile (uniform)
            if (i < 2 || second) dma16_async(ra, st + i * 8192, aoff[i], kb * kGroup);
#pragma unroll
        for (int i = 0; i < C::NBI; ++i) dma16_async(rw, st + kP2StageA + i * 8192, l16, bsoff[i] + kb * C::FB);
        const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_s + s * C::Stage);
        if (sc_a) dma4_async(rxs, ss, scoff, kb * 4);
        else dma4_async(rws, ss, scoff, kb * 64);
    };
    issue(0, 0);

    v4f acc[8][4];   // [row fragment][gate 0, 1 | up 2, 3]
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15, x8 = r16 & 7, G = lane >> 4;
    const int nact = __builtin_amdgcn_readfirstlane(min(8, max(0, (nvalid - wm * kPfBM + 15) >> 4)));
    for (int kb = 0; kb < KB; ++kb) {
        wait_vm<0>();      // block kb landed (this thread's pieces) ...
        __syncthreads();   // ... and everyone's; every wave is done with block kb - 1's stage
        if (kb + 1 < KB) issue(kb + 1, (kb + 1) & 1);
        if (nact > 0) {
            const uint8_t* cur = buf + (kb & 1) * C::Stage;
            v8i bf[4];
            int sb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = j < 2 ? 2 * wn + j : 6 + 2 * wn + j;
                bf[j] = mx_lds_wfrag_at<WF>(cur + kP2StageA, f, lane);
                sb[j] = cur[C::SB + f * 64 + lane];
            }
            auto afrag = [&](int mi, int& sa) __attribute__((always_inline)) {
                const int row = (wm * 8 + mi) * 16 + r16;
                const uint8_t* rowp = cur + row * kGroup;
                const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((G ^ x8) << 4));
                const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((G + 4) ^ x8) << 4));
                sa = (int)((*reinterpret_cast<const uint32_t*>(cur + C::SA + row * 4) >> (8 * G)) & 0xFFu);
                return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            };
            int s0, s1;
            v8i a0 = afrag(0, s0), a1 = afrag(1, s1);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                v8i n0 = a0, n1 = a1;
                int t0s = s0, t1s = s1;
                if (p < 3) {
                    n0 = afrag(2 * p + 2, t0s);
                    n1 = afrag(2 * p + 3, t1s);
                }
                if (2 * p < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[2 * p][j] = mx_mfma<WF>(a0, bf[j], acc[2 * p][j], s0, sb[j]);
                }
                if (2 * p + 1 < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[2 * p + 1][j] = mx_mfma<WF>(a1, bf[j], acc[2 * p + 1][j], s1, sb[j]);
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
                s0 = t0s;
                s1 = t1s;
            }
        }
    }

    // SwiGLU; the wave's two fragments are one 32-column MX group (see k_gemm1_mxpf)
    GuBias bias[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) bias[jj] = gu_bias(a.b13, e, a.I, ib * 128 + (2 * wn + jj) * 16 + r16);
    float hv[8][2][4];
    int ex[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi < nact) {
            float m[4];
            swiglu_frag(acc[mi], a.b13, bias, hv[mi], m);
            tap_frag<TAP>(a.htap, a.I, rowbase, (wm * 8 + mi) * 16, nvalid, ib * 128 + 2 * wn * 16, hv[mi]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ex[mi][i] = mx_scale_exponent<kWfmtE4M3>(m[i]);
        }
    }
    __syncthreads();   // every wave is done reading the stages before buf is reused
    uint8_t* s_h = buf;   // [256 rows][128], 16-byte chunks XOR-swizzled by row % 8
    const int q = lane & 3, g4 = 4 * (lane >> 4), KS2 = a.I / kMx;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi < nact) {
            const int row = (wm * 8 + mi) * 16 + g4 + q;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                *reinterpret_cast<uint32_t*>(s_h + row * 128 + (((2 * wn + jj) ^ (row & 7)) << 4) + 4 * (r16 >> 2)) =
                    e4m3_quad_rows(hv[mi][jj], ex[mi], q);
            if (r16 == 0) {   // the pair's two tiles are consecutive: tile row t0 * 128 + row
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.hs[((int64_t)t0 * kPfBM + (wm * 8 + mi) * 16 + g4 + i) * KS2 + ib * 4 + wn] =
                        (uint8_t)(ex[mi][i] + 127);
            }
        }
    }
    __syncthreads();
    const int KB2 = a.I / kGroup, nf = second ? 16 : 8;
    for (int q2 = tid; q2 < nf * 128; q2 += 512) {
        const int mf = q2 >> 7, w = q2 & 127, hh = w >> 6, ln = w & 63;
        const int R = mf * 16 + (ln & 15), c = 4 * hh + (ln >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(s_h + R * 128 + ((c ^ (R & 7)) << 4));
        *reinterpret_cast<uint4*>(a.hq + (((int64_t)t0 * 8 + mf) * KB2 + ib) * kFragBytes + hh * 1024 + ln * 16) = v;
    }
}

template <int WF>
__global__ __launch_bounds__(512, 1) void k_gemm2_mxp2(G2Args a) {
    using C = MxP2<WF>;
    int nb, pair;
    if (!pf_work_item(a.ord, a.H / 256, __builtin_amdgcn_readfirstlane(*a.npairs), pair, nb)) return;
    const int4 pi = a.pairs[pair];
    const int t0 = __builtin_amdgcn_readfirstlane(pi.x), e = __builtin_amdgcn_readfirstlane(pi.y);
    const int rowbase = __builtin_amdgcn_readfirstlane(pi.z), nvalid = __builtin_amdgcn_readfirstlane(pi.w);
    const bool second = nvalid > kPfBM;
    const int KB = a.I / kGroup, KS2 = a.I / kMx;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 2, wn = wv & 3;

    __shared__ __align__(16) uint8_t buf[2 * C::Stage];

    const int NB16 = a.H / 16, nt = second ? 2 : 1;
    // a missing second tile reads as zeros (outside the descriptors' ranges)
    const v4i_t ra = make_srd(a.hq + (int64_t)t0 * 8 * KB * kFragBytes, (uint32_t)nt * 8 * KB * kFragBytes);
    const v4i_t rw = make_srd(a.w2p + (int64_t)e * NB16 * KB * C::FB, (uint32_t)NB16 * KB * C::FB);
    const v4i_t rhs = make_srd(a.hs + (int64_t)t0 * kPfBM * KS2, (uint32_t)nt * kPfBM * KS2);
    const v4i_t rws = make_srd(a.w2s + (int64_t)e * NB16 * KB * 64, (uint32_t)NB16 * KB * 64);
    const uint32_t l16 = lane * 16;
    uint32_t asoff[4], bsoff[C::NBI];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = wv + 8 * i;   // piece group: fragment g / 2, half g % 2 of the pair's 16 row fragments
        asoff[i] = __builtin_amdgcn_readfirstlane((g >> 1) * KB * kFragBytes + (g & 1) * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::NBI; ++i) {
        const int b = (wv * 64 + 512 * i) * 16;
        bsoff[i] = __builtin_amdgcn_readfirstlane((nb * 16 + b / C::FB) * KB * C::FB + b % C::FB);
    }
    const bool sc_a = wv < 4;
    uint32_t scoff;
    if (sc_a) {
        scoff = (uint32_t)(wv * 64 + lane) * KS2;
    } else {
        const int t = (wv - 4) * 64 + lane;
        scoff = (uint32_t)(nb * 16 + (t >> 4)) * KB * 64 + (t & 15) * 4;
    }
    const uint32_t lds_w = lds_addr(buf) + wv * 1024;
    const uint32_t lds_s = lds_addr(buf) + (sc_a ? C::SA + wv * 256 : C::SB + (wv - 4) * 256);
    auto issue = [&](int kb, int s) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_w + s * C::Stage);
#pragma unroll
        for (int i = 0; i < 4; ++i)   // fragments 8.. only for a pair with a second tile (uniform)
            if (i < 2 || second) dma16_async(ra, st + i * 8192, l16, asoff[i] + kb * kFragBytes);
#pragma unroll
        for (int i = 0; i < C::NBI; ++i) dma16_async(rw, st + kP2StageA + i * 8192, l16, bsoff[i] + kb * C::FB);
        const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_s + s * C::Stage);
        if (sc_a) dma4_async(rhs, ss, scoff, kb * 4);
        else dma4_async(rws, ss, scoff, kb * 64);
    };
    issue(0, 0);

    v4f acc[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15, G = lane >> 4;
    const int nact = __builtin_amdgcn_readfirstlane(min(8, max(0, (nvalid - wm * kPfBM + 15) >> 4)));
    for (int kb = 0; kb < KB; ++kb) {
        wait_vm<0>();
        __syncthreads();
        if (kb + 1 < KB) issue(kb + 1, (kb + 1) & 1);
        if (nact > 0) {
            const uint8_t* cur = buf + (kb & 1) * C::Stage;
            v8i bf[4];
            int sb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf[j] = mx_lds_wfrag_at<WF>(cur + kP2StageA, wn * 4 + j, lane);
                sb[j] = cur[C::SB + (wn * 4 + j) * 64 + lane];
            }
            auto afrag = [&](int mi, int& sa) __attribute__((always_inline)) {
                const int mf = wm * 8 + mi;
                sa = (int)((*reinterpret_cast<const uint32_t*>(cur + C::SA + (mf * 16 + r16) * 4) >> (8 * G)) & 0xFFu);
                return lds_frag(cur + mf * kFragBytes, lane);
            };
            int s0, s1;
            v8i a0 = afrag(0, s0), a1 = afrag(1, s1);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                v8i n0 = a0, n1 = a1;
                int t0s = s0, t1s = s1;
                if (p < 3) {
                    n0 = afrag(2 * p + 2, t0s);
                    n1 = afrag(2 * p + 3, t1s);
                }
                if (2 * p < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[2 * p][j] = mx_mfma<WF>(a0, bf[j], acc[2 * p][j], s0, sb[j]);
                }
                if (2 * p + 1 < nact) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[2 * p + 1][j] = mx_mfma<WF>(a1, bf[j], acc[2 * p + 1][j], s1, sb[j]);
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
                s0 = t0s;
                s1 = t1s;
            }
        }
    }
    if (a.b2) {   // down bias of the lane's columns
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float bv = a.b2[(int64_t)e * a.H + nb * 256 + wn * 64 + 16 * j + r16];
#pragma unroll
            for (int mi = 0; mi < 8; ++mi)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mi][j][i] += bv;
        }
    }
    __syncthreads();   // every wave is done reading the stages
    p2_store_output<2 * C::Stage>(a, acc, buf, rowbase, nvalid, nb, nact);
}

// ----------------------------------------------------------------------------------------
// The super-tile order pays off once the tiles fill several of its 64-tile windows.
int ffn_super_tile_order(int ntiles_max) { return ntiles_max >= 512 ? 1 : 0; }
// The 256-row down GEMM takes the super-tile order from twice as many tiles on: on the
// DeepSeek-V3-shaped prefill (512 tiles, one pair per expert, so no two pairs share weight
// columns) the column-block order measured 3% faster for it, while its gate/up GEMM and the
// Zipf prefill's (1152 tiles, many pairs per expert) keep gaining from super-tiles.
static int ffn_super_tile_order_down(int ntiles_max) { return ntiles_max >= 1024 ? 1 : 0; }

// Launch a gate+up kernel template with TAP (the float32 h test output) on or off.
#define MOE_LAUNCH_TAP(tap, KERNEL, grid, block, ...)                                       \
    do {                                                                                     \
        if (tap) hipLaunchKernelGGL((KERNEL<__VA_ARGS__ true>), grid, block, 0, st, g1);     \
        else hipLaunchKernelGGL((KERNEL<__VA_ARGS__ false>), grid, block, 0, st, g1);        \
    } while (0)

static G1Args g1_args(const FfnArgs& f, const FfnWs& w, int ord) {
    return G1Args{f.xq, f.xs, f.T, f.k, f.H, f.I, f.counts, f.offsets, f.sorted_assign, w.tiles, w.ntiles, f.w13p,
                  f.w13s, w.hq, w.hs, ord, w.pairs, w.npairs, f.debug_h, f.b13};
}

static G2Args g2_args(const FfnArgs& f, const FfnWs& w, int ord) {
    return G2Args{w.hq, w.hs, f.H, f.I, f.counts, f.offsets, w.tiles, w.ntiles, f.w2p, f.w2s, f.out, f.out_bf16,
                  ord, w.pairs, w.npairs, f.b2};
}

template <int MFW, int NFW1, int NFW2, int WM, int WN, int PF1, int PF2>
static hipError_t run_ffn(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    const G1Args g1 = g1_args(f, w, ffn_super_tile_order(p.ntiles_max));
    MOE_LAUNCH_TAP(f.debug_h, k_gemm1, dim3(p.ntiles_max, f.I / kGroup), dim3(64 * WM * WN), MFW, NFW1, WM, WN, PF1,);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    const G2Args g2 = g2_args(f, w, ffn_super_tile_order(p.ntiles_max));
    const int ncols = 16 * NFW2 * WN;
    hipLaunchKernelGGL((k_gemm2<MFW, NFW2, WM, WN, PF2>), dim3(p.ntiles_max, f.H / ncols), dim3(64 * WM * WN), 0,
                       st, g2);
    return hipGetLastError();
}

template <int NFW1, int WN1, int PF1, int NFW2, int WN2, int PF2>
static hipError_t run_ffn_dec(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    const G1Args g1 = g1_args(f, w, ffn_super_tile_order(p.ntiles_max));
    MOE_LAUNCH_TAP(f.debug_h, k_gemm1_dec, dim3(p.ntiles_max, f.I / kGroup), dim3(64 * WN1), NFW1, WN1, PF1,);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    const G2Args g2 = g2_args(f, w, ffn_super_tile_order(p.ntiles_max));
    hipLaunchKernelGGL((k_gemm2_dec<NFW2, WN2, PF2>), dim3(p.ntiles_max, f.H / (16 * NFW2 * WN2)), dim3(64 * WN2), 0,
                       st, g2);
    return hipGetLastError();
}

static hipError_t launch_gemm2_p2(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, int ord, hipStream_t st) {
    G2Args g2 = g2_args(f, w, ord);
    // experts averaging at most one 256-row item: each weight byte is read by one workgroup,
    // and streaming the weights past the caches leaves those to the hq tiles
    g2.wnt = (int64_t)f.T * f.k <= (int64_t)256 * f.E;
    const int grid2 = ord ? kXcds * ord_ranks(p.npairs_max, f.H / 256)
                          : (int)(ceil_div((int64_t)(f.H / 256) * p.npairs_max, kXcds) * kXcds);
    hipLaunchKernelGGL(k_gemm2_p2, dim3(grid2), dim3(512), 0, st, g2);
    return hipGetLastError();
}

template <int WF>
static hipError_t run_ffn_mx_pf(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid) {
    const G1Args g1 = g1_args(f, w, ffn_super_tile_order(p.ntiles_max));
    const int grid1 = g1.ord ? kXcds * ord_ranks(p.ntiles_max, f.I / kGroup)
                             : (int)(ceil_div((int64_t)(f.I / kGroup) * p.ntiles_max, kXcds) * kXcds);
    if (f.debug_h) hipLaunchKernelGGL((k_gemm1_mxpf<WF, true>), dim3(grid1), dim3(512), 0, st, g1);
    else hipLaunchKernelGGL((k_gemm1_mxpf<WF, false>), dim3(grid1), dim3(512), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    const G2Args g2 = g2_args(f, w, ffn_super_tile_order(p.ntiles_max));
    const int grid2 = g2.ord ? kXcds * ord_ranks(p.ntiles_max, f.H / 256)
                             : (int)(ceil_div((int64_t)(f.H / 256) * p.ntiles_max, kXcds) * kXcds);
    hipLaunchKernelGGL((k_gemm2_mxpf<WF>), dim3(grid2), dim3(512), 0, st, g2);
    return hipGetLastError();
}

template <int WF>
static hipError_t run_ffn_mx_p2(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid,
                                bool pairs_ready) {
    if (!pairs_ready)
        hipLaunchKernelGGL(k_pairs, dim3(1), dim3(1024), 0, st, f.counts, f.offsets, f.E, w.pairs, w.npairs);
    const int ord = ffn_super_tile_order(p.ntiles_max);
    const G1Args g1 = g1_args(f, w, ord);
    const int grid1 = ord ? kXcds * ord_ranks(p.npairs_max, f.I / kGroup)
                          : (int)(ceil_div((int64_t)(f.I / kGroup) * p.npairs_max, kXcds) * kXcds);
    if (f.debug_h) hipLaunchKernelGGL((k_gemm1_mxp2<WF, true>), dim3(grid1), dim3(512), 0, st, g1);
    else hipLaunchKernelGGL((k_gemm1_mxp2<WF, false>), dim3(grid1), dim3(512), 0, st, g1);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    const int ord2 = ffn_super_tile_order_down(p.ntiles_max);
    const G2Args g2 = g2_args(f, w, ord2);
    const int grid2 = ord2 ? kXcds * ord_ranks(p.npairs_max, f.H / 256)
                           : (int)(ceil_div((int64_t)(f.H / 256) * p.npairs_max, kXcds) * kXcds);
    hipLaunchKernelGGL((k_gemm2_mxp2<WF>), dim3(grid2), dim3(512), 0, st, g2);
    return hipGetLastError();
}

// The MX schemes on 128-row tiles, or on 256-row items (tile pairs) when the plan asks for them
// (the plan takes either only for H % 256 == 0).
hipError_t launch_ffn_mx_pf(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid,
                            bool pairs_ready) {
    if (f.H % 256 != 0) return hipErrorInvalidValue;
    if (p.pairs)
        return f.quant == kQuantW4A8 ? run_ffn_mx_p2<kWfmtE2M1>(f, p, w, st, mid, pairs_ready)
                                     : run_ffn_mx_p2<kWfmtE4M3>(f, p, w, st, mid, pairs_ready);
    return f.quant == kQuantW4A8 ? run_ffn_mx_pf<kWfmtE2M1>(f, p, w, st, mid)
                                 : run_ffn_mx_pf<kWfmtE4M3>(f, p, w, st, mid);
}

static hipError_t run_ffn_pf(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid,
                             bool pairs_ready) {
    const G1Args g1 = g1_args(f, w, ffn_super_tile_order(p.ntiles_max));
    const int KB1 = f.H / kGroup, pgrid = persistent_grid();
#ifndef MOE_NO_PP
    // the persistent kernel where its staged scales and item table fit
    if (KB1 >= 2 && KB1 <= kPpMaxKB && persistent_items_per_wg(p.ntiles_max, f.I / kGroup, pgrid) <= kPpMaxItems) {
        if (KB1 <= 8) MOE_LAUNCH_TAP(f.debug_h, k_gemm1_pp, dim3(pgrid), dim3(512), 2,);
        else if (KB1 <= 16) MOE_LAUNCH_TAP(f.debug_h, k_gemm1_pp, dim3(pgrid), dim3(512), 4,);
        else MOE_LAUNCH_TAP(f.debug_h, k_gemm1_pp, dim3(pgrid), dim3(512), 8,);
    } else
#endif
    {
        const int grid1 = g1.ord ? kXcds * ord_ranks(p.ntiles_max, f.I / kGroup)
                                 : (int)(ceil_div((int64_t)(f.I / kGroup) * p.ntiles_max, kXcds) * kXcds);
        MOE_LAUNCH_TAP(f.debug_h, k_gemm1_pf, dim3(grid1), dim3(512),);
    }
    (void)pgrid;
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    if (p.pairs_down) {   // 256-row down items over the same hq / hs tile slots
        if (!pairs_ready)
            hipLaunchKernelGGL(k_pairs, dim3(1), dim3(1024), 0, st, f.counts, f.offsets, f.E, w.pairs, w.npairs);
        return launch_gemm2_p2(f, p, w, ffn_super_tile_order_down(p.ntiles_max), st);
    }
    const G2Args g2 = g2_args(f, w, ffn_super_tile_order(p.ntiles_max));
#ifndef MOE_NO_RB
    // the persistent down GEMM (k_ffn_rb.hip) where its item tables fit
    if (ffn_rb_supported(f.H, f.I, f.E, p.ntiles_max)) return launch_gemm2_rb(f, w, p.ntiles_max, g2.ord, st);
#endif
    const int grid2 = g2.ord ? kXcds * ord_ranks(p.ntiles_max, f.H / 256)
                             : (int)(ceil_div((int64_t)(f.H / 256) * p.ntiles_max, kXcds) * kXcds);
    hipLaunchKernelGGL(k_gemm2_pf, dim3(grid2), dim3(512), 0, st, g2);
    return hipGetLastError();
}

hipError_t launch_pairs(const int32_t* counts, const int32_t* offsets, int E, int4* pairs, int32_t* npairs,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_pairs, dim3(1), dim3(1024), 0, st, counts, offsets, E, pairs, npairs);
    return hipGetLastError();
}

static hipError_t run_ffn_p2(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid,
                             bool pairs_ready) {
    if (!pairs_ready)
        hipLaunchKernelGGL(k_pairs, dim3(1), dim3(1024), 0, st, f.counts, f.offsets, f.E, w.pairs, w.npairs);
    const int ord = ffn_super_tile_order(p.ntiles_max);
    const G1Args g1 = g1_args(f, w, ord);
    const int grid1 = ord ? kXcds * ord_ranks(p.npairs_max, f.I / kGroup)
                          : (int)(ceil_div((int64_t)(f.I / kGroup) * p.npairs_max, kXcds) * kXcds);
    MOE_LAUNCH_TAP(f.debug_h, k_gemm1_p2, dim3(grid1), dim3(512),);
    if (mid) {
        const hipError_t e = hipEventRecord(mid, st);
        if (e != hipSuccess) return e;
    }
    return launch_gemm2_p2(f, p, w, ffn_super_tile_order_down(p.ntiles_max), st);
}

FfnWs carve_ffn_ws(const FfnArgs& f, void* ws) {
    const FfnWsLayout l = ffn_ws_layout(f.T, f.H, f.I, f.E, f.k, f.quant);
    uint8_t* w = static_cast<uint8_t*>(ws);
    FfnWs r;
    r.tiles = reinterpret_cast<int2*>(w + l.tiles);
    r.ntiles = reinterpret_cast<int32_t*>(w + l.ntiles);
    r.hq = w + l.hq;
    r.hs = w + l.hs;
    r.bs = ffn_plan(f.T, f.k, f.E, f.quant, f.H).BM == 128 ? reinterpret_cast<uint32_t*>(w + l.bs) : nullptr;
    r.pairs = reinterpret_cast<int4*>(w + l.pairs);
    r.npairs = reinterpret_cast<int32_t*>(w + l.npairs);
    return r;
}

// ----------------------------------------------------------------------------------------
// Test outputs: copy the re-quantised h and its scales out of the down GEMM's operand layout
// into row-major [A, I] and [A, I / group] in sorted order.  The hq layouts (tile slots of BM
// rows, fragment mf = row / 16 of the slot, one 2 KB block per 128 columns; lane ln and half
// hh hold 16 bytes b):
//   E4M3 per 128 (decode, staged and plain 128-row tiles): row 16 mf + ln % 16, column
//     32 (ln / 16) + 16 hh + b;
//   MX (the instruction's K order for 32-element scales): row ln % 16, column
//     64 hh + 16 (ln / 16) + b;
//   W8A16: bf16 rows [tile][16][I].
// The hs layouts: [tile * BM + row][I / 128] (decode and plain 128-row tiles),
// [tile][I / 128][row % 16][row / 16] (staged 128-row tiles), [tile * 16 + row][I / 32] (MX).
enum HLayout { kHlDec = 0, kHlStaged = 1, kHlPlain = 2, kHlMx = 3, kHlW16 = 4 };

__global__ __launch_bounds__(256) void k_unpack_h(const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                                                  const int32_t* __restrict__ counts,
                                                  const int32_t* __restrict__ offsets, int BM, int I, int layout,
                                                  const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
                                                  uint8_t* __restrict__ dq, uint8_t* __restrict__ ds) {
    const int tile = blockIdx.x;
    if (tile >= *ntiles) return;
    const int2 te = tiles[tile];
    const int nvalid = min(BM, counts[te.x] - te.y);
    const int64_t rowbase = offsets[te.x] + te.y;
    if (layout == kHlW16) {
        for (int idx = threadIdx.x; idx < nvalid * I; idx += 256) {
            const int R = idx / I, c = idx - R * I;
            reinterpret_cast<uint16_t*>(dq)[(rowbase + R) * I + c] =
                reinterpret_cast<const uint16_t*>(hq)[((int64_t)tile * 16 + R) * I + c];
        }
        return;
    }
    const int KB2 = I / kGroup, MF = BM / 16;
    for (int idx = threadIdx.x; idx < nvalid * I; idx += 256) {
        const int R = idx / I, c = idx - R * I;
        const int kb = c >> 7, cc = c & 127, mf = R >> 4, r = R & 15;
        int ln, hh;
        if (layout == kHlMx) {
            hh = cc >> 6;
            ln = r + 16 * ((cc >> 4) & 3);
        } else {
            hh = (cc >> 4) & 1;
            ln = r + 16 * (cc >> 5);
        }
        dq[(rowbase + R) * I + c] = hq[(((int64_t)tile * MF + mf) * KB2 + kb) * kFragBytes + hh * 1024 + ln * 16 + (cc & 15)];
    }
    const int ng = layout == kHlMx ? I / 32 : KB2;
    for (int idx = threadIdx.x; idx < nvalid * ng; idx += 256) {
        const int R = idx / ng, g = idx - R * ng;
        int64_t src;
        if (layout == kHlStaged) src = ((int64_t)tile * KB2 + g) * 128 + (R & 15) * 8 + (R >> 4);
        else src = ((int64_t)tile * BM + R) * ng + g;
        ds[(rowbase + R) * ng + g] = hs[src];
    }
}

hipError_t launch_grouped_ffn(const FfnArgs& f, void* ws, hipStream_t st, hipEvent_t mid, bool tiles_ready,
                              bool pairs_ready) {
    const FfnPlan p = ffn_plan(f.T, f.k, f.E, f.quant, f.H);
    const FfnWs w = carve_ffn_ws(f, ws);
    if (!tiles_ready) {
        const hipError_t e = launch_tiles(f.counts, f.E, p.BM, w.tiles, w.ntiles, st);
        if (e != hipSuccess) return e;
    }
    hipError_t e;
    int layout;
    if (f.quant == kQuantW8A16) {
        layout = kHlW16;
        e = launch_ffn_w16(f, p, w, st, mid);
    } else if (f.quant != kQuantFp8Block128) {
        layout = kHlMx;
        e = p.BM == 128 ? launch_ffn_mx_pf(f, p, w, st, mid, pairs_ready) : launch_ffn_mx(f, p, w, st, mid);
    } else if (p.BM == 16) {
        // output columns per workgroup of the down GEMM = 128, a divisor of H
        layout = kHlDec;
        e = run_ffn_dec<MOE_DEC_GEMM1, MOE_DEC_GEMM2>(f, p, w, st, mid);
    } else if (f.H / kGroup <= kPfMaxKB && f.I / kGroup <= kPfMaxKB && f.H % 256 == 0) {
        // 128-row tiles: the staged kernels need the tile's A scales in LDS and 256-column
        // down-GEMM blocks; other shapes take the plain 128-row kernels
        layout = kHlStaged;
#ifndef MOE_NO_PAIRS
        if (p.pairs) e = run_ffn_p2(f, p, w, st, mid, pairs_ready);
        else
#endif
            e = run_ffn_pf(f, p, w, st, mid, pairs_ready);
    } else {
        layout = kHlPlain;
        e = run_ffn<4, 4, 4, 2, 2, 2, 2>(f, p, w, st, mid);
    }
    if (e != hipSuccess || !f.debug_h) return e;
    hipLaunchKernelGGL(k_unpack_h, dim3(p.ntiles_max), dim3(256), 0, st, w.tiles, w.ntiles, f.counts, f.offsets, p.BM,
                       f.I, layout, w.hq, w.hs, f.debug_hq, f.debug_hs);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Combine: workgroup (token, 256 x CPT column groups); a group is the columns of one
// expert row that one load brings in: 16 bytes (4 float32 columns, or 8 bf16 ones), or 8
// bytes (4 bf16 columns) for bf16 rows whose length is not a multiple of 8.  Each thread owns
// CPT groups 256 apart and issues the loads of up to 8 expert rows for all of them before
// summing them in slot order j = 0, 1, ... (expert_out is read exactly once: non-temporal
// loads keep it from displacing cached lines).
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));

template <bool BF16, int CW, int CPT>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ eo, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int k, int H,
                                                 uint16_t* __restrict__ y) {
    static_assert(BF16 ? (CW == 8 || CW == 4) : CW == 4, "16-byte groups, or 8-byte bf16 groups");
    constexpr int EB = BF16 ? 2 : 4;        // bytes per expert_out element
    constexpr int NW = CW * EB / 4;         // dwords per group load
    typedef std::conditional_t<NW == 4, v4u_t, v2u_t> ld_t;
    const int t = blockIdx.x;
    const int g0 = blockIdx.y * 256 * CPT + threadIdx.x;
    const int ng = H / CW;
    float acc[CPT][CW];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int i = 0; i < CW; ++i) acc[c][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        ld_t v[8][CPT];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int p = j < k ? pos[(int64_t)t * k + j] : -1;
            wj[u] = p >= 0 ? w[(int64_t)t * k + j] : 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int g = g0 + c * 256;
                if (p >= 0 && g < ng) {
                    const int64_t off = ((int64_t)p * H + (int64_t)g * CW) * EB;
                    v[u][c] = __builtin_nontemporal_load(
                        reinterpret_cast<const ld_t*>(reinterpret_cast<const uint8_t*>(eo) + off));
                } else {
                    v[u][c] = ld_t{};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
#pragma unroll
                    for (int i = 0; i < CW; ++i) {
                        float x;
                        if constexpr (BF16) x = bf16_to_f32(i & 1 ? v[u][c][i / 2] >> 16 : v[u][c][i / 2] & 0xFFFFu);
                        else x = __uint_as_float(v[u][c][i]);
                        acc[c][i] = fmaf(wj[u], x, acc[c][i]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int g = g0 + c * 256;
        if (g < ng) {
            uint32_t o[CW / 2];
#pragma unroll
            for (int i = 0; i < CW / 2; ++i)
                o[i] = (uint32_t)f32_to_bf16(acc[c][2 * i]) | ((uint32_t)f32_to_bf16(acc[c][2 * i + 1]) << 16);
            if constexpr (CW == 8) *reinterpret_cast<uint4*>(y + (int64_t)t * H + g * CW) = make_uint4(o[0], o[1], o[2], o[3]);
            else *reinterpret_cast<uint2*>(y + (int64_t)t * H + g * CW) = make_uint2(o[0], o[1]);
        }
    }
}

// Column groups per thread: the largest of 4, 2, 1 whose 256 x CPT slots the row fills.
// More groups per thread put more independent loads in flight (fp32 rows of H = 4096: 4
// measured best); for short rows the unused slots only cost registers and occupancy (fp32
// rows of H = 768: 1 cut the combine from 14.6 to 11.8 us).
template <bool BF16, int CW>
static void launch_combine_t(const void* eo, const int32_t* pos, const float* w, int T, int k, int H, uint16_t* y,
                             hipStream_t st) {
    const int ng = H / CW;
    if (ng >= 256 * 4)
        hipLaunchKernelGGL((k_combine<BF16, CW, 4>), dim3(T, (unsigned)ceil_div(ng, 256 * 4)), dim3(256), 0, st, eo,
                           pos, w, k, H, y);
    else if (ng >= 256 * 2)
        hipLaunchKernelGGL((k_combine<BF16, CW, 2>), dim3(T, (unsigned)ceil_div(ng, 256 * 2)), dim3(256), 0, st, eo,
                           pos, w, k, H, y);
    else
        hipLaunchKernelGGL((k_combine<BF16, CW, 1>), dim3(T, (unsigned)ceil_div(ng, 256)), dim3(256), 0, st, eo, pos,
                           w, k, H, y);
}

hipError_t launch_combine(const void* eo, int bf16, const int32_t* pos, const float* w, int T, int k, int H,
                          uint16_t* y, hipStream_t st) {
    // bf16 rows of a length that is a multiple of 8 load 16 bytes per group, the rest 8
    if (bf16 && H % 8 == 0) launch_combine_t<true, 8>(eo, pos, w, T, k, H, y, st);
    else if (bf16) launch_combine_t<true, 4>(eo, pos, w, T, k, H, y, st);
    else launch_combine_t<false, 4>(eo, pos, w, T, k, H, y, st);
    return hipGetLastError();
}

}  // namespace moe
