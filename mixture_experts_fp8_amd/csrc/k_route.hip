// Routing, gate prelude and the static dispatch (gfx950).
//
// Routing follows the MindIE-SD "Fused MoE" page (parameter table and section
// "路由选择"): softmax or sigmoid scores, optional group-limited selection, top-k,
// renormalisation and routed_scaling_factor.  The gate prelude follows mlx-native
// "moe_gate.rs" (RMSNorm, float32 router matmul, top-K, softmax, per-expert scale).
// Dispatch is the static dispatcher ("Dispatcher 策略"): a stable counting sort of the
// flat assignments by expert id.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------------------
// Gate prelude: logits[t, e] = r_t * sum_h x[t,h] * norm_w[h] * W_r[e, h], with
// r_t = 1 / sqrt(mean_h x[t,h]^2 + eps) -- RMSNorm then the float32 router matmul, with the
// per-token factor r_t applied once to the finished dot product.
// Workgroup (expert e, 4 tokens), 4 waves splitting H into interleaved 256-wide steps:
// lane l owns 4 consecutive h per step, loaded as one 16-byte W_r / norm load and one 8-byte
// load per token; each token's sum of squares comes from the same loaded values.  The loads
// of kPreB steps are issued before any of their sums (one memory round trip per kPreB steps;
// the sums still run in h order).  Partial sums meet in LDS.
constexpr int kPreT = 4;
constexpr int kPreB = 4;

__global__ __launch_bounds__(256) void k_gate_prelude(const uint16_t* __restrict__ x, int T, int H, int E,
                                                      const float* __restrict__ norm_w,
                                                      const float* __restrict__ router_w, float eps,
                                                      float* __restrict__ logits) {
    __shared__ float s_part[4][2 * kPreT];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * kPreT;
    const int nt = min(kPreT, T - t0);
    const float* wr = router_w + (int64_t)e * H;
    float d[kPreT], ss[kPreT];
#pragma unroll
    for (int t = 0; t < kPreT; ++t) d[t] = ss[t] = 0.f;
    for (int hb = (wv * 64 + lane) * 4; hb < H; hb += 1024 * kPreB) {
        float4 w4[kPreB], n4[kPreB];
        uint2 u[kPreB][kPreT];
#pragma unroll
        for (int i = 0; i < kPreB; ++i) {
            const int h = hb + 1024 * i;
            if (h < H) {
                w4[i] = *reinterpret_cast<const float4*>(wr + h);
                n4[i] = *reinterpret_cast<const float4*>(norm_w + h);
#pragma unroll
                for (int t = 0; t < kPreT; ++t)
                    if (t < nt) u[i][t] = *reinterpret_cast<const uint2*>(x + (int64_t)(t0 + t) * H + h);
            }
        }
#pragma unroll
        for (int i = 0; i < kPreB; ++i) {
            if (hb + 1024 * i < H) {
                const float wn0 = w4[i].x * n4[i].x, wn1 = w4[i].y * n4[i].y;
                const float wn2 = w4[i].z * n4[i].z, wn3 = w4[i].w * n4[i].w;
#pragma unroll
                for (int t = 0; t < kPreT; ++t) {
                    if (t < nt) {
                        const float x0 = bf16_to_f32(u[i][t].x & 0xFFFFu), x1 = bf16_to_f32(u[i][t].x >> 16);
                        const float x2 = bf16_to_f32(u[i][t].y & 0xFFFFu), x3 = bf16_to_f32(u[i][t].y >> 16);
                        d[t] = fmaf(x0, wn0, fmaf(x1, wn1, fmaf(x2, wn2, fmaf(x3, wn3, d[t]))));
                        ss[t] = fmaf(x0, x0, fmaf(x1, x1, fmaf(x2, x2, fmaf(x3, x3, ss[t]))));
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kPreT; ++t) {
        const float dt = wave_sum(d[t]);
        const float st = wave_sum(ss[t]);
        if (lane == 0) {
            s_part[wv][t] = dt;
            s_part[wv][kPreT + t] = st;
        }
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = threadIdx.x;
        const float dt = (s_part[0][t] + s_part[1][t]) + (s_part[2][t] + s_part[3][t]);
        const float st = (s_part[0][kPreT + t] + s_part[1][kPreT + t]) + (s_part[2][kPreT + t] + s_part[3][kPreT + t]);
        logits[(int64_t)(t0 + t) * E + e] = dt * (1.0f / sqrtf(st / (float)H + eps));
    }
}

hipError_t launch_gate_prelude(const uint16_t* x, int T, int H, int E, const float* norm_w,
                               const float* router_w, float eps, float* logits, hipStream_t st) {
    dim3 grid((unsigned)E, (unsigned)ceil_div(T, kPreT));
    hipLaunchKernelGGL(k_gate_prelude, grid, dim3(256), 0, st, x, T, H, E, norm_w, router_w, eps, logits);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Top-k routing: order-preserving keys and the wave maximum over them.

__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);   // +0 and -0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave maximum of 64-bit keys (all lanes active): DPP butterfly inside each 16-lane row on
// both halves, then the four row maxima read from lanes 0, 16, 32, 48 (uniform result).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint64_t w = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
    return w > v ? w : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<0xB1>(v);
    v = dpp_max_u64<0x4E>(v);
    v = dpp_max_u64<0x124>(v);
    v = dpp_max_u64<0x128>(v);
    uint64_t r = 0;
#pragma unroll
    for (int l = 0; l < 64; l += 16) {
        const uint64_t w = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
        r = w > r ? w : r;
    }
    return r;
}

// The token row's activation quantisation: loads of the 128-column blocks g0 .. g0 + 31
// (16 lanes per block, 8 columns per lane), then their E4M3 codes and UE8M0 scales per group
// of qo.group columns -- 128 (one scale per block, amax over the 16 lanes) or 32 (four scales
// per block, amax over aligned quads of lanes); the scale rule is the same.  The row is read
// once: non-temporal.
__device__ __forceinline__ void xrow_load(const QuantOut& qo, int t, int g0, int lane, uint4 (&v)[8]) {
    const int ngc = qo.H / kGroup;
    const uint16_t* xr = qo.x + (int64_t)t * qo.H;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int g = g0 + (lane >> 4) + 4 * i;
        if (g < ngc) {
            const v4u_t u = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(xr + g * kGroup + (lane & 15) * 8));
            v[i] = make_uint4(u[0], u[1], u[2], u[3]);
        }
    }
}
// 8 bf16 values of a 32-column group whose other 24 sit in the lane's quad.
__device__ __forceinline__ void quant_group4_v(const uint4 v, uint8_t* __restrict__ dq, uint8_t* __restrict__ ds,
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
    amax = fmaxf(amax, dpp_f32<0xB1>(amax));
    amax = fmaxf(amax, dpp_f32<0x4E>(amax));
    const int e = scale_exponent(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = ldexpf(f[i], -e);
    uint2 q;
    q.x = cvt4_e4m3(f[0], f[1], f[2], f[3]);
    q.y = cvt4_e4m3(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<uint2*>(dq + sub * 8) = q;
    if ((sub & 3) == 0) *ds = (uint8_t)(e + 127);
}

__device__ __forceinline__ void xrow_quant(const QuantOut& qo, int t, int g0, int lane, const uint4 (&v)[8]) {
    const int ngc = qo.H / kGroup;
    const int nsc = qo.H / qo.group;   // scales per row
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int g = g0 + (lane >> 4) + 4 * i;
        if (g < ngc) {
            uint8_t* dq = qo.xq + (int64_t)t * qo.H + g * kGroup;
            if (qo.group == kGroup)
                quant_group16_v(v[i], dq, qo.xs + (int64_t)t * nsc + g, lane & 15);
            else
                quant_group4_v(v[i], dq, qo.xs + (int64_t)t * nsc + g * (kGroup / 32) + (lane & 15) / 4, lane & 15);
        }
    }
}

// One token's routing on one wave64 (every wave of the workgroup calls it once: it holds
// workgroup barriers).  Lane l holds experts l, l+64, ... (EPL per lane).  Selection runs on
// 64-bit keys (order-preserving float bits << 32 | ~id): the wave maximum is the largest
// value with the lowest id, which is exactly "descending score, ties to the lower id".
// s_wave is the wave's LDS: E scores, then k selected ids, logits and per-expert scales.
// The logits, the per-expert scales and the activation row's first 32 groups are requested
// together at the start, so the row's loads are in flight during the selection.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, const RouteCfg& c,
                                            const float* __restrict__ pe_scale, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, const QuantOut& qo, int t, float* s_wave) {
    const int lane = threadIdx.x & 63;
    const int E = c.E, k = c.k;
    float* s_score = s_wave;
    int* s_sel = reinterpret_cast<int*>(s_score + E);
    float* s_sell = reinterpret_cast<float*>(s_sel + k);
    float* s_selp = s_sell + k;
    const bool active = t < c.T;

    float lg[EPL], sc[EPL], pe[EPL];
    uint32_t avail = 0;   // bit i: expert lane + 64 i exists and is still selectable
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const bool ok = active && e < E;
        lg[i] = ok ? logits[(int64_t)t * E + e] : -INFINITY;
        pe[i] = (ok && pe_scale) ? pe_scale[e] : 1.0f;
        if (ok) avail |= 1u << i;
    }
    const bool quant = active && qo.x != nullptr;
    uint4 xv[8];
    if (quant) xrow_load(qo, t, 0, lane, xv);

    // scores
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, lg[i]);
    mx = wave_max(mx);
    float sum = 0.f;
    if (c.scoring == 0) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            sc[i] = (avail >> i & 1) ? expf(lg[i] - mx) : 0.f;
            sum += sc[i];
        }
        sum = wave_sum(sum);
#pragma unroll
        for (int i = 0; i < EPL; ++i) sc[i] = sc[i] / sum;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) sc[i] = 1.0f / (1.0f + expf(-lg[i]));
    }

    // group-limited selection: lane g < G scores group g over its contiguous experts
    if (c.G > 1) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E) s_score[e] = (c.mode == 0) ? lg[i] : sc[i];
        }
        __syncthreads();
        const int per = E / c.G;
        uint64_t gkey = 0;
        if (lane < c.G) {
            float a = -INFINITY, b = -INFINITY;   // two largest in the group
            for (int j = 0; j < per; ++j) {
                const float v = s_score[lane * per + j];
                if (v > a) { b = a; a = v; } else if (v > b) { b = v; }
            }
            // mode 0 ranks groups by their largest logit (same order as the largest score)
            const float gs = (c.mode == 0) ? a : a + b;
            gkey = ((uint64_t)ordered_bits(gs) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)lane);
        }
        uint64_t keep = 0;   // bitmask over groups
        for (int j = 0; j < c.k_group; ++j) {
            const uint64_t best = wave_max_u64(gkey);
            if (best == 0) break;                       // inactive wave
            const int g = (int)(0xFFFFFFFFu - (uint32_t)best);
            keep |= 1ull << g;
            if (lane == g) gkey = 0;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((keep >> (e / per)) & 1ull)) avail &= ~(1u << i);
        }
    }

    // top-k by logit
    for (int j = 0; j < k; ++j) {
        uint64_t key = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (avail >> i & 1) {
                const uint64_t kk = ((uint64_t)ordered_bits(lg[i]) << 32) |
                                    (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i));
                key = kk > key ? kk : key;
            }
        }
        key = wave_max_u64(key);
        const int id = (int)(0xFFFFFFFFu - (uint32_t)key);
        if (key != 0 && lane == (id & 63)) {     // the owner lane records the winner
            avail &= ~(1u << (id >> 6));
            s_sel[j] = id;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (id >> 6)) {
                    s_sell[j] = lg[i];
                    s_selp[j] = pe[i];
                }
        }
    }
    __syncthreads();

    // weights of the selected experts
    // softmax, not renormalised: p(id) = exp(l - max) / sum over all experts
    // softmax renormalised / prelude: exp(l - lmax_sel) / sum over the selected
    // sigmoid: s(id) / sum over the selected
    const float lsel0 = s_sell[0];   // the largest selected logit
    float part = 0.f;
    for (int j = lane; j < k; j += 64) {
        const float l = s_sell[j];
        float v;
        if (c.scoring == 1) v = 1.0f / (1.0f + expf(-l));
        else if (c.renormalize || c.prelude) v = expf(l - lsel0);
        else v = expf(l - mx) / sum;
        part += v;
    }
    const float denom = wave_sum(part);
    const bool normalise = c.scoring == 1 || c.renormalize || c.prelude;
    if (active) {
        for (int j = lane; j < k; j += 64) {
            const float l = s_sell[j];
            const int id = s_sel[j];
            float v;
            if (c.scoring == 1) v = 1.0f / (1.0f + expf(-l));
            else if (c.renormalize || c.prelude) v = expf(l - lsel0);
            else v = expf(l - mx) / sum;
            if (normalise) v = v / denom;
            if (c.prelude && pe_scale) v *= s_selp[j];
            v *= c.rsf;
            ids[(int64_t)t * c.ld + j] = id;
            wts[(int64_t)t * c.ld + j] = v;
        }
        if (c.shared_id >= 0 && lane == 0) {   // the shared expert, unweighted
            ids[(int64_t)t * c.ld + k] = c.shared_id;
            wts[(int64_t)t * c.ld + k] = 1.0f;
        }
        if (quant) {
            const int ngc = qo.H / kGroup;
            for (int g0 = 0; g0 < ngc; g0 += 32) {
                if (g0 > 0) xrow_load(qo, t, g0, lane, xv);
                xrow_quant(qo, t, g0, lane, xv);
            }
        }
    }
}

// Top-k routing over many workgroups: one wave per token, one token per workgroup (spreads a
// decode batch's tokens over as many CUs as it has tokens).
template <int EPL>
__global__ __launch_bounds__(64) void k_route(const float* __restrict__ logits, RouteCfg c,
                                               const float* __restrict__ pe_scale, int32_t* __restrict__ ids,
                                               float* __restrict__ wts, QuantOut qo) {
    extern __shared__ float s_route[];
    route_token<EPL>(logits, c, pe_scale, ids, wts, qo, blockIdx.x, s_route);
}

hipError_t launch_route(const float* logits, const RouteCfg& c, const float* pe_scale, int32_t* ids,
                        float* weights, hipStream_t st, QuantOut qo) {
    const dim3 grid((unsigned)c.T), block(64);
    const size_t lds = (size_t)(c.E + 3 * c.k) * 4;
    const int epl = (int)ceil_div(c.E, 64);
    if (epl <= 1) hipLaunchKernelGGL(k_route<1>, grid, block, lds, st, logits, c, pe_scale, ids, weights, qo);
    else if (epl <= 2) hipLaunchKernelGGL(k_route<2>, grid, block, lds, st, logits, c, pe_scale, ids, weights, qo);
    else if (epl <= 4) hipLaunchKernelGGL(k_route<4>, grid, block, lds, st, logits, c, pe_scale, ids, weights, qo);
    else if (epl <= 8) hipLaunchKernelGGL(k_route<8>, grid, block, lds, st, logits, c, pe_scale, ids, weights, qo);
    else hipLaunchKernelGGL(k_route<16>, grid, block, lds, st, logits, c, pe_scale, ids, weights, qo);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Dispatch.  The flat assignments are cut into chunks of kScatterChunk; each chunk's
// per-expert counts are scanned over chunks (per expert) and over experts, and each
// assignment lands at offsets[e] + (earlier chunks' count of e) + (its rank among the
// equal ids before it in its chunk).  Ranks come from wave ballots, no atomics on the
// positions, so the result is the stable counting sort exactly.

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int A, int E,
                                              int32_t* __restrict__ chunk_counts) {
    extern __shared__ int s_cnt[];
    for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kScatterChunk;
    for (int i = threadIdx.x; i < kScatterChunk; i += 256) {
        const int64_t f = base + i;
        if (f < A) {
            const int e = ids[f];
            if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);   // ids outside [0, E) are dropped
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// Inclusive scan over a workgroup of 1024 threads.
__device__ int block_inclusive_scan_1024(int v, int* s_tmp /*[16]*/) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_tmp[wv] = v;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wv; ++w) add += s_tmp[w];
    __syncthreads();
    return v + add;
}

// One workgroup: chunk_counts -> per-chunk bases (offsets[e] + earlier chunks), counts, offsets.
// gpe = 1024 / E' threads share an expert (E' = E rounded up to a power of two); thread
// (g, e) owns the contiguous chunks [g * cpt, (g + 1) * cpt), so its loads are independent
// of one another; the per-thread sums are scanned across g, then the expert totals across e.
// With `tiles`, it also writes the GEMM tile list (expert order, BM rows per tile) and, with
// `pairs`, the pair list of the 256-row items ({first tile, expert, first sorted row, valid
// rows} per pair), as k_tiles / k_pairs do.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ cc, int nchunks, int E, int Ep,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int BM,
                                               int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                               int4* __restrict__ pairs, int32_t* __restrict__ npairs) {
    __shared__ int s_tmp[16];
    __shared__ int s_part[1024];
    const int gpe = 1024 / Ep, e = threadIdx.x % Ep, g = threadIdx.x / Ep;
    const int cpt = (nchunks + gpe - 1) / gpe, c0 = g * cpt, c1 = min(nchunks, c0 + cpt);
    const bool act = e < E;
    int sum = 0;
    if (act) {
        for (int c = c0; c < c1; c += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = c + u < c1 ? cc[(int64_t)(c + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) sum += v[u];
        }
    }
    s_part[threadIdx.x] = sum;
    __syncthreads();
    int before = 0, run = 0;   // this thread's chunks start after `before` of expert e's ids
    for (int h = 0; h < gpe; ++h) {
        const int x = s_part[h * Ep + e];
        before += h < g ? x : 0;
        run += x;
    }
    // expert offsets: scan of the totals over e (one contributor per expert: g == 0)
    const int incl = block_inclusive_scan_1024(act && g == 0 ? run : 0, s_tmp);
    __syncthreads();
    if (g == 0) s_part[e] = incl - (act ? run : 0);
    __syncthreads();
    const int off = s_part[e];
    if (act) {
        if (g == 0) {
            counts[e] = run;
            offsets[e] = off;
            if (e == E - 1) offsets[E] = off + run;
        }
        int p = off + before;
        for (int c = c0; c < c1; c += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = c + u < c1 ? cc[(int64_t)(c + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c + u < c1) cc[(int64_t)(c + u) * E + e] = p;
                p += v[u];
            }
        }
    }
    if (tiles) {   // uniform: every thread takes part in the scans
        const bool own = act && g == 0;   // thread e holds expert e's total
        const int nt = own ? (run + BM - 1) / BM : 0;
        const int it = block_inclusive_scan_1024(nt, s_tmp);
        const int np = own && pairs ? (run + 2 * BM - 1) / (2 * BM) : 0;
        const int ip = block_inclusive_scan_1024(np, s_tmp);
        if (own) {
            const int t0 = it - nt, p0 = ip - np;
            for (int i = 0; i < nt; ++i) tiles[t0 + i] = make_int2(e, i * BM);
            for (int i = 0; i < np; ++i)
                pairs[p0 + i] = make_int4(t0 + 2 * i, e, off + 2 * BM * i, min(2 * BM, run - 2 * BM * i));
            if (e == E - 1) {
                *ntiles = it;
                if (pairs) *npairs = ip;
            }
        }
    }
}

// The chunk's ranking and stores, given its per-expert bases base(e) (offsets[e] plus the
// earlier chunks' counts of e).  s_wc: [4][E] ints of LDS.
template <typename BaseFn>
__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ ids, int A, int E, int nbits, BaseFn base,
                                              int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
                                              int* s_wc) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4 * E; i += 256) s_wc[i] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    const int64_t b0 = (int64_t)blockIdx.x * kScatterChunk + wv * (kScatterChunk / 4);
    int rank[kScatterChunk / 256], eid[kScatterChunk / 256];
#pragma unroll
    for (int r = 0; r < kScatterChunk / 256; ++r) {
        const int64_t f = b0 + r * 64 + lane;
        int e = f < A ? ids[f] : 0;
        const bool valid = f < A && (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        if (f < A && !valid) assign_pos[f] = -1;   // dropped assignment
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        int prev = 0;
        if (valid) prev = s_wc[wv * E + e];
        const int before = __popcll(peers & lt);
        rank[r] = prev + before;
        eid[r] = valid ? e : -1;
        if (valid && before == 0) s_wc[wv * E + e] = prev + __popcll(peers);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const int a = s_wc[e], b = s_wc[E + e], c2 = s_wc[2 * E + e];
        s_wc[e] = 0;
        s_wc[E + e] = a;
        s_wc[2 * E + e] = a + b;
        s_wc[3 * E + e] = a + b + c2;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kScatterChunk / 256; ++r) {
        const int e = eid[r];
        if (e >= 0) {
            const int64_t f = b0 + r * 64 + lane;
            const int pos = base(e) + s_wc[wv * E + e] + rank[r];
            sorted_assign[pos] = (int32_t)f;
            assign_pos[f] = pos;
        }
    }
}

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ ids, int A, int E, int nbits,
                                                 const int32_t* __restrict__ chunk_base,
                                                 int32_t* __restrict__ sorted_assign,
                                                 int32_t* __restrict__ assign_pos) {
    extern __shared__ int s_wc[];   // [4][E] per-wave running counts, then per-wave bases
    const int32_t* cb = chunk_base + (int64_t)blockIdx.x * E;
    scatter_chunk(ids, A, E, nbits, [&](int e) { return cb[e]; }, sorted_assign, assign_pos, s_wc);
}

// Exclusive scan over a workgroup of 256 threads; *total receives the sum (every thread).
__device__ int block_exclusive_scan_256(int v, int* s_tmp /*[4]*/, int* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(x, o);
        if (lane >= o) x += u;
    }
    if (lane == 63) s_tmp[wv] = x;
    __syncthreads();
    int add = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        add += w < wv ? s_tmp[w] : 0;
        all += s_tmp[w];
    }
    __syncthreads();
    *total = all;
    return add + x - v;
}

// Scatter that forms its own bases, for launches where every chunk's counts are few
// (at most kScanInScatterMaxChunks chunks and nchunks * E <= kScanInScatterMax): each workgroup (one chunk) sums all chunks' counts per
// expert, scans the totals over the experts (offsets) and adds the earlier chunks' counts,
// which is what k_scan writes for it; workgroup 0 also writes counts, offsets and the tile /
// pair lists.  One launch instead of k_scan + k_scatter.
constexpr int kScanInScatterMax = 32768, kScanInScatterMaxChunks = 256;
constexpr int kSisEpt = MOE_DISPATCH_MAX_E / 256;   // experts per thread
__global__ __launch_bounds__(256) void k_scatter_scan(const int32_t* __restrict__ ids, int A, int E, int nbits,
                                                      const int32_t* __restrict__ cc, int nchunks,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_assign,
                                                      int32_t* __restrict__ assign_pos, int BM,
                                                      int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                      int4* __restrict__ pairs, int32_t* __restrict__ npairs) {
    extern __shared__ int s_dyn[];   // [4][E] for the ranking, then [E] chunk bases
    int* s_cb = s_dyn + 4 * E;
    __shared__ int s_tmp[4];
    const int tid = threadIdx.x, c0 = blockIdx.x;
    int tot[kSisEpt], bef[kSisEpt];
#pragma unroll
    for (int q = 0; q < kSisEpt; ++q) {   // expert e = tid + 256 q
        const int e = tid + 256 * q;
        int t = 0, b = 0;
        if (e < E) {
            for (int c = 0; c < nchunks; c += 32) {   // 32 loads in flight
                int v[32];
#pragma unroll
                for (int u = 0; u < 32; ++u) v[u] = c + u < nchunks ? cc[(int64_t)(c + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 32; ++u) {
                    t += v[u];
                    b += c + u < c0 ? v[u] : 0;
                }
            }
        }
        tot[q] = t;
        bef[q] = b;
    }
    // expert offsets: exclusive scan of the totals in expert order (q outer, thread inner)
    int run = 0, off[kSisEpt];
#pragma unroll
    for (int q = 0; q < kSisEpt; ++q) {
        if (256 * q >= E) {   // uniform
            off[q] = run;
            continue;
        }
        int all;
        off[q] = run + block_exclusive_scan_256(tot[q], s_tmp, &all);
        run += all;
    }
#pragma unroll
    for (int q = 0; q < kSisEpt; ++q) {
        const int e = tid + 256 * q;
        if (e < E) s_cb[e] = off[q] + bef[q];
    }
    if (c0 == 0) {   // uniform: counts, offsets, tile and pair lists (as k_scan writes them)
#pragma unroll
        for (int q = 0; q < kSisEpt; ++q) {
            const int e = tid + 256 * q;
            if (e < E) {
                counts[e] = tot[q];
                offsets[e] = off[q];
                if (e == E - 1) offsets[E] = off[q] + tot[q];
            }
        }
        if (tiles) {
            int trun = 0, prun = 0;
#pragma unroll
            for (int q = 0; q < kSisEpt; ++q) {
                if (256 * q >= E) continue;   // uniform
                const int e = tid + 256 * q;
                const int nt = e < E ? (tot[q] + BM - 1) / BM : 0;
                const int np = e < E && pairs ? (tot[q] + 2 * BM - 1) / (2 * BM) : 0;
                int allt, allp;
                const int t0 = trun + block_exclusive_scan_256(nt, s_tmp, &allt);
                const int p0 = prun + block_exclusive_scan_256(np, s_tmp, &allp);
                for (int i = 0; i < nt; ++i) tiles[t0 + i] = make_int2(e, i * BM);
                for (int i = 0; i < np; ++i)
                    pairs[p0 + i] = make_int4(t0 + 2 * i, e, off[q] + 2 * BM * i, min(2 * BM, tot[q] - 2 * BM * i));
                trun += allt;
                prun += allp;
            }
            if (tid == 0) {
                *ntiles = trun;
                if (pairs) *npairs = prun;
            }
        }
    }
    __syncthreads();   // s_cb complete before the ranking uses it
    scatter_chunk(ids, A, E, nbits, [&](int e) { return s_cb[e]; }, sorted_assign, assign_pos, s_dyn);
}

// Single-workgroup dispatch for small A (8 waves).  Wave w owns the contiguous segment
// [w*seg, (w+1)*seg) of the flat assignments: pass 1 counts ids per wave, the bases
// offsets[e] + (earlier waves' count of e) follow from one scan, pass 2 ranks equal ids
// inside each 64-wide round with ballots and keeps per-wave running positions.  With
// tiles != nullptr it also writes the GEMM tile list of BM-row tiles.
constexpr int kOneWaves = 8;

__global__ __launch_bounds__(64 * kOneWaves) void k_dispatch_one(const int32_t* __restrict__ ids, int A, int E,
                                                                  int nbits, int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_assign,
                                                                  int32_t* __restrict__ assign_pos, int BM,
                                                                  int2* __restrict__ tiles,
                                                                  int32_t* __restrict__ ntiles) {
    __shared__ int s_w[kOneWaves][MOE_DISPATCH_MAX_E];   // per-wave counts, then per-wave positions
    __shared__ int s_tmp[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < kOneWaves * E; i += 64 * kOneWaves) s_w[i / E][i % E] = 0;
    __syncthreads();
    const int seg = (int)ceil_div(A, kOneWaves);
    const int b0 = wv * seg, b1 = min(A, b0 + seg);
    // the lane's ids stay in registers for the second pass (seg <= 64 * kOneRounds)
    constexpr int kOneRounds = kDispatchOneMaxA / kOneWaves / 64;
    int ev[kOneRounds];
#pragma unroll
    for (int r = 0; r < kOneRounds; ++r) {
        const int f = b0 + 64 * r + lane;
        ev[r] = f < b1 ? ids[f] : -1;
    }
#pragma unroll
    for (int r = 0; r < kOneRounds; ++r)
        if ((unsigned)ev[r] < (unsigned)E) atomicAdd(&s_w[wv][ev[r]], 1);
    __syncthreads();
    // per expert: total count, then the exclusive scan over experts and the per-wave bases
    int tot[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = tid + q * 64 * kOneWaves;
        if (e < E)
            for (int w = 0; w < kOneWaves; ++w) tot[q] += s_w[w][e];
    }
    // scan of tot over e = tid (q=0) then e = tid + 512 (q=1)
    int run_base = 0;
    int excl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int v = tot[q];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(v, o);
            if (lane >= o) v += u;
        }
        if (lane == 63) s_tmp[wv] = v;
        __syncthreads();
        int add = 0, all = 0;
        for (int w = 0; w < kOneWaves; ++w) {
            if (w < wv) add += s_tmp[w];
            all += s_tmp[w];
        }
        __syncthreads();
        excl[q] = run_base + add + v - tot[q];
        run_base += all;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = tid + q * 64 * kOneWaves;
        if (e < E) {
            counts[e] = tot[q];
            offsets[e] = excl[q];
            if (e == E - 1) offsets[E] = excl[q] + tot[q];
            int p = excl[q];
            for (int w = 0; w < kOneWaves; ++w) {
                const int c = s_w[w][e];
                s_w[w][e] = p;
                p += c;
            }
        }
    }
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
#pragma unroll
    for (int r = 0; r < kOneRounds; ++r) {
        const int f0 = b0 + 64 * r;
        if (f0 >= b1) break;   // wave-uniform
        const int f = f0 + lane;
        int e = f < b1 ? ev[r] : 0;
        const bool valid = f < b1 && (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        if (f < b1 && !valid) assign_pos[f] = -1;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        int base = 0;
        if (valid) base = s_w[wv][e];
        const int before = __popcll(peers & lt);
        if (valid) {
            const int pos = base + before;
            sorted_assign[pos] = f;
            assign_pos[f] = pos;
            if (before == 0) s_w[wv][e] = base + __popcll(peers);
        }
    }
    if (tiles) {
        // tile list: BM-row tiles per expert in expert order (counts are in global memory now)
        __syncthreads();
        int n[2], st[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + q * 64 * kOneWaves;
            n[q] = e < E ? (tot[q] + BM - 1) / BM : 0;
        }
        int base2 = 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            int v = n[q];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(v, o);
                if (lane >= o) v += u;
            }
            if (lane == 63) s_tmp[wv] = v;
            __syncthreads();
            int add = 0, all = 0;
            for (int w = 0; w < kOneWaves; ++w) {
                if (w < wv) add += s_tmp[w];
                all += s_tmp[w];
            }
            __syncthreads();
            st[q] = base2 + add + v - n[q];
            base2 += all;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + q * 64 * kOneWaves;
            for (int i = 0; i < n[q]; ++i) tiles[st[q] + i] = make_int2(e, i * BM);
        }
        if (tid == 0) *ntiles = base2;
    }
}

hipError_t launch_dispatch(const int32_t* ids, int A, int E, int32_t* chunk_ws, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, hipStream_t st,
                           int BM, int2* tiles, int32_t* ntiles, int4* pairs, int32_t* npairs) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    if (A <= kDispatchOneMaxA) {
        hipLaunchKernelGGL(k_dispatch_one, dim3(1), dim3(64 * kOneWaves), 0, st, ids, A, E, nbits, counts, offsets,
                           sorted_assign, assign_pos, BM, tiles, ntiles);
        if (pairs) return launch_pairs(counts, offsets, E, pairs, npairs, st);
        return hipGetLastError();
    }
    const int nchunks = (int)ceil_div(A, kScatterChunk);
    hipLaunchKernelGGL(k_hist, dim3(nchunks), dim3(256), (size_t)E * 4, st, ids, A, E, chunk_ws);
    if (nchunks <= kScanInScatterMaxChunks && (int64_t)nchunks * E <= kScanInScatterMax) {
        hipLaunchKernelGGL(k_scatter_scan, dim3(nchunks), dim3(256), (size_t)5 * E * 4, st, ids, A, E, nbits, chunk_ws,
                           nchunks, counts, offsets, sorted_assign, assign_pos, BM, tiles, ntiles,
                           tiles ? pairs : nullptr, npairs);
        return hipGetLastError();
    }
    int Ep = 1;
    while (Ep < E) Ep <<= 1;
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, chunk_ws, nchunks, E, Ep, counts, offsets, BM, tiles, ntiles,
                       tiles ? pairs : nullptr, npairs);
    hipLaunchKernelGGL(k_scatter, dim3(nchunks), dim3(256), (size_t)4 * E * 4, st, ids, A, E, nbits, chunk_ws,
                       sorted_assign, assign_pos);
    return hipGetLastError();
}

}  // namespace moe
