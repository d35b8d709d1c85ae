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

// ----------------------------------------------------------------------------------------
// Gate prelude: logits[t, e] = sum_h ((x[t,h] * r_t) * norm_w[h]) * W_r[e, h] with
// r_t = 1 / sqrt(mean_h x^2 + eps).  Workgroup (t, expert chunk of 32): the token's
// normalised row is built in LDS, then each wave takes 8 experts.
constexpr int kPreludeExperts = 32;

__global__ __launch_bounds__(256) void k_gate_prelude(const uint16_t* __restrict__ x, int H, int E,
                                                      const float* __restrict__ norm_w,
                                                      const float* __restrict__ router_w, float eps,
                                                      float* __restrict__ logits) {
    extern __shared__ float s_xn[];   // [H]
    __shared__ float s_part[4];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint16_t* xr = x + (int64_t)t * H;
    float ss = 0.f;
    for (int h = tid; h < H; h += 256) {
        const float v = bf16_to_f32(xr[h]);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) s_part[wv] = ss;
    __syncthreads();
    const float mean = (s_part[0] + s_part[1] + s_part[2] + s_part[3]) / (float)H;
    const float r = 1.0f / sqrtf(mean + eps);
    for (int h = tid; h < H; h += 256) s_xn[h] = (bf16_to_f32(xr[h]) * r) * norm_w[h];
    __syncthreads();
    const int e0 = blockIdx.y * kPreludeExperts;
    for (int i = 0; i < kPreludeExperts / 4; ++i) {
        const int e = e0 + wv * (kPreludeExperts / 4) + i;
        if (e >= E) break;
        const float* wr = router_w + (int64_t)e * H;
        float acc = 0.f;
        for (int h = lane; h < H; h += 64) acc = fmaf(s_xn[h], wr[h], acc);
        acc = wave_sum(acc);
        if (lane == 0) logits[(int64_t)t * E + e] = acc;
    }
}

hipError_t launch_gate_prelude(const uint16_t* x, int T, int H, int E, const float* norm_w,
                               const float* router_w, float eps, float* logits, hipStream_t st) {
    dim3 grid(T, (unsigned)ceil_div(E, kPreludeExperts));
    hipLaunchKernelGGL(k_gate_prelude, grid, dim3(256), (size_t)H * sizeof(float), st, x, H, E, norm_w,
                       router_w, eps, logits);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Top-k routing: one wave64 per token, 4 tokens per workgroup.  Lane l holds experts
// l, l+64, ... (EPL per lane).  Selection runs on 64-bit keys
// (order-preserving float bits << 32 | ~id): the wave maximum is the largest value with
// the lowest id, which is exactly "descending score, ties to the lower id".

__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);   // +0 and -0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, o);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o);
        const uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, RouteCfg c,
                                               const float* __restrict__ pe_scale, int32_t* __restrict__ ids,
                                               float* __restrict__ wts) {
    extern __shared__ unsigned char s_raw[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    const int E = c.E, k = c.k;
    // per wave: scores [E] float, selected ids [k] int, selected logits [k] float
    float* s_score = reinterpret_cast<float*>(s_raw) + (size_t)wv * (E + 2 * k);
    int* s_sel = reinterpret_cast<int*>(s_score + E);
    float* s_sell = reinterpret_cast<float*>(s_sel + k);
    const bool active = t < c.T;

    float lg[EPL], sc[EPL];
    uint32_t avail = 0;   // bit i: expert lane + 64 i exists and is still selectable
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const bool ok = active && e < E;
        lg[i] = ok ? logits[(int64_t)t * E + e] : -INFINITY;
        if (ok) avail |= 1u << i;
    }
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
                if (i == (id >> 6)) s_sell[j] = lg[i];
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
            if (c.prelude && pe_scale) v *= pe_scale[id];
            v *= c.rsf;
            ids[(int64_t)t * k + j] = id;
            wts[(int64_t)t * k + j] = v;
        }
    }
}

hipError_t launch_route(const float* logits, const RouteCfg& c, const float* pe_scale, int32_t* ids,
                        float* weights, hipStream_t st) {
    const dim3 grid((unsigned)ceil_div(c.T, 4)), block(256);
    const size_t lds = (size_t)4 * (c.E + 2 * c.k) * 4;
    const int epl = (int)ceil_div(c.E, 64);
    if (epl <= 1) hipLaunchKernelGGL(k_route<1>, grid, block, lds, st, logits, c, pe_scale, ids, weights);
    else if (epl <= 2) hipLaunchKernelGGL(k_route<2>, grid, block, lds, st, logits, c, pe_scale, ids, weights);
    else if (epl <= 4) hipLaunchKernelGGL(k_route<4>, grid, block, lds, st, logits, c, pe_scale, ids, weights);
    else if (epl <= 8) hipLaunchKernelGGL(k_route<8>, grid, block, lds, st, logits, c, pe_scale, ids, weights);
    else hipLaunchKernelGGL(k_route<16>, grid, block, lds, st, logits, c, pe_scale, ids, weights);
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
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ cc, int nchunks, int E,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
    __shared__ int s_tmp[16];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            const int v = cc[(int64_t)c * E + e];
            cc[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    const int incl = block_inclusive_scan_1024(e < E ? run : 0, s_tmp);
    const int off = incl - (e < E ? run : 0);
    if (e < E) {
        counts[e] = run;
        offsets[e] = off;
        if (e == E - 1) offsets[E] = incl;
        for (int c = 0; c < nchunks; ++c) cc[(int64_t)c * E + e] += off;
    }
}

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ ids, int A, int E, int nbits,
                                                 const int32_t* __restrict__ chunk_base,
                                                 int32_t* __restrict__ sorted_assign,
                                                 int32_t* __restrict__ assign_pos) {
    extern __shared__ int s_wc[];   // [4][E] per-wave running counts, then per-wave bases
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 4 * E; i += 256) s_wc[i] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    const int64_t base = (int64_t)blockIdx.x * kScatterChunk + wv * (kScatterChunk / 4);
    int rank[kScatterChunk / 256], eid[kScatterChunk / 256];
#pragma unroll
    for (int r = 0; r < kScatterChunk / 256; ++r) {
        const int64_t f = base + r * 64 + lane;
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
            const int64_t f = base + r * 64 + lane;
            const int pos = chunk_base[(int64_t)blockIdx.x * E + e] + s_wc[wv * E + e] + rank[r];
            sorted_assign[pos] = (int32_t)f;
            assign_pos[f] = pos;
        }
    }
}

hipError_t launch_dispatch(const int32_t* ids, int A, int E, int32_t* chunk_ws, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, hipStream_t st) {
    const int nchunks = (int)ceil_div(A, kScatterChunk);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipLaunchKernelGGL(k_hist, dim3(nchunks), dim3(256), (size_t)E * 4, st, ids, A, E, chunk_ws);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, chunk_ws, nchunks, E, counts, offsets);
    hipLaunchKernelGGL(k_scatter, dim3(nchunks), dim3(256), (size_t)4 * E * 4, st, ids, A, E, nbits, chunk_ws,
                       sorted_assign, assign_pos);
    return hipGetLastError();
}

}  // namespace moe
