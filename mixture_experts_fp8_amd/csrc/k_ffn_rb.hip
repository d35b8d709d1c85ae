// Persistent down GEMM of the grouped expert FFN for 128-row expert tiles (gfx950).
//
// The down products of run_fp8_grouped_w8a8 (metrale "fp8_grouped_tc_w8a8.rs") on the
// re-quantised SwiGLU output hq: expert_out[row] = dequant(hq[row]) . dequant(w2[e]), on
// v_mfma_scale_f32_16x16x128_f8f6f4 with the per-(row, 128) activation scales and the
// 128x128 weight-block scales as the instruction's UE8M0 operand scales.
//
// Work: an item is (MT consecutive 128-row tiles of one expert, 256 output columns).  One
// workgroup of 8 waves (two per SIMD) runs on each CU and walks its share of the item list;
// wave w owns 32 of the 256 columns for all 128 MT rows (8 MT x 2 fragments), so no two
// waves load the same weights.  MT = 2 halves the weight bytes per flop, but its 128
// accumulator registers per lane leave room for only one K block in flight (P = 1), and that
// measured slower than MT = 1 with four blocks in flight, the default.
//
// Operand streams run over one flattened sequence of K blocks covering all of the
// workgroup's items, so the next item's loads are in flight during the current item's
// epilogue (the output stores):
//   * A (the item's hq tile slots, 16 KB per tile and K block, already in matrix-core order)
//     goes global -> LDS by the LDS-DMA form of the buffer load into a ring of P + 1 stages,
//     P blocks ahead;
//   * B (pre-packed weights, 4 KB per wave per K block) goes straight into a register ring,
//     P blocks ahead, two 1 KB coalesced loads per fragment;
//   * scales: the 8 A-row scales a lane needs per K block are one 8-byte load from hs, kept
//     in [tile][kb][row % 16][row / 16] order, picked per fragment by the instruction's scale
//     byte select; the weight-block scale is one uniform dword load from a per-call
//     [expert][column block][kb] table (scale in byte 0).  No loaded value is touched before
//     the matrix-core instruction that consumes it, so no load has to land early.
// Each K block: wait for this thread's DMA of the block, barrier (everyone's DMA landed;
// everyone is done with the stage about to be refilled), DMA block + P, B and scale loads of
// block + P, then the 8 MT A fragments from LDS and 16 MT matrix-core instructions per wave.
#include "moe_common.h"
#include "moe_internal.h"
#include "work_items.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace moe {

constexpr int kRbBM = 128;                    // rows per tile
constexpr int kRbWaves = 8;
constexpr int kRbThreads = 64 * kRbWaves;     // two waves per SIMD
constexpr int kRbStage = kRbBM * kGroup;      // A bytes per K block (8 fragments)
constexpr int kRb2MaxItems = 256;             // items per workgroup (LDS item table)
constexpr int kRbXcds = 8;

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef int v4i_rb __attribute__((ext_vector_type(4)));

// Buffer descriptor as four scalar dwords (for the LDS-DMA asm operand).
__device__ __forceinline__ v4i_rb rb_srd(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    v4i_rb r;
    r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)b);
    r[1] = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu);
    r[2] = (int)__builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t rb_lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p);
}

// 16 bytes per lane from the buffer at voff + soff into LDS at m0base + 16 * lane.  The
// compiler does not see this load: completion is awaited explicitly with rb_wait_vm.
__device__ __forceinline__ void rb_dma16(const v4i_rb& srd, uint32_t m0base, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0base), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void rb_wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ v8i rb_lds_frag(const uint8_t* base, int lane) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 1024 + lane * 16);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// One 2 KB packed weight operand (lane l: 16 bytes at soff + 16 l and at soff + 1024 + 16 l),
// default cache policy: the workgroups running together on an XCD read the same weight
// columns, so these loads should stay in its L2.
__device__ __forceinline__ v8i rb_frag(rsrc_t r, uint32_t lane16, uint32_t soff) {
    const v4i_rb lo = __builtin_amdgcn_raw_buffer_load_b128(r, lane16, soff, 0);
    const v4i_rb hi = __builtin_amdgcn_raw_buffer_load_b128(r, lane16, soff + 1024, 0);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// f(integral_constant<0>), f(integral_constant<1>), ... in order
template <typename F, int... Is>
__device__ __forceinline__ void rb_static_for(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}

// Matrix-core product with the A scale taken from byte SEL of sa (B scale: byte 0 of sb).
template <int SEL>
__device__ __forceinline__ v4f rb_mfma(v8i a, v8i b, v4f acc, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, SEL, sa, 0, sb);
}
__device__ __forceinline__ v4f rb_mfma_sel(int sel, v8i a, v8i b, v4f acc, int sa, int sb) {
    switch (sel) {
        case 0: return rb_mfma<0>(a, b, acc, sa, sb);
        case 1: return rb_mfma<1>(a, b, acc, sa, sb);
        case 2: return rb_mfma<2>(a, b, acc, sa, sb);
        default: return rb_mfma<3>(a, b, acc, sa, sb);
    }
}

// ----------------------------------------------------------------------------------------
// Per-call table of the down GEMM's weight-block scales as dwords in [expert][column block][kb]
// order, so a wave's scale for a K block is one aligned uniform load whose byte 0 feeds the
// matrix-core instruction as is.
__global__ __launch_bounds__(256) void k_rb_scales(const uint8_t* __restrict__ w2s, int E, int KB, int NBS,
                                                   uint32_t* __restrict__ bs) {
    const int64_t n = (int64_t)E * KB * NBS, per = (int64_t)NBS * KB;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < n; o += (int64_t)gridDim.x * 256) {
        const int64_t e = o / per, rem = o - e * per;
        const int c = (int)(rem / KB), kb = (int)(rem - (int64_t)c * KB);
        bs[o] = w2s[(e * KB + kb) * NBS + c];
    }
}

// ----------------------------------------------------------------------------------------
struct Rb2Args {
    const uint8_t* hq;          // [tile][8][I/128][2 KB]
    const uint8_t* hs;          // [tile][I/128][16][8]
    const uint32_t* bs;         // [E][H/128][I/128]
    int H, I, E, ntiles_max;
    const int2* tiles;
    const int32_t* ntiles;
    const int32_t* counts;
    const int32_t* offsets;
    const uint8_t* w2p;         // packed [E][H/16][I/128][2 KB]
    void* out;                  // [A, H] fp32 or bf16, expert-sorted rows
    int out_bf16;
    int ord;                    // 1: super-tile work order (ord_item), 0: column blocks per tile group
    const float* b2;            // optional down bias [E, H]
};

template <int P, int MT>
__global__ __launch_bounds__(kRbThreads, 1) void k_gemm2_rb(Rb2Args a) {
    constexpr int R = P + 1, NST = P + 1, MF = 8 * MT;   // MF 16-row fragments per item
    // per K block and thread: 2 MT DMA + 4 B + MT A-scale + 1 B-scale
    constexpr int kOpsPerStep = 2 * MT + 4 + MT + 1;
    constexpr int kOpsAfter = (kOpsPerStep - 2 * MT) + (P - 1) * kOpsPerStep;
    static_assert(kOpsAfter <= 63, "vmcnt range");

    __shared__ __align__(16) uint8_t ring[NST * MT * kRbStage];
    __shared__ int4 s_it[kRb2MaxItems];
    __shared__ int s_nv[kRb2MaxItems];

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntiles = __builtin_amdgcn_readfirstlane(*a.ntiles);
    const int ncol = a.H / 256, KB = a.I / kGroup;
    const int NB16 = a.H / 16, NBS = a.H / kGroup;
    __shared__ int s_cnt[kRbWaves];
    ItSched sch;
    sch.n = it_fill_items<MT>(a.ord, ncol, ntiles, a.tiles, a.counts, a.offsets, s_it, s_nv, kRb2MaxItems, s_cnt);
    if (sch.n <= 0) return;
    __syncthreads();
    const int G = sch.n * KB;

    // ---- A stream: the item's hq tile slots (consecutive), 8 MT fragments of 2 KB per K
    // block; piece q of this thread is fragment 4q + wv/2, half wv%2, lane
    const v4i_rb ra = rb_srd(a.hq, (uint32_t)a.ntiles_max * 8 * KB * kFragBytes);
    const uint32_t lds_ring = rb_lds_addr(ring) + wv * 1024;
    const uint32_t apiece = (uint32_t)((wv >> 1) * KB * kFragBytes + (wv & 1) * 1024 + lane * 16);
    int a_i = 0, a_kb = 0;
    uint32_t abase = __builtin_amdgcn_readfirstlane((uint32_t)s_it[0].x * 8 * KB * kFragBytes);
    auto dma_a = [&](int g) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_ring + (g % NST) * (MT * kRbStage));
#pragma unroll
        for (int q = 0; q < 2 * MT; ++q)
            rb_dma16(ra, st + q * 8192, apiece, abase + (uint32_t)(4 * q * KB + a_kb) * kFragBytes);
        const bool wrap = ++a_kb == KB;
        a_kb = wrap ? 0 : a_kb;
        a_i = wrap ? min(a_i + 1, sch.n - 1) : a_i;
        abase = __builtin_amdgcn_readfirstlane((uint32_t)s_it[a_i].x * 8 * KB * kFragBytes);
    };

    rsrc_t rw;
    const rsrc_t rbs = make_rsrc(a.bs, (uint32_t)a.E * NBS * KB * 4);
    const rsrc_t rsa = make_rsrc(a.hs, (uint32_t)a.ntiles_max * KB * kRbBM);
    uint32_t bo[2], sbo, sao;
    int b_i = 0, b_kb = 0;
    auto b_setup = [&](int i) __attribute__((always_inline)) {
        const int4 it = s_it[i];
        const int tile = __builtin_amdgcn_readfirstlane(it.x), col = __builtin_amdgcn_readfirstlane(it.y);
        const int e = __builtin_amdgcn_readfirstlane(it.z);
        rw = make_rsrc(a.w2p + (int64_t)e * NB16 * KB * kFragBytes, (uint32_t)NB16 * KB * kFragBytes);
#pragma unroll
        for (int j = 0; j < 2; ++j) bo[j] = (uint32_t)(col * 16 + wv * 2 + j) * KB * kFragBytes;
        sbo = (uint32_t)((e * NBS + col * 2 + (wv >> 2)) * KB) * 4;
        sao = (uint32_t)tile * KB * kRbBM;
    };
    b_setup(0);
    v8i Bf[R][2];
    v2i_t Sa[R][MT];
    int Sb[R];
    const uint32_t l16 = lane * 16, la8 = (lane & 15) * 8;
    auto load_b = [&](v8i* bf, v2i_t* sa, int& sb) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = rb_frag(rw, l16, bo[j] + b_kb * kFragBytes);
#pragma unroll
        for (int t = 0; t < MT; ++t)   // tile t of the item: its hs block follows the previous one
            sa[t] = __builtin_amdgcn_raw_buffer_load_b64(rsa, la8, sao + (t * KB + b_kb) * kRbBM, 0);
        sb = __builtin_amdgcn_raw_buffer_load_b32(rbs, 0, sbo + b_kb * 4, 0);
        const bool wrap = ++b_kb == KB;
        b_kb = wrap ? 0 : b_kb;
        b_i = wrap ? min(b_i + 1, sch.n - 1) : b_i;
        b_setup(b_i);
    };

    v4f acc[MF][2];
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int g = 0; g < P; ++g) {
        dma_a(g);
        load_b(Bf[g], Sa[g], Sb[g]);
    }

    int c_i = 0, c_kb = 0;
    auto epilogue = [&]() __attribute__((always_inline)) {
        const int4 it = s_it[c_i];
        const int col = __builtin_amdgcn_readfirstlane(it.y), rowbase = __builtin_amdgcn_readfirstlane(it.w);
        const int nvalid = __builtin_amdgcn_readfirstlane(s_nv[c_i]);
        // lane holds rows r0 + 16 mi + i; one per-lane row limit keeps the 4 MF row
        // tests as comparisons with constants
        const int r0 = 4 * (lane >> 4), lim = nvalid - r0;
        const int64_t o0 = (int64_t)(rowbase + r0) * a.H + col * 256 + wv * 32 + (lane & 15);
        float bias[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bias[j] = out_bias(a.b2, it.z, a.H, col * 256 + wv * 32 + 16 * j + (lane & 15));
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (mi * 16 + i < lim) {
                    const int64_t o = o0 + (int64_t)(mi * 16 + i) * a.H;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float v = add_bias(a.b2, acc[mi][j][i], bias[j]);
                        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o + j * 16] = f32_to_bf16(v);
                        else reinterpret_cast<float*>(a.out)[o + j * 16] = v;
                    }
                }
            }
        }
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[mi][j] = v4f{0.f, 0.f, 0.f, 0.f};
    };

    auto step = [&](int s, auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value, un = (u + P) % R;
        rb_wait_vm<kOpsAfter>();
        __syncthreads();
        dma_a(s + P);
        load_b(Bf[un], Sa[un], Sb[un]);
        const uint8_t* cur = ring + (s % NST) * (MT * kRbStage);
        // fragments holding no valid row of the item are skipped (the count is uniform)
        const int nact = min(MF, (__builtin_amdgcn_readfirstlane(s_nv[c_i]) + 15) >> 4);
        // fragment mi + 1 is read from LDS while the instructions of fragment mi run; the
        // scheduling barriers keep the compiler from hoisting all 8 MT reads (registers)
        v8i af = rb_lds_frag(cur, lane);
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
            v8i an = af;
            if (mi + 1 < MF) an = rb_lds_frag(cur + (mi + 1) * kFragBytes, lane);
            if (mi < nact) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[mi][j] = rb_mfma_sel(mi & 3, af, Bf[u][j], acc[mi][j], Sa[u][mi >> 3][(mi & 7) >> 2], Sb[u]);
            }
            __builtin_amdgcn_sched_barrier(0);
            af = an;
        }
        if (++c_kb == KB) {
            epilogue();
            c_kb = 0;
            ++c_i;
        }
    };

    for (int s = 0; s < G; s += R) {
        rb_static_for(
            [&](auto U) __attribute__((always_inline)) {
                if (s + decltype(U)::value < G) step(s + decltype(U)::value, U);
            },
            std::make_integer_sequence<int, R>{});
    }
    rb_wait_vm<0>();
}

// ----------------------------------------------------------------------------------------
// K blocks in flight and 128-row tiles per item of the persistent down GEMM
#ifndef MOE_RB_P
#define MOE_RB_P 4
#endif
#ifndef MOE_RB_MT
#define MOE_RB_MT 1
#endif

int persistent_grid() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < kRbXcds)
            n = 256;
        cached[dev] = n / kRbXcds * kRbXcds;
    }
    return cached[dev];
}

int64_t persistent_items_per_wg(int ntiles_max, int ncol, int grid) {
    // the larger of the two work orders' per-workgroup counts
    const int64_t nx = grid / kRbXcds;
    return std::max(ceil_div(ord_ranks(ntiles_max, ncol), nx), ceil_div(ceil_div((int64_t)ntiles_max * ncol, kRbXcds), nx));
}

bool ffn_rb_supported(int H, int I, int E, int ntiles_max) {
    if (H % 256 != 0 || I % kGroup != 0) return false;
    // every buffer the kernel addresses takes 32-bit byte offsets
    const int64_t lim = (int64_t)1 << 32;
    if ((int64_t)ntiles_max * kRbBM * I >= lim || (int64_t)H * I >= lim || (int64_t)E * H * I / (kGroup * kGroup) * 4 >= lim)
        return false;
    return persistent_items_per_wg(ntiles_max, H / 256, persistent_grid()) <= kRb2MaxItems;
}

hipError_t launch_gemm2_rb(const FfnArgs& f, const FfnWs& w, int ntiles_max, int ord, hipStream_t st) {
    const int KB = f.I / kGroup, NBS = f.H / kGroup;
    const int64_t n = (int64_t)f.E * KB * NBS;
    hipLaunchKernelGGL(k_rb_scales, dim3((unsigned)std::min<int64_t>(1024, ceil_div(n, 256))), dim3(256), 0, st, f.w2s,
                       f.E, KB, NBS, w.bs);
    Rb2Args g2{w.hq, w.hs, w.bs, f.H, f.I, f.E, ntiles_max, w.tiles, w.ntiles, f.counts, f.offsets, f.w2p, f.out,
               f.out_bf16, ord, f.b2};
    hipLaunchKernelGGL((k_gemm2_rb<MOE_RB_P, MOE_RB_MT>), dim3(persistent_grid()), dim3(kRbThreads), 0, st, g2);
    return hipGetLastError();
}

}  // namespace moe
