// Item lists of the persistent grouped-GEMM kernels (one workgroup of 512 threads per CU).
// An item is (tile, column block) over the expert-ordered list of 128-row tiles; each
// workgroup builds the list of its own items in LDS at start.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kItWaves = 8;
constexpr int kItThreads = 64 * kItWaves;
constexpr int kItXcds = 8;
constexpr int kItGroupTiles = 4;     // tiles per super-block of the column-block work order
constexpr int kItTileRows = 128;

// The items of persistent workgroup L: the list of ntiles * ncol items is cut into kItXcds
// contiguous shares, share x for the workgroups on XCD x (workgroup L runs on XCD L % 8);
// inside a share the nx workgroups of the XCD take items j, j + nx, ... so the ones running
// together walk consecutive items.  Item w: super-block w / (4 * ncol) of 4 consecutive
// tiles (mostly one expert), column block outer inside it, so concurrent workgroups share
// A rows and weight columns through the XCD's L2.
struct ItSched {
    int base, stride, n;
};
__device__ __forceinline__ ItSched it_sched(int total) {
    const int nx = gridDim.x / kItXcds;
    const int L = blockIdx.x, x = L % kItXcds, j = L / kItXcds;
    const int per = (total + kItXcds - 1) / kItXcds;
    ItSched s;
    s.base = x * per + j;
    s.stride = nx;
    const int in_share = j < per ? (per - 1 - j) / nx + 1 : 0;
    const int lim = total - s.base;   // items w = base + nx * i < total
    const int in_total = lim > 0 ? (lim - 1) / nx + 1 : 0;
    s.n = min(in_share, in_total);
    return s;
}

__device__ __forceinline__ void it_tile_col(int w, int ncol, int ntiles, int& tile, int& col) {
    const int sb = w / (kItGroupTiles * ncol), r = w - sb * kItGroupTiles * ncol;
    const int t0 = sb * kItGroupTiles;
    const int g = min(kItGroupTiles, ntiles - t0);
    col = r / g;
    tile = t0 + r - col * g;
}

// Item table in LDS: {tile, column block, expert, first sorted row}, and valid rows.  An
// item covers MT consecutive 128-row tiles of one expert: with MT = 2 only a tile that starts
// an expert's even 256-row block leads an item, and the item's rows run on into the next
// tile when the expert has one.  The workgroup's items are the valid ones among its
// candidates, in order: with the super-tile order (ord) ranks j, j + nx, ... of its XCD's
// share (ord_item); otherwise its contiguous share of the column-block order (it_sched).
// Returns the item count.
template <int MT>
__device__ __forceinline__ int it_fill_items(int ord, int ncol, int ntiles, const int2* tiles, const int32_t* counts,
                                             const int32_t* offsets, int4* s_it, int* s_nv, int cap, int* s_cnt) {
    const int nx = gridDim.x / kItXcds, x = blockIdx.x % kItXcds, j = blockIdx.x / kItXcds;
    const ItSched sch = it_sched(ntiles * ncol);
    int ncand;
    if (ord) {
        const int total = ord_ranks(ntiles, ncol);   // ranks per XCD
        ncand = j < total ? (total - 1 - j) / nx + 1 : 0;
    } else {
        ncand = sch.n;
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int base = 0;
    for (int c0 = 0; c0 < ncand; c0 += kItThreads) {
        const int c = c0 + threadIdx.x;
        int tile = 0, col = 0;
        bool v = false;
        if (c < ncand) {
            if (ord) {
                v = ord_item(x, j + nx * c, ntiles, ncol, tile, col);
            } else {
                it_tile_col(sch.base + sch.stride * c, ncol, ntiles, tile, col);
                v = true;
            }
        }
        int2 te = make_int2(0, 0);
        if (v) {
            te = tiles[tile];
            if (MT == 2) v = te.y % (2 * kItTileRows) == 0;
        }
        const uint64_t m = __ballot(v);
        if (lane == 0) s_cnt[wv] = __popcll(m);
        __syncthreads();
        int off = base, tot = 0;
        for (int w = 0; w < kItWaves; ++w) {
            off += w < wv ? s_cnt[w] : 0;
            tot += s_cnt[w];
        }
        const int pos = off + __popcll(m & ((1ull << lane) - 1));
        if (v && pos < cap) {
            s_it[pos] = make_int4(tile, col, te.x, offsets[te.x] + te.y);
            s_nv[pos] = min(MT * kItTileRows, counts[te.x] - te.y);
        }
        base += tot;
        __syncthreads();
    }
    // Every load above has been used; the wait (which the compiler sees) keeps a load it
    // skipped on some path from being waited for later, inside the caller's DMA stream.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    return min(base, cap);
}

}  // namespace moe
