// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_plan.h"

namespace moe {

// ---- quantisation / layout
hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                            hipStream_t st);
hipError_t launch_quant_weight_blocks(const float* w, int E, int K, int N, uint8_t* q, uint8_t* s,
                                      hipStream_t st);
hipError_t launch_prepack(const uint8_t* w, int E, int K, int N, uint8_t* out, hipStream_t st);
hipError_t launch_quant_act_mx(const uint16_t* x, int rows, int cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                               hipStream_t st);
hipError_t launch_quant_weight_mx(const float* w, int E, int K, int N, int wfmt, uint8_t* q, uint8_t* s,
                                  hipStream_t st);
hipError_t launch_prepack_mx(const uint8_t* q, const uint8_t* s, int E, int K, int N, int wfmt, uint8_t* packed,
                             uint8_t* packed_s, hipStream_t st);

// ---- routing and dispatch
struct RouteCfg {
    int T, E, k;
    int scoring;            // 0 softmax, 1 sigmoid
    int renormalize;
    int G, k_group, mode;
    float rsf;
    int prelude;            // weights = softmax over selected * per_expert_scale
    int ld;                 // row stride of ids / weights (>= k)
    int shared_id;          // >= 0: column k of each row gets this expert with weight 1
};

hipError_t launch_gate_prelude(const uint16_t* x, int T, int H, int E, const float* norm_w,
                               const float* router_w, float eps, float* logits, hipStream_t st);
// optional fused activation quantisation in the routing kernel (x == nullptr: none)
struct QuantOut {
    const uint16_t* x;   // [T, H] bf16
    int H;
    uint8_t* xq;         // [T, H] E4M3
    uint8_t* xs;         // [T, H/group] UE8M0
    int group;           // elements per scale: 128, or 32 for the micro-scaled schemes
};
hipError_t launch_route(const float* logits, const RouteCfg& c, const float* pe_scale, int32_t* ids,
                        float* weights, hipStream_t st, QuantOut qo = QuantOut{nullptr, 0, nullptr, nullptr, 128});
// Dispatch (stable counting sort).  A <= kDispatchOneMaxA: one workgroup; otherwise
// hist + scan + scatter over chunks (chunk_ws holds nchunks*E int32).  With tiles given,
// also the GEMM tile list for BM-row tiles.
hipError_t launch_dispatch(const int32_t* ids, int A, int E, int32_t* chunk_ws, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, hipStream_t st,
                           int BM = 0, int2* tiles = nullptr, int32_t* ntiles = nullptr, int4* pairs = nullptr,
                           int32_t* npairs = nullptr);
// pair list of the 256-row items from the expert counts (k_ffn.hip)
hipError_t launch_pairs(const int32_t* counts, const int32_t* offsets, int E, int4* pairs, int32_t* npairs,
                        hipStream_t st);
hipError_t launch_tiles(const int32_t* counts, int E, int BM, int2* tiles, int32_t* ntiles, hipStream_t st);

// ---- grouped FFN (plan and workspace layout: moe_plan.h)
struct FfnArgs {
    int T, k, H, I, E;
    const uint8_t* xq;
    const uint8_t* xs;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const uint8_t* w13p;
    const uint8_t* w13s;
    const uint8_t* w2p;
    const uint8_t* w2s;
    void* out;
    int out_bf16;
    int quant;       // kQuant*; for the MX schemes w13s / w2s are the packed MX scales
    const uint16_t* x = nullptr;   // kQuantW8A16: the bf16 hidden states [T, H] (xq, xs unused)
    // optional test outputs (moe_ffn_args.debug_*): float32 h before re-quantisation, and the
    // re-quantised h and scales unpacked from the down GEMM's operand order, [A, I] in sorted order
    float* debug_h = nullptr;
    uint8_t* debug_hq = nullptr;
    uint8_t* debug_hs = nullptr;
    // optional float32 biases: gate/up sums [E, 2I] (before SwiGLU), down output [E, H]
    const float* b13 = nullptr;
    const float* b2 = nullptr;
};
struct FfnWs {
    int2* tiles;
    int32_t* ntiles;
    uint8_t* hq;
    uint8_t* hs;
    uint32_t* bs;        // 128-row tiles: down-GEMM weight-block scales per [expert][column block][kb]
    int4* pairs;         // 256-row items: {first tile, expert, first sorted row, valid rows} per pair
    int32_t* npairs;
};
FfnWs carve_ffn_ws(const FfnArgs& a, void* ws);
// `mid`: optional event recorded between the gate+up and the down GEMM; tiles_ready: the
// tile list in the workspace was already written (by launch_dispatch)
hipError_t launch_grouped_ffn(const FfnArgs& a, void* ws, hipStream_t st, hipEvent_t mid = nullptr,
                              bool tiles_ready = false, bool pairs_ready = false);
// MX schemes on 16-row tiles (k_mx.hip)
hipError_t launch_ffn_mx(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid);
// MX schemes on 128-row tiles (k_ffn.hip)
hipError_t launch_ffn_mx_pf(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid,
                            bool pairs_ready);
// W8A16 on 16-row tiles (k_w16.hip); h in bf16 takes the hq region (sized 2 bytes per element)
hipError_t launch_ffn_w16(const FfnArgs& f, const FfnPlan& p, const FfnWs& w, hipStream_t st, hipEvent_t mid);

int ffn_super_tile_order(int ntiles_max);
// persistent down GEMM for 128-row tiles (k_ffn_rb.hip)
bool ffn_rb_supported(int H, int I, int E, int ntiles_max);
// persistent kernels: workgroups (the CU count, a multiple of 8) and the largest item count
// one workgroup takes from ntiles_max x ncol items in either work order
int persistent_grid();
int64_t persistent_items_per_wg(int ntiles_max, int ncol, int grid);
hipError_t launch_gemm2_rb(const FfnArgs& f, const FfnWs& w, int ntiles_max, int ord, hipStream_t st);

hipError_t launch_combine(const void* eo, int bf16, const int32_t* pos, const float* w, int T, int k, int H,
                          uint16_t* y, hipStream_t st);

}  // namespace moe
