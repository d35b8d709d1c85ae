// Host-side arithmetic of the C ABI: work plans, workspace layouts and argument validation.
// Plain C++ (no HIP): the same translation unit is built into the library and, on its own,
// into a CPU test under the address and undefined-behaviour sanitizers.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_fp8.h"

namespace moe {

// ---- quantisation schemes of the grouped FFN (values of moe_ffn_args.quant)
constexpr int kQuantFp8Block128 = 0;   // E4M3 per (row, 128), weights per 128 x 128 block
constexpr int kQuantMxfp8 = 1;         // E4M3 per (row, 32), E4M3 weights per (32 x 1)
constexpr int kQuantW4A8 = 2;          // E4M3 per (row, 32), E2M1 weights per (32 x 1)
constexpr int kQuantW8A16 = 3;         // bf16 activations, E4M3 weights per 128 x 128 block
constexpr int kWfmtE4M3 = 0, kWfmtE2M1 = 1;

constexpr int kScatterChunk = 1024;    // assignments per dispatch workgroup
constexpr int kDispatchOneMaxA = 4096; // largest assignment count of the one-workgroup dispatch
#define MOE_DISPATCH_MAX_E 1024

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- grouped FFN work plan
struct FfnPlan {
    int BM;           // rows per tile
    int ntiles_max;   // grid bound on tiles
    int pairs;        // 1: the 128-row tiles run as 256-row items (pairs of tiles)
    int pairs_down;   // 1: the down GEMM runs on pairs (always with pairs; also below their
                      //    threshold, where gate/up keeps 128-row tiles)
    int npairs_max;   // grid bound on pairs
};
FfnPlan ffn_plan(int T, int k, int E, int quant, int H);

// Byte offsets of the grouped FFN's workspace regions (from a 256-byte aligned base):
// tiles int2 [ntiles_max] | ntiles | hq [rows, I] (bf16 for W8A16) | hs [rows, I/32] |
// (128-row tiles) down-GEMM weight-scale table [E][H/128][I/128] u32 | pairs int4 | npairs
struct FfnWsLayout {
    size_t tiles, ntiles, hq, hs, bs, pairs, npairs, end;
};
FfnWsLayout ffn_ws_layout(int T, int H, int I, int E, int k, int quant);
size_t ffn_rb_scale_table_bytes(int H, int I, int E);
// covers every quantisation scheme
size_t ffn_workspace_bytes(int T, int H, int I, int E, int k);

size_t route_chunk_bytes(int T, int E, int k);
size_t route_ws_bytes(int T, int E, int k, int with_prelude);

// Byte offsets of moe_fused's workspace regions (E and k already include the shared expert):
// ids | weights | counts | offsets | sorted | pos | route ws | xq | xs | ffn ws | expert_out
struct FusedWsLayout {
    size_t ids, wts, counts, offsets, sorted, pos, route, xq, xs, ffn, eo, end;
};
FusedWsLayout fused_ws_layout(int T, int H, int I, int E, int k, int eo_bytes);

// ---- validation (each returns MOE_OK or an error code and sets the thread's message)
namespace host {
int fail(int code, const char* fmt, ...);
int ok();
const char* last_error();

int check_route(const moe_route_params* p, int32_t T, const float* logits, const uint16_t* hidden, int32_t H,
                const moe_gate_prelude* prelude, int32_t flags, const void* const outs[6], const void* ws,
                size_t ws_bytes);
int check_quant_act(const char* op, const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, const uint8_t* xq,
                    const uint8_t* xs, int group);
int check_quant_weight_blocks(const float* w, int32_t E, int32_t K, int32_t N, const uint8_t* q, const uint8_t* s);
int check_prepack(const uint8_t* w, int32_t E, int32_t K, int32_t N, const uint8_t* packed);
int check_quant_weight_mx(const float* w, int32_t E, int32_t K, int32_t N, int32_t wfmt, const uint8_t* q,
                          const uint8_t* s);
int check_prepack_mx(const uint8_t* q, const uint8_t* s, int32_t E, int32_t K, int32_t N, int32_t wfmt,
                     const uint8_t* packed, const uint8_t* packed_s);
int check_grouped_ffn(const moe_ffn_args* a);
int check_combine(const void* eo, int32_t dtype, const int32_t* pos, const float* w, int32_t T, int32_t k, int32_t H,
                  const uint16_t* y);
int check_fused(const moe_fused_args* a);
// moe_fused_static: the library's scratch array of `scratch_bytes` replaces the workspace
int check_fused_static(const moe_fused_args* a, size_t scratch_bytes);
}  // namespace host

}  // namespace moe
