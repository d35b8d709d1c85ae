// Host-side arithmetic of the C ABI (plain C++, no HIP): the grouped FFN's work plan, the
// workspace layouts, and the validation of every entry point's arguments.  Every check runs
// before the first launch, so a rejected call enqueues nothing (the launch guard of
// run_fp8_grouped_w8a8 in the metrale page: launch nothing unless the shapes and buffers
// fit); error texts follow the "moe_gate.rs" validation style ("<op>: <what> must be ...").
//
// 32-bit addressing.  The kernels address buffers through descriptors with 32-bit sizes and
// byte offsets, and some index products are 32-bit integers.  The products that feed them,
// and the bound each call enforces (MOE_ERR_UNSUPPORTED beyond it):
//   T * H            activation rows (xq, the bf16 hidden states): offsets tok * H + c, and
//                    the decode kernels mark past-the-end refills with bit 31    < 2^31
//   2 * I * H        one expert's packed w13 (and I * H of w2): fragment offsets
//                    ((n16 * (H/128) + kb) * 2048) are int                       < 2^31
//   T * k            assignments (int ids and positions); T * k * 4 is the byte size of
//                    the sorted-assignment descriptor                             < 2^29
//   rows_max * I     the hq tile slots (rows_max = tile bound * rows per tile; x2 bytes for
//                    W8A16), addressed by the persistent down GEMM with 32-bit offsets only
//                    when it fits (k_ffn_rb.hip checks), 64-bit elsewhere         (no bound)
//   A * H * 4        expert_out: 64-bit row offsets                               (no bound)
#include "moe_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace moe {

// Decode tiles (16 rows) while experts average at most this many rows; 128-row tiles above.
#ifndef MOE_DEC_MAX_AVG_ROWS
#define MOE_DEC_MAX_AVG_ROWS 24
#endif
// 256-row items (tile pairs) once experts average at least this many rows; the down GEMM
// takes them from a lower average on (measured: at 64 rows per expert, of which half the
// experts are empty, 256-row down items beat the persistent 128-row kernel while the gate/up
// GEMM stays faster on 128-row tiles).
#ifndef MOE_PAIR_MIN_AVG_ROWS
#define MOE_PAIR_MIN_AVG_ROWS 128
#endif
#ifndef MOE_PAIR_DOWN_MIN_AVG_ROWS
#define MOE_PAIR_DOWN_MIN_AVG_ROWS 64
#endif

FfnPlan ffn_plan(int T, int k, int E, int quant, int H) {
    const int64_t A = (int64_t)T * k;
    const int64_t avg = A / E;
    FfnPlan p;
    // 128-row tiles once experts average more than a decode batch's rows: every shape for the
    // 128-element scheme (its plain kernels take any H), H % 256 == 0 for the MX schemes (their
    // down GEMM works in 256-column blocks); W8A16 stays on 16-row tiles
    const bool fp8 = quant == kQuantFp8Block128, mx = quant == kQuantMxfp8 || quant == kQuantW4A8;
    p.BM = avg > MOE_DEC_MAX_AVG_ROWS && (fp8 || (mx && H % 256 == 0)) ? 128 : 16;
    p.ntiles_max = (int)(cdiv(A, p.BM) + std::min<int64_t>(E, A));
    // 256-row items: both GEMMs from 128 rows per expert on; the 128-element scheme's down GEMM
    // takes them from 64 on
    p.pairs = p.BM == 128 && avg >= MOE_PAIR_MIN_AVG_ROWS;
    p.pairs_down = p.pairs || (fp8 && p.BM == 128 && avg >= MOE_PAIR_DOWN_MIN_AVG_ROWS);
    // an expert's pairs number ceil(tiles / 2)
    p.npairs_max = (p.ntiles_max + (int)std::min<int64_t>(E, A)) / 2 + 1;
    return p;
}

size_t ffn_rb_scale_table_bytes(int H, int I, int E) { return (size_t)E * (I / 128) * (H / 128) * 4; }

// bytes per element of h in the hq region: E4M3, or bf16 for W8A16
static size_t h_bytes(int quant) { return quant == kQuantW8A16 ? 2 : 1; }

FfnWsLayout ffn_ws_layout(int T, int H, int I, int E, int k, int quant) {
    const FfnPlan p = ffn_plan(T, k, E, quant, H);
    const size_t rows = (size_t)p.ntiles_max * p.BM;
    FfnWsLayout l;
    size_t o = 0;
    l.tiles = o;
    o += align256((size_t)p.ntiles_max * 8);
    l.ntiles = o;
    o += align256(4);
    l.hq = o;
    o += align256(rows * I * h_bytes(quant));
    l.hs = o;   // one scale per 32 columns of h (the MX schemes; the 128 scheme uses a quarter)
    o += align256(rows * (I / 32));
    l.bs = o;
    if (p.BM == 128) o += align256(ffn_rb_scale_table_bytes(H, I, E));
    l.pairs = o;
    o += align256((size_t)p.npairs_max * 16);
    l.npairs = o;
    o += align256(4);
    l.end = o;
    return l;
}

size_t ffn_workspace_bytes(int T, int H, int I, int E, int k) {
    return std::max({ffn_ws_layout(T, H, I, E, k, kQuantFp8Block128).end,
                     ffn_ws_layout(T, H, I, E, k, kQuantMxfp8).end,
                     ffn_ws_layout(T, H, I, E, k, kQuantW8A16).end});
}

size_t route_chunk_bytes(int T, int E, int k) {
    return align256((size_t)cdiv((int64_t)T * k, kScatterChunk) * E * 4);
}

size_t route_ws_bytes(int T, int E, int k, int with_prelude) {
    size_t b = route_chunk_bytes(T, E, k);
    if (with_prelude) b += align256((size_t)T * E * 4);
    return b;
}

FusedWsLayout fused_ws_layout(int T, int H, int I, int E, int k, int eo_bytes) {
    const size_t A = (size_t)T * k;
    FusedWsLayout l;
    size_t o = 0;
    auto take = [&](size_t n) {
        const size_t r = o;
        o += align256(n);
        return r;
    };
    l.ids = take(A * 4);
    l.wts = take(A * 4);
    l.counts = take((size_t)E * 4);
    l.offsets = take((size_t)(E + 1) * 4);
    l.sorted = take(A * 4);
    l.pos = take(A * 4);
    l.route = o;
    o += route_ws_bytes(T, E, k, 1);
    l.xq = take((size_t)T * H);
    l.xs = take((size_t)T * (H / 32));
    l.ffn = o;
    o += ffn_workspace_bytes(T, H, I, E, k);
    l.eo = take(A * H * eo_bytes);
    l.end = o;
    return l;
}

namespace host {

namespace {

thread_local char g_err[512];

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// optional float32 biases: NULL or 4-byte aligned
int check_biases(const char* op, const float* b13, const float* b2) {
    if ((b13 && !aligned(b13, 4)) || (b2 && !aligned(b2, 4)))
        return fail(MOE_ERR_INVALID, "%s: w13_bias and w2_bias must be 4-byte aligned", op);
    return MOE_OK;
}

bool valid_quant(int q) {
    return q == MOE_QUANT_FP8_BLOCK128 || q == MOE_QUANT_MXFP8 || q == MOE_QUANT_W4A8 || q == MOE_QUANT_W8A16;
}

int check_route_params(const char* op, const moe_route_params* p, int T) {
    if (!p) return fail(MOE_ERR_INVALID, "%s: route params must not be NULL", op);
    const int E = p->num_experts;
    if (T < 1) return fail(MOE_ERR_INVALID, "%s: T (%d) must be > 0", op, T);
    if (E < 1) return fail(MOE_ERR_INVALID, "%s: num_experts (%d) must be > 0", op, E);
    if (E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_UNSUPPORTED, "%s: num_experts (%d) exceeds max %d", op, E, MOE_MAX_EXPERTS);
    if (p->top_k < 1 || p->top_k > E)
        return fail(MOE_ERR_INVALID, "%s: top_k (%d) must be in [1, num_experts=%d]", op, p->top_k, E);
    if (p->scoring != MOE_SCORING_SOFTMAX && p->scoring != MOE_SCORING_SIGMOID)
        return fail(MOE_ERR_INVALID, "%s: scoring (%d) must be 0 (softmax) or 1 (sigmoid)", op, p->scoring);
    if (p->group_count < 1) return fail(MOE_ERR_INVALID, "%s: group_count (%d) must be > 0", op, p->group_count);
    if (E % p->group_count)
        return fail(MOE_ERR_INVALID, "%s: num_experts (%d) must be divisible by group_count (%d)", op, E,
                    p->group_count);
    if (p->group_count > MOE_MAX_GROUPS)
        return fail(MOE_ERR_UNSUPPORTED, "%s: group_count (%d) exceeds max %d", op, p->group_count, MOE_MAX_GROUPS);
    if (p->k_group < 1 || p->k_group > p->group_count)
        return fail(MOE_ERR_INVALID, "%s: k_group (%d) must be in [1, group_count=%d]", op, p->k_group,
                    p->group_count);
    const int per = E / p->group_count;
    if (p->group_count > 1) {
        if (p->group_select_mode != 0 && p->group_select_mode != 1)
            return fail(MOE_ERR_INVALID, "%s: group_select_mode (%d) must be 0 or 1", op, p->group_select_mode);
        if (p->top_k > p->k_group * per)
            return fail(MOE_ERR_INVALID, "%s: top_k (%d) must not exceed the experts in the kept groups (%d)", op,
                        p->top_k, p->k_group * per);
        if (p->group_select_mode == 1 && per < 2)
            return fail(MOE_ERR_INVALID, "%s: group_select_mode 1 needs at least 2 experts per group (have %d)", op,
                        per);
    }
    if (!std::isfinite(p->routed_scaling_factor))
        return fail(MOE_ERR_INVALID, "%s: routed_scaling_factor must be finite", op);
    if ((int64_t)T * p->top_k >= ((int64_t)1 << 29))
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * top_k (%lld) must be below 2^29", op, (long long)T * p->top_k);
    return MOE_OK;
}

int check_prelude(const char* op, const moe_gate_prelude* g, const uint16_t* hidden, int H) {
    if (!g->norm_weight || !g->router_weight)
        return fail(MOE_ERR_INVALID, "%s: prelude norm_weight and router_weight must not be NULL", op);
    if (!hidden) return fail(MOE_ERR_INVALID, "%s: hidden_states must not be NULL with a prelude", op);
    if (H < 1) return fail(MOE_ERR_INVALID, "%s: H (%d) must be > 0", op, H);
    if (H % 4) return fail(MOE_ERR_UNSUPPORTED, "%s: prelude H (%d) must be a multiple of 4", op, H);
    if (!aligned(g->norm_weight, 16) || !aligned(g->router_weight, 16) || !aligned(hidden, 8))
        return fail(MOE_ERR_UNSUPPORTED, "%s: prelude weights must be 16-byte and hidden_states 8-byte aligned", op);
    if (!(g->rms_eps >= 0.f) || !std::isfinite(g->rms_eps))
        return fail(MOE_ERR_INVALID, "%s: rms_eps must be finite and >= 0", op);
    return MOE_OK;
}

int check_ffn_shapes(const char* op, int T, int k, int H, int I, int E) {
    if (T < 1 || k < 1 || H < 1 || I < 1 || E < 1)
        return fail(MOE_ERR_INVALID, "%s: T, k, H, I, E (%d, %d, %d, %d, %d) must be > 0", op, T, k, H, I, E);
    if (k > E) return fail(MOE_ERR_INVALID, "%s: top_k (%d) must be <= num_experts (%d)", op, k, E);
    if (E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_UNSUPPORTED, "%s: num_experts (%d) exceeds max %d", op, E, MOE_MAX_EXPERTS);
    if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: hidden size H (%d) must be a multiple of 128", op, H);
    if (I % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: intermediate size I (%d) must be a multiple of 128", op, I);
    if (H > 32768 || I > 32768)
        return fail(MOE_ERR_UNSUPPORTED, "%s: H (%d) and I (%d) must not exceed 32768", op, H, I);
    if ((int64_t)T * k >= ((int64_t)1 << 29))
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * top_k (%lld) must be below 2^29", op, (long long)T * k);
    if ((int64_t)T * H >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * H (%lld) must be below 2^31 (32-bit activation offsets)", op,
                    (long long)T * H);
    if ((int64_t)2 * I * H >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: 2 * I * H (%lld) must be below 2^31 (32-bit weight offsets)", op,
                    (long long)2 * I * H);
    return MOE_OK;
}

int check_weights(const char* op, const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s) {
    if (!w13 || !w13s || !w2 || !w2s) return fail(MOE_ERR_INVALID, "%s: weights and scales must not be NULL", op);
    if (!aligned(w13, 16) || !aligned(w2, 16))
        return fail(MOE_ERR_INVALID, "%s: packed weights must be 16-byte aligned", op);
    return MOE_OK;
}

bool overlap(const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    return (uintptr_t)a < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)a + na;
}

}  // namespace

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return MOE_OK;
}

const char* last_error() { return g_err; }

int check_route(const moe_route_params* p, int32_t T, const float* logits, const uint16_t* hidden, int32_t H,
                const moe_gate_prelude* prelude, int32_t flags, const void* const outs[6], const void* ws,
                size_t ws_bytes) {
    const char* op = "moe_route";
    int rc = check_route_params(op, p, T);
    if (rc) return rc;
    if (flags & ~MOE_ROUTE_IDS_GIVEN) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", op, flags);
    const bool given = flags & MOE_ROUTE_IDS_GIVEN;
    if (!given) {
        if (prelude) {
            if ((rc = check_prelude(op, prelude, hidden, H))) return rc;
            if ((int64_t)T * H >= ((int64_t)1 << 31))
                return fail(MOE_ERR_UNSUPPORTED, "%s: T * H (%lld) must be below 2^31", op, (long long)T * H);
        } else if (!logits) {
            return fail(MOE_ERR_INVALID, "%s: router_logits must not be NULL without a prelude", op);
        }
    }
    for (int i = 0; i < 6; ++i)
        if (!outs[i]) return fail(MOE_ERR_INVALID, "%s: output pointers must not be NULL", op);
    const size_t need = route_ws_bytes(T, p->num_experts, p->top_k, !given && prelude);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    return MOE_OK;
}

int check_quant_act(const char* op, const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, const uint8_t* xq,
                    const uint8_t* xs, int group) {
    if (!x || !xq || !xs) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID, "%s: rows (%d) and cols (%d) must be > 0", op, rows, cols);
    if (cols % group) return fail(MOE_ERR_UNSUPPORTED, "%s: cols (%d) must be a multiple of %d", op, cols, group);
    if (ld < cols) return fail(MOE_ERR_INVALID, "%s: ld (%lld) must be >= cols (%d)", op, (long long)ld, cols);
    if (ld % 8 || !aligned(x, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned with ld %% 8 == 0", op);
    if (!aligned(xq, 8)) return fail(MOE_ERR_UNSUPPORTED, "%s: xq must be 8-byte aligned", op);
    return MOE_OK;
}

int check_quant_weight_blocks(const float* w, int32_t E, int32_t K, int32_t N, const uint8_t* q, const uint8_t* s) {
    const char* op = "moe_quant_weight_blocks";
    if (!w || !q || !s) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (K % 128 || N % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) and N (%d) must be multiples of 128", op, K, N);
    if (!aligned(w, 16) || !aligned(q, 4)) return fail(MOE_ERR_UNSUPPORTED, "%s: w must be 16-byte and q 4-byte aligned", op);
    if ((int64_t)E * (K / 128) * (N / 128) > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: too many blocks", op);
    return MOE_OK;
}

int check_prepack(const uint8_t* w, int32_t E, int32_t K, int32_t N, const uint8_t* packed) {
    const char* op = "moe_prepack_weights";
    if (!w || !packed) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (K % 128 || N % 16) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 128 and N (%d) of 16", op, K, N);
    if (!aligned(packed, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: packed must be 16-byte aligned", op);
    const uintptr_t n = (uintptr_t)E * K * N;
    if (overlap(w, n, packed, n)) return fail(MOE_ERR_INVALID, "%s: packed must not overlap w", op);
    return MOE_OK;
}

int check_quant_weight_mx(const float* w, int32_t E, int32_t K, int32_t N, int32_t wfmt, const uint8_t* q,
                          const uint8_t* s) {
    const char* op = "moe_quant_weight_mx";
    if (!w || !q || !s) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (wfmt != MOE_WFMT_E4M3 && wfmt != MOE_WFMT_E2M1)
        return fail(MOE_ERR_INVALID, "%s: wfmt (%d) must be MOE_WFMT_E4M3 or MOE_WFMT_E2M1", op, wfmt);
    if (K % 32 || N % 2) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 32 and N (%d) even", op, K, N);
    return MOE_OK;
}

int check_prepack_mx(const uint8_t* q, const uint8_t* s, int32_t E, int32_t K, int32_t N, int32_t wfmt,
                     const uint8_t* packed, const uint8_t* packed_s) {
    const char* op = "moe_prepack_weights_mx";
    if (!q || !s || !packed || !packed_s) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (wfmt != MOE_WFMT_E4M3 && wfmt != MOE_WFMT_E2M1)
        return fail(MOE_ERR_INVALID, "%s: wfmt (%d) must be MOE_WFMT_E4M3 or MOE_WFMT_E2M1", op, wfmt);
    if (K % 128 || N % 16) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 128 and N (%d) of 16", op, K, N);
    if (!aligned(packed, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: packed must be 16-byte aligned", op);
    const uintptr_t nq = (uintptr_t)E * K * N / (wfmt == MOE_WFMT_E2M1 ? 2 : 1), ns = (uintptr_t)E * K * N / 32;
    if (overlap(q, nq, packed, nq) || overlap(s, ns, packed_s, ns) || overlap(q, nq, packed_s, ns) ||
        overlap(s, ns, packed, nq))
        return fail(MOE_ERR_INVALID, "%s: outputs must not overlap the inputs", op);
    return MOE_OK;
}

int check_grouped_ffn(const moe_ffn_args* a) {
    const char* op = "moe_grouped_ffn";
    if (!a) return fail(MOE_ERR_INVALID, "%s: args must not be NULL", op);
    int rc = check_ffn_shapes(op, a->T, a->k, a->H, a->I, a->E);
    if (rc) return rc;
    if (!valid_quant(a->quant)) return fail(MOE_ERR_INVALID, "%s: quant (%d) must be one of MOE_QUANT_*", op, a->quant);
    const bool w16 = a->quant == MOE_QUANT_W8A16;
    if (w16 ? !a->x : (!a->xq || !a->xs))
        return fail(MOE_ERR_INVALID, "%s: %s must not be NULL", op, w16 ? "x" : "xq and xs");
    if (!a->expert_counts || !a->expert_offsets || !a->sorted_assign || !a->expert_out)
        return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if ((rc = check_weights(op, a->w13, a->w13_scale, a->w2, a->w2_scale))) return rc;
    if (a->out_dtype != MOE_DTYPE_F32 && a->out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID, "%s: out_dtype (%d) must be MOE_DTYPE_F32 or MOE_DTYPE_BF16", op, a->out_dtype);
    if (!aligned(w16 ? (const void*)a->x : (const void*)a->xq, 16))
        return fail(MOE_ERR_UNSUPPORTED, "%s: %s must be 16-byte aligned", op, w16 ? "x" : "xq");
    if ((rc = check_biases(op, a->w13_bias, a->w2_bias))) return rc;
    if (a->debug_h) {
        if (!a->debug_hq || (!w16 && !a->debug_hs))
            return fail(MOE_ERR_INVALID, "%s: debug_h needs debug_hq%s", op, w16 ? "" : " and debug_hs");
    } else if (a->debug_hq || a->debug_hs) {
        return fail(MOE_ERR_INVALID, "%s: debug_hq and debug_hs are taken only with debug_h", op);
    }
    const size_t need = ffn_workspace_bytes(a->T, a->H, a->I, a->E, a->k);
    if (!a->workspace || a->workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    return MOE_OK;
}

int check_combine(const void* eo, int32_t dtype, const int32_t* pos, const float* w, int32_t T, int32_t k, int32_t H,
                  const uint16_t* y) {
    const char* op = "moe_combine";
    if (!eo || !pos || !w || !y) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (T < 1 || k < 1 || H < 1) return fail(MOE_ERR_INVALID, "%s: T, k, H (%d, %d, %d) must be > 0", op, T, k, H);
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID, "%s: dtype (%d) must be MOE_DTYPE_F32 or MOE_DTYPE_BF16", op, dtype);
    if (H % 4) return fail(MOE_ERR_UNSUPPORTED, "%s: H (%d) must be a multiple of 4", op, H);
    if ((int64_t)T * k >= ((int64_t)1 << 29))
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * k (%lld) must be below 2^29", op, (long long)T * k);
    if (!aligned(eo, 16) || !aligned(y, 8))
        return fail(MOE_ERR_UNSUPPORTED, "%s: expert_out must be 16-byte and y 8-byte aligned", op);
    return MOE_OK;
}

namespace {
int check_fused_common(const char* op, const moe_fused_args* a, size_t* need);
}

int check_fused(const moe_fused_args* a) {
    const char* op = "moe_fused";
    size_t need = 0;
    int rc = check_fused_common(op, a, &need);
    if (rc) return rc;
    if (!a->workspace || a->workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    return MOE_OK;
}

int check_fused_static(const moe_fused_args* a, size_t scratch_bytes) {
    const char* op = "moe_fused_static";
    size_t need = 0;
    int rc = check_fused_common(op, a, &need);
    if (rc) return rc;
    if (a->workspace || a->workspace_bytes)
        return fail(MOE_ERR_INVALID, "%s: runs in the library's own scratch array: workspace must be NULL and "
                    "workspace_bytes 0", op);
    if (need > scratch_bytes)
        return fail(MOE_ERR_UNSUPPORTED, "%s: the step needs %zu bytes of scratch, above the library's maximum of "
                    "%zu (use moe_fused with a workspace)", op, need, scratch_bytes);
    return MOE_OK;
}

namespace {
// every check of moe_fused except the workspace's; *need = the workspace bytes the step uses
int check_fused_common(const char* op, const moe_fused_args* a, size_t* need_out) {
    if (!a) return fail(MOE_ERR_INVALID, "%s: args must not be NULL", op);
    int rc = check_route_params(op, &a->route, a->T);
    if (rc) return rc;
    const int T = a->T, H = a->H, I = a->I, E = a->route.num_experts, k = a->route.top_k;
    // with the shared expert the FFN, dispatch and combine see E + 1 experts and k + 1 slots
    const int sh = (a->flags & MOE_FUSED_SHARED_EXPERT) ? 1 : 0;
    if ((rc = check_ffn_shapes(op, T, k + sh, H, I, E + sh))) return rc;
    if (!a->hidden_states || !a->y) return fail(MOE_ERR_INVALID, "%s: hidden_states and y must not be NULL", op);
    if (a->prelude) {
        if ((rc = check_prelude(op, a->prelude, a->hidden_states, H))) return rc;
    } else if (!a->router_logits) {
        return fail(MOE_ERR_INVALID, "%s: router_logits must not be NULL without a prelude", op);
    }
    if ((rc = check_weights(op, a->w13, a->w13_scale, a->w2, a->w2_scale))) return rc;
    if (a->flags & ~(MOE_FUSED_EXPERT_OUT_BF16 | MOE_FUSED_SHARED_EXPERT))
        return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", op, a->flags);
    if (!valid_quant(a->quant)) return fail(MOE_ERR_INVALID, "%s: quant (%d) must be one of MOE_QUANT_*", op, a->quant);
    if (!aligned(a->hidden_states, 16) || !aligned(a->y, 8))
        return fail(MOE_ERR_UNSUPPORTED, "%s: hidden_states must be 16-byte and y 8-byte aligned", op);
    if ((rc = check_biases(op, a->w13_bias, a->w2_bias))) return rc;
    *need_out = fused_ws_layout(T, H, I, E + sh, k + sh, (a->flags & MOE_FUSED_EXPERT_OUT_BF16) ? 2 : 4).end;
    if ((a->act_q && !aligned(a->act_q, 16)) || (a->act_scales && !aligned(a->act_scales, 16)))
        return fail(MOE_ERR_INVALID, "%s: act_q and act_scales must be 16-byte aligned", op);
    if (a->quant == MOE_QUANT_W8A16 && (a->act_q || a->act_scales))
        return fail(MOE_ERR_INVALID, "%s: MOE_QUANT_W8A16 quantises no activations: act_q and act_scales must be NULL",
                    op);
    return MOE_OK;
}
}  // namespace

}  // namespace host
}  // namespace moe
