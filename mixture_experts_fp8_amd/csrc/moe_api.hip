// C ABI of the routed FP8 MoE step: host-side validation, workspace carving and launch
// order.  Every check happens before the first launch, so a rejected call enqueues
// nothing (the launch guard of run_fp8_grouped_w8a8 in the metrale page); error texts
// follow the "moe_gate.rs" validation style ("<op>: <what> must be ...").
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe_fp8.h"
#include "moe_common.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[512];

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
int hip_fail(const char* op, hipError_t e) {
    return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", op, (int)e, hipGetErrorString(e));
}
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

using moe::align256;

size_t route_ws_bytes(int T, int E, int k, int with_prelude) {
    const int64_t A = (int64_t)T * k;
    const int64_t nchunks = moe::ceil_div(A, moe::kScatterChunk);
    size_t b = align256((size_t)nchunks * E * 4);
    if (with_prelude) b += align256((size_t)T * E * 4);
    return b;
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
    if ((int64_t)T * p->top_k > INT32_MAX / 2)
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * top_k (%lld) too large", op, (long long)T * p->top_k);
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

moe::RouteCfg route_cfg(const moe_route_params* p, int T, bool prelude) {
    moe::RouteCfg c;
    c.T = T;
    c.E = p->num_experts;
    c.k = p->top_k;
    c.scoring = p->scoring;
    c.renormalize = p->renormalize != 0;
    c.G = p->group_count;
    c.k_group = p->k_group;
    c.mode = p->group_select_mode;
    c.rsf = p->routed_scaling_factor;
    c.prelude = prelude ? 1 : 0;
    c.ld = c.k;
    c.shared_id = -1;
    return c;
}

size_t route_chunk_bytes(int T, int E, int k) {
    return align256((size_t)moe::ceil_div((int64_t)T * k, moe::kScatterChunk) * E * 4);
}

// route + dispatch with all pointers already validated; ws holds route_ws_bytes
hipError_t do_route(const moe_route_params* p, int T, const float* logits, const uint16_t* hidden, int H,
                    const moe_gate_prelude* g, int flags, int32_t* ids, float* wts, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, uint8_t* ws, hipStream_t st) {
    const int E = p->num_experts, k = p->top_k;
    const int64_t A = (int64_t)T * k;
    int32_t* chunk_ws = reinterpret_cast<int32_t*>(ws);
    uint8_t* after = ws + route_chunk_bytes(T, E, k);
    hipError_t e = hipSuccess;
    if (!(flags & MOE_ROUTE_IDS_GIVEN)) {
        const float* lg = logits;
        if (g) {
            float* pl = reinterpret_cast<float*>(after);
            e = moe::launch_gate_prelude(hidden, T, H, E, g->norm_weight, g->router_weight, g->rms_eps, pl, st);
            if (e != hipSuccess) return e;
            lg = pl;
        }
        e = moe::launch_route(lg, route_cfg(p, T, g != nullptr), g ? g->per_expert_scale : nullptr, ids, wts, st);
        if (e != hipSuccess) return e;
    }
    return moe::launch_dispatch(ids, (int)A, E, chunk_ws, counts, offsets, sorted_assign, assign_pos, st);
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
    if ((int64_t)T * k > INT32_MAX / 2)
        return fail(MOE_ERR_UNSUPPORTED, "%s: T * top_k (%lld) too large", op, (long long)T * k);
    return MOE_OK;
}

int check_weights(const char* op, const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s) {
    if (!w13 || !w13s || !w2 || !w2s) return fail(MOE_ERR_INVALID, "%s: weights and scales must not be NULL", op);
    if (!aligned(w13, 16) || !aligned(w2, 16))
        return fail(MOE_ERR_INVALID, "%s: packed weights must be 16-byte aligned", op);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t top_k, int32_t H, int32_t with_prelude) {
    (void)H;
    if (T < 1 || E < 1 || top_k < 1) return 0;
    return route_ws_bytes(T, E, top_k, with_prelude);
}

int moe_route(const moe_route_params* p, int32_t T, const float* router_logits, const uint16_t* hidden_states,
              int32_t H, const moe_gate_prelude* prelude, int32_t flags, int32_t* topk_ids, float* topk_weights,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_assign, int32_t* assign_pos,
              void* workspace, size_t workspace_bytes, void* stream) {
    const char* op = "moe_route";
    int rc = check_route_params(op, p, T);
    if (rc) return rc;
    if (flags & ~MOE_ROUTE_IDS_GIVEN) return fail(MOE_ERR_INVALID, "%s: unknown flags 0x%x", op, flags);
    const bool given = flags & MOE_ROUTE_IDS_GIVEN;
    if (!given) {
        if (prelude) {
            if ((rc = check_prelude(op, prelude, hidden_states, H))) return rc;
        } else if (!router_logits) {
            return fail(MOE_ERR_INVALID, "%s: router_logits must not be NULL without a prelude", op);
        }
    }
    if (!topk_ids || !topk_weights || !expert_counts || !expert_offsets || !sorted_assign || !assign_pos)
        return fail(MOE_ERR_INVALID, "%s: output pointers must not be NULL", op);
    const size_t need = route_ws_bytes(T, p->num_experts, p->top_k, !given && prelude);
    if (!workspace || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    const hipError_t e = do_route(p, T, router_logits, hidden_states, H, given ? nullptr : prelude, flags, topk_ids,
                                  topk_weights, expert_counts, expert_offsets, sorted_assign, assign_pos,
                                  static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_quant_act(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                  void* stream) {
    const char* op = "moe_quant_act";
    if (!x || !xq || !xs) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID, "%s: rows (%d) and cols (%d) must be > 0", op, rows, cols);
    if (cols % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: cols (%d) must be a multiple of 128", op, cols);
    if (ld < cols) return fail(MOE_ERR_INVALID, "%s: ld (%lld) must be >= cols (%d)", op, (long long)ld, cols);
    if (ld % 8 || !aligned(x, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned with ld %% 8 == 0", op);
    if (!aligned(xq, 8)) return fail(MOE_ERR_UNSUPPORTED, "%s: xq must be 8-byte aligned", op);
    const hipError_t e = moe::launch_quant_act(x, rows, cols, ld, xq, xs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_quant_weight_blocks(const float* w, int32_t E, int32_t K, int32_t N, uint8_t* q, uint8_t* scale,
                            void* stream) {
    const char* op = "moe_quant_weight_blocks";
    if (!w || !q || !scale) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (K % 128 || N % 128) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) and N (%d) must be multiples of 128", op, K, N);
    if (!aligned(w, 16) || !aligned(q, 4)) return fail(MOE_ERR_UNSUPPORTED, "%s: w must be 16-byte and q 4-byte aligned", op);
    if ((int64_t)E * (K / 128) * (N / 128) > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: too many blocks", op);
    const hipError_t e = moe::launch_quant_weight_blocks(w, E, K, N, q, scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_prepack_weights(const uint8_t* w, int32_t E, int32_t K, int32_t N, uint8_t* packed, void* stream) {
    const char* op = "moe_prepack_weights";
    if (!w || !packed) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (K % 128 || N % 16) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 128 and N (%d) of 16", op, K, N);
    if (!aligned(packed, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: packed must be 16-byte aligned", op);
    const uintptr_t n = (uintptr_t)E * K * N;
    if ((uintptr_t)w < (uintptr_t)packed + n && (uintptr_t)packed < (uintptr_t)w + n)
        return fail(MOE_ERR_INVALID, "%s: packed must not overlap w", op);
    const hipError_t e = moe::launch_prepack(w, E, K, N, packed, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_quant_act_mx(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                     void* stream) {
    const char* op = "moe_quant_act_mx";
    if (!x || !xq || !xs) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID, "%s: rows (%d) and cols (%d) must be > 0", op, rows, cols);
    if (cols % 32) return fail(MOE_ERR_UNSUPPORTED, "%s: cols (%d) must be a multiple of 32", op, cols);
    if (ld < cols) return fail(MOE_ERR_INVALID, "%s: ld (%lld) must be >= cols (%d)", op, (long long)ld, cols);
    if (ld % 8 || !aligned(x, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned with ld %% 8 == 0", op);
    if (!aligned(xq, 8)) return fail(MOE_ERR_UNSUPPORTED, "%s: xq must be 8-byte aligned", op);
    const hipError_t e = moe::launch_quant_act_mx(x, rows, cols, ld, xq, xs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_quant_weight_mx(const float* w, int32_t E, int32_t K, int32_t N, int32_t wfmt, uint8_t* q, uint8_t* scale,
                        void* stream) {
    const char* op = "moe_quant_weight_mx";
    if (!w || !q || !scale) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (wfmt != MOE_WFMT_E4M3 && wfmt != MOE_WFMT_E2M1)
        return fail(MOE_ERR_INVALID, "%s: wfmt (%d) must be MOE_WFMT_E4M3 or MOE_WFMT_E2M1", op, wfmt);
    if (K % 32 || N % 2) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 32 and N (%d) even", op, K, N);
    const hipError_t e = moe::launch_quant_weight_mx(w, E, K, N, wfmt, q, scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_prepack_weights_mx(const uint8_t* q, const uint8_t* scale, int32_t E, int32_t K, int32_t N, int32_t wfmt,
                           uint8_t* packed, uint8_t* packed_scale, void* stream) {
    const char* op = "moe_prepack_weights_mx";
    if (!q || !scale || !packed || !packed_scale) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (E < 1 || K < 1 || N < 1) return fail(MOE_ERR_INVALID, "%s: E, K, N (%d, %d, %d) must be > 0", op, E, K, N);
    if (wfmt != MOE_WFMT_E4M3 && wfmt != MOE_WFMT_E2M1)
        return fail(MOE_ERR_INVALID, "%s: wfmt (%d) must be MOE_WFMT_E4M3 or MOE_WFMT_E2M1", op, wfmt);
    if (K % 128 || N % 16) return fail(MOE_ERR_UNSUPPORTED, "%s: K (%d) must be a multiple of 128 and N (%d) of 16", op, K, N);
    if (!aligned(packed, 16)) return fail(MOE_ERR_UNSUPPORTED, "%s: packed must be 16-byte aligned", op);
    const uintptr_t nq = (uintptr_t)E * K * N / (wfmt == MOE_WFMT_E2M1 ? 2 : 1), ns = (uintptr_t)E * K * N / 32;
    auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
        return (uintptr_t)a < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)a + na;
    };
    if (overlap(q, nq, packed, nq) || overlap(scale, ns, packed_scale, ns) || overlap(q, nq, packed_scale, ns) ||
        overlap(scale, ns, packed, nq))
        return fail(MOE_ERR_INVALID, "%s: outputs must not overlap the inputs", op);
    const hipError_t e = moe::launch_prepack_mx(q, scale, E, K, N, wfmt, packed, packed_scale,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

size_t moe_ffn_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
    if (T < 1 || H < 1 || I < 128 || E < 1 || k < 1) return 0;
    return moe::ffn_workspace_bytes(T, H, I, E, k);
}

int moe_grouped_ffn(const moe_ffn_args* a) {
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
    const size_t need = moe::ffn_workspace_bytes(a->T, a->H, a->I, a->E, a->k);
    if (!a->workspace || a->workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    moe::FfnArgs f{a->T, a->k, a->H, a->I, a->E, a->xq, a->xs, a->expert_counts, a->expert_offsets,
                   a->sorted_assign, a->w13, a->w13_scale, a->w2, a->w2_scale, a->expert_out,
                   a->out_dtype == MOE_DTYPE_BF16, a->quant, w16 ? a->x : nullptr};
    const hipError_t e = moe::launch_grouped_ffn(f, a->workspace, static_cast<hipStream_t>(a->stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

int moe_combine(const void* expert_out, int32_t dtype, const int32_t* assign_pos, const float* topk_weights,
                int32_t T, int32_t k, int32_t H, uint16_t* y, void* stream) {
    const char* op = "moe_combine";
    if (!expert_out || !assign_pos || !topk_weights || !y) return fail(MOE_ERR_INVALID, "%s: pointers must not be NULL", op);
    if (T < 1 || k < 1 || H < 1) return fail(MOE_ERR_INVALID, "%s: T, k, H (%d, %d, %d) must be > 0", op, T, k, H);
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID, "%s: dtype (%d) must be MOE_DTYPE_F32 or MOE_DTYPE_BF16", op, dtype);
    if (H % 4) return fail(MOE_ERR_UNSUPPORTED, "%s: H (%d) must be a multiple of 4", op, H);
    if (!aligned(expert_out, 16) || !aligned(y, 8))
        return fail(MOE_ERR_UNSUPPORTED, "%s: expert_out must be 16-byte and y 8-byte aligned", op);
    const hipError_t e = moe::launch_combine(expert_out, dtype == MOE_DTYPE_BF16, assign_pos, topk_weights, T, k, H,
                                             y, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

// fused workspace: ids | weights | counts | offsets | sorted | pos | route ws | xq | xs | ffn ws | expert_out
size_t moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t flags) {
    if (T < 1 || H < 128 || I < 128 || E < 1 || k < 1) return 0;
    if (flags & MOE_FUSED_SHARED_EXPERT) {   // one more expert, one more column per token
        ++E;
        ++k;
    }
    const size_t A = (size_t)T * k;
    const size_t eo = (flags & MOE_FUSED_EXPERT_OUT_BF16) ? 2 : 4;
    return 4 * align256(A * 4) + align256((size_t)E * 4) + align256((size_t)(E + 1) * 4) +
           route_ws_bytes(T, E, k, 1) + align256((size_t)T * H) + align256((size_t)T * (H / 32)) +
           moe::ffn_workspace_bytes(T, H, I, E, k) + align256(A * H * eo);
}

int moe_fused(const moe_fused_args* a) {
    const char* op = "moe_fused";
    if (!a) return fail(MOE_ERR_INVALID, "%s: args must not be NULL", op);
    int rc = check_route_params(op, &a->route, a->T);
    if (rc) return rc;
    const int T = a->T, H = a->H, I = a->I, E = a->route.num_experts, k = a->route.top_k;
    // with the shared expert the FFN, dispatch and combine see E + 1 experts and k + 1 slots
    const int sh = (a->flags & MOE_FUSED_SHARED_EXPERT) ? 1 : 0, Ef = E + sh, kf = k + sh;
    if ((rc = check_ffn_shapes(op, T, kf, H, I, Ef))) return rc;
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
    const size_t need = moe_workspace_size(T, H, I, E, k, a->flags);
    if (!a->workspace || a->workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace too small: need %zu bytes, have %zu", op, need,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(MOE_ERR_INVALID, "%s: workspace must be 256-byte aligned", op);
    if ((a->act_q && !aligned(a->act_q, 16)) || (a->act_scales && !aligned(a->act_scales, 16)))
        return fail(MOE_ERR_INVALID, "%s: act_q and act_scales must be 16-byte aligned", op);
    if (a->quant == MOE_QUANT_W8A16 && (a->act_q || a->act_scales))
        return fail(MOE_ERR_INVALID, "%s: MOE_QUANT_W8A16 quantises no activations: act_q and act_scales must be NULL",
                    op);

    const size_t A = (size_t)T * kf;
    uint8_t* w = static_cast<uint8_t*>(a->workspace);
    auto take = [&](size_t n) { uint8_t* p = w; w += align256(n); return p; };
    int32_t* ids = reinterpret_cast<int32_t*>(take(A * 4));
    float* wts = reinterpret_cast<float*>(take(A * 4));
    int32_t* counts = reinterpret_cast<int32_t*>(take((size_t)Ef * 4));
    int32_t* offsets = reinterpret_cast<int32_t*>(take((size_t)(Ef + 1) * 4));
    int32_t* sorted = reinterpret_cast<int32_t*>(take(A * 4));
    int32_t* pos = reinterpret_cast<int32_t*>(take(A * 4));
    uint8_t* rws = w;
    w += route_ws_bytes(T, Ef, kf, 1);
    uint8_t* xq = take((size_t)T * H);
    uint8_t* xs = take((size_t)T * (H / 32));
    if (a->act_q) xq = a->act_q;
    if (a->act_scales) xs = a->act_scales;
    uint8_t* fws = w;
    w += moe::ffn_workspace_bytes(T, H, I, Ef, kf);
    void* eo = take(A * H * ((a->flags & MOE_FUSED_EXPERT_OUT_BF16) ? 2 : 4));
    if (a->topk_ids) ids = a->topk_ids;
    if (a->topk_weights) wts = a->topk_weights;
    if (a->expert_counts) counts = a->expert_counts;

    hipStream_t st = static_cast<hipStream_t>(a->stream);
    hipEvent_t ev[MOE_STAGES + 1] = {};
    if (a->stage_events)
        for (int i = 0; i <= MOE_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(a->stage_events[i]);
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (e == hipSuccess && ev[i]) e = hipEventRecord(ev[i], st);
    };
    const int bf = (a->flags & MOE_FUSED_EXPERT_OUT_BF16) ? 1 : 0;
    const bool mx = a->quant == MOE_QUANT_MXFP8 || a->quant == MOE_QUANT_W4A8;
    const bool w16 = a->quant == MOE_QUANT_W8A16;   // the bf16 hidden states go in as they are
    moe::FfnArgs f{T, kf, H, I, Ef, xq, xs, counts, offsets, sorted, a->w13, a->w13_scale, a->w2, a->w2_scale, eo, bf,
                   a->quant, w16 ? a->hidden_states : nullptr};
    const moe::FfnWs fw = moe::carve_ffn_ws(f, fws);
    const moe::FfnPlan plan = moe::ffn_plan(T, kf, Ef, a->quant);
    moe::RouteCfg rcfg = route_cfg(&a->route, T, a->prelude != nullptr);
    rcfg.ld = kf;
    rcfg.shared_id = sh ? E : -1;
    // the activation quantisation (128- or 32-column groups) runs inside the routing kernel,
    // one wave per token
    mark(0);
    mark(1);
    float* pl = reinterpret_cast<float*>(rws + route_chunk_bytes(T, Ef, kf));
    if (e == hipSuccess && a->prelude)
        e = moe::launch_gate_prelude(a->hidden_states, T, H, E, a->prelude->norm_weight, a->prelude->router_weight,
                                     a->prelude->rms_eps, pl, st);
    if (e == hipSuccess)
        e = moe::launch_route(a->prelude ? pl : a->router_logits, rcfg, a->prelude ? a->prelude->per_expert_scale : nullptr,
                              ids, wts, st,
                              w16 ? moe::QuantOut{nullptr, 0, nullptr, nullptr, 128}
                                  : moe::QuantOut{a->hidden_states, H, xq, xs, mx ? 32 : 128});
    mark(2);
    if (e == hipSuccess)
        e = moe::launch_dispatch(ids, (int)A, Ef, reinterpret_cast<int32_t*>(rws), counts, offsets, sorted, pos, st,
                                 plan.BM, fw.tiles, fw.ntiles, plan.pairs_down ? fw.pairs : nullptr, fw.npairs);
    mark(3);
    if (e == hipSuccess) e = moe::launch_grouped_ffn(f, fws, st, ev[4], true, plan.pairs_down != 0);
    mark(5);
    if (e == hipSuccess) e = moe::launch_combine(eo, bf, pos, wts, T, kf, H, a->y, st);
    mark(6);
    if (e != hipSuccess) return hip_fail(op, e);
    return ok();
}

}  // extern "C"
