// C ABI of the routed FP8 MoE step: launch order and workspace carving.  The arguments of
// every entry point are checked first by the plain C++ validators of moe_host.cpp, so a
// rejected call enqueues nothing.
#include <cstdio>
#include <mutex>

#include "../../include/moe_fp8.h"
#include "moe_common.h"
#include "moe_internal.h"

namespace {

using moe::host::fail;
using moe::host::ok;

int hip_fail(const char* op, hipError_t e) {
    return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", op, (int)e, hipGetErrorString(e));
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

// route + dispatch with all pointers already validated; ws holds route_ws_bytes
hipError_t do_route(const moe_route_params* p, int T, const float* logits, const uint16_t* hidden, int H,
                    const moe_gate_prelude* g, int flags, int32_t* ids, float* wts, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, uint8_t* ws, hipStream_t st) {
    const int E = p->num_experts, k = p->top_k;
    const int64_t A = (int64_t)T * k;
    int32_t* chunk_ws = reinterpret_cast<int32_t*>(ws);
    uint8_t* after = ws + moe::route_chunk_bytes(T, E, k);
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

}  // namespace

extern "C" {

const char* moe_last_error(void) { return moe::host::last_error(); }

size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t top_k, int32_t H, int32_t with_prelude) {
    (void)H;
    if (T < 1 || E < 1 || top_k < 1) return 0;
    return moe::route_ws_bytes(T, E, top_k, with_prelude);
}

int moe_route(const moe_route_params* p, int32_t T, const float* router_logits, const uint16_t* hidden_states,
              int32_t H, const moe_gate_prelude* prelude, int32_t flags, int32_t* topk_ids, float* topk_weights,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_assign, int32_t* assign_pos,
              void* workspace, size_t workspace_bytes, void* stream) {
    const void* const outs[6] = {topk_ids, topk_weights, expert_counts, expert_offsets, sorted_assign, assign_pos};
    int rc = moe::host::check_route(p, T, router_logits, hidden_states, H, prelude, flags, outs, workspace,
                                    workspace_bytes);
    if (rc) return rc;
    const bool given = flags & MOE_ROUTE_IDS_GIVEN;
    const hipError_t e = do_route(p, T, router_logits, hidden_states, H, given ? nullptr : prelude, flags, topk_ids,
                                  topk_weights, expert_counts, expert_offsets, sorted_assign, assign_pos,
                                  static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_route", e);
    return ok();
}

int moe_quant_act(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                  void* stream) {
    int rc = moe::host::check_quant_act("moe_quant_act", x, rows, cols, ld, xq, xs, 128);
    if (rc) return rc;
    const hipError_t e = moe::launch_quant_act(x, rows, cols, ld, xq, xs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_quant_act", e);
    return ok();
}

int moe_quant_weight_blocks(const float* w, int32_t E, int32_t K, int32_t N, uint8_t* q, uint8_t* scale,
                            void* stream) {
    int rc = moe::host::check_quant_weight_blocks(w, E, K, N, q, scale);
    if (rc) return rc;
    const hipError_t e = moe::launch_quant_weight_blocks(w, E, K, N, q, scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_quant_weight_blocks", e);
    return ok();
}

int moe_prepack_weights(const uint8_t* w, int32_t E, int32_t K, int32_t N, uint8_t* packed, void* stream) {
    int rc = moe::host::check_prepack(w, E, K, N, packed);
    if (rc) return rc;
    const hipError_t e = moe::launch_prepack(w, E, K, N, packed, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_prepack_weights", e);
    return ok();
}

int moe_quant_act_mx(const uint16_t* x, int32_t rows, int32_t cols, int64_t ld, uint8_t* xq, uint8_t* xs,
                     void* stream) {
    int rc = moe::host::check_quant_act("moe_quant_act_mx", x, rows, cols, ld, xq, xs, 32);
    if (rc) return rc;
    const hipError_t e = moe::launch_quant_act_mx(x, rows, cols, ld, xq, xs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_quant_act_mx", e);
    return ok();
}

int moe_quant_weight_mx(const float* w, int32_t E, int32_t K, int32_t N, int32_t wfmt, uint8_t* q, uint8_t* scale,
                        void* stream) {
    int rc = moe::host::check_quant_weight_mx(w, E, K, N, wfmt, q, scale);
    if (rc) return rc;
    const hipError_t e = moe::launch_quant_weight_mx(w, E, K, N, wfmt, q, scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_quant_weight_mx", e);
    return ok();
}

int moe_prepack_weights_mx(const uint8_t* q, const uint8_t* scale, int32_t E, int32_t K, int32_t N, int32_t wfmt,
                           uint8_t* packed, uint8_t* packed_scale, void* stream) {
    int rc = moe::host::check_prepack_mx(q, scale, E, K, N, wfmt, packed, packed_scale);
    if (rc) return rc;
    const hipError_t e = moe::launch_prepack_mx(q, scale, E, K, N, wfmt, packed, packed_scale,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_prepack_weights_mx", e);
    return ok();
}

size_t moe_ffn_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
    if (T < 1 || H < 1 || I < 128 || E < 1 || k < 1) return 0;
    return moe::ffn_workspace_bytes(T, H, I, E, k);
}

int moe_grouped_ffn(const moe_ffn_args* a) {
    int rc = moe::host::check_grouped_ffn(a);
    if (rc) return rc;
    const bool w16 = a->quant == MOE_QUANT_W8A16;
    moe::FfnArgs f{a->T, a->k, a->H, a->I, a->E, a->xq, a->xs, a->expert_counts, a->expert_offsets,
                   a->sorted_assign, a->w13, a->w13_scale, a->w2, a->w2_scale, a->expert_out,
                   a->out_dtype == MOE_DTYPE_BF16, a->quant, w16 ? a->x : nullptr,
                   a->debug_h, a->debug_hq, a->debug_hs, a->w13_bias, a->w2_bias};
    const hipError_t e = moe::launch_grouped_ffn(f, a->workspace, static_cast<hipStream_t>(a->stream));
    if (e != hipSuccess) return hip_fail("moe_grouped_ffn", e);
    return ok();
}

int moe_combine(const void* expert_out, int32_t dtype, const int32_t* assign_pos, const float* topk_weights,
                int32_t T, int32_t k, int32_t H, uint16_t* y, void* stream) {
    int rc = moe::host::check_combine(expert_out, dtype, assign_pos, topk_weights, T, k, H, y);
    if (rc) return rc;
    const hipError_t e = moe::launch_combine(expert_out, dtype == MOE_DTYPE_BF16, assign_pos, topk_weights, T, k, H,
                                             y, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("moe_combine", e);
    return ok();
}

size_t moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t flags) {
    if (T < 1 || H < 128 || I < 128 || E < 1 || k < 1) return 0;
    const int sh = (flags & MOE_FUSED_SHARED_EXPERT) ? 1 : 0;   // one more expert, one more slot per token
    return moe::fused_ws_layout(T, H, I, E + sh, k + sh, (flags & MOE_FUSED_EXPERT_OUT_BF16) ? 2 : 4).end;
}

}  // extern "C"

namespace {

// The whole step on validated arguments, with its temporaries carved from `base` (at least
// fused_ws_layout(...).end bytes of device memory, 256-byte aligned).
int run_fused(const char* op, const moe_fused_args* a, uint8_t* base) {
    const int T = a->T, H = a->H, I = a->I, E = a->route.num_experts, k = a->route.top_k;
    // with the shared expert the FFN, dispatch and combine see E + 1 experts and k + 1 slots
    const int sh = (a->flags & MOE_FUSED_SHARED_EXPERT) ? 1 : 0, Ef = E + sh, kf = k + sh;
    const int bf = (a->flags & MOE_FUSED_EXPERT_OUT_BF16) ? 1 : 0;
    const moe::FusedWsLayout L = moe::fused_ws_layout(T, H, I, Ef, kf, bf ? 2 : 4);
    int32_t* ids = a->topk_ids ? a->topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
    float* wts = a->topk_weights ? a->topk_weights : reinterpret_cast<float*>(base + L.wts);
    int32_t* counts = a->expert_counts ? a->expert_counts : reinterpret_cast<int32_t*>(base + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    int32_t* pos = reinterpret_cast<int32_t*>(base + L.pos);
    uint8_t* rws = base + L.route;
    uint8_t* xq = a->act_q ? a->act_q : base + L.xq;
    uint8_t* xs = a->act_scales ? a->act_scales : base + L.xs;
    uint8_t* fws = base + L.ffn;
    void* eo = base + L.eo;
    const size_t A = (size_t)T * kf;

    hipStream_t st = static_cast<hipStream_t>(a->stream);
    hipEvent_t ev[MOE_STAGES + 1] = {};
    if (a->stage_events)
        for (int i = 0; i <= MOE_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(a->stage_events[i]);
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (e == hipSuccess && ev[i]) e = hipEventRecord(ev[i], st);
    };
    const bool mx = a->quant == MOE_QUANT_MXFP8 || a->quant == MOE_QUANT_W4A8;
    const bool w16 = a->quant == MOE_QUANT_W8A16;   // the bf16 hidden states go in as they are
    moe::FfnArgs f{T, kf, H, I, Ef, xq, xs, counts, offsets, sorted, a->w13, a->w13_scale, a->w2, a->w2_scale, eo, bf,
                   a->quant, w16 ? a->hidden_states : nullptr, nullptr, nullptr, nullptr, a->w13_bias, a->w2_bias};
    const moe::FfnWs fw = moe::carve_ffn_ws(f, fws);
    const moe::FfnPlan plan = moe::ffn_plan(T, kf, Ef, a->quant, H);
    moe::RouteCfg rcfg = route_cfg(&a->route, T, a->prelude != nullptr);
    rcfg.ld = kf;
    rcfg.shared_id = sh ? E : -1;
    // the activation quantisation (128- or 32-column groups) runs inside the routing kernel,
    // one wave per token
    mark(0);
    mark(1);
    float* pl = reinterpret_cast<float*>(rws + moe::route_chunk_bytes(T, Ef, kf));
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

// Scratch memory of moe_fused_static: a file-scope device array that every GPU the library
// runs on holds until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in symbol): its device address is looked up once per device,
// with that device current, and kept.
constexpr size_t kStaticScratchBytes = (size_t)MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// this device's address of `scratch` (nullptr and *err set on failure)
uint8_t* scratch_on_current_device(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_fused_static(const moe_fused_args* a) {
    int rc = moe::host::check_fused_static(a, kStaticScratchBytes);
    if (rc) return rc;
    hipError_t e = hipSuccess;
    uint8_t* base = scratch_on_current_device(&e);
    if (!base) return hip_fail("moe_fused_static", e);
    return run_fused("moe_fused_static", a, base);
}

int moe_fused(const moe_fused_args* a) {
    int rc = moe::host::check_fused(a);
    if (rc) return rc;
    return run_fused("moe_fused", a, static_cast<uint8_t*>(a->workspace));
}

}  // extern "C"
