// CPU driver for the library's host-side arithmetic and argument validation (moe_host.cpp),
// built without HIP under the address and undefined-behaviour sanitizers by
// tests/test_host_sanitized.py.  Exits non-zero on the first failed check.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../mixture_experts_fp8_amd/csrc/moe_plan.h"

using namespace moe;

static int g_checks = 0;
#define CHECK(cond)                                                                             \
    do {                                                                                        \
        ++g_checks;                                                                             \
        if (!(cond)) {                                                                          \
            std::fprintf(stderr, "%s:%d: CHECK(%s) failed; last error: %s\n", __FILE__, __LINE__, \
                         #cond, host::last_error());                                            \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

// pointers that are never dereferenced: validation only looks at their values
static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(0x10000000u + off); }
template <typename T>
static T* fp(uintptr_t off = 0) { return static_cast<T*>(fake(off)); }

static moe_route_params rp(int E, int k) {
    moe_route_params p{};
    p.num_experts = E;
    p.top_k = k;
    p.scoring = MOE_SCORING_SOFTMAX;
    p.renormalize = 1;
    p.group_count = 1;
    p.k_group = 1;
    p.group_select_mode = 0;
    p.routed_scaling_factor = 1.0f;
    return p;
}

static moe_ffn_args ffn(int T, int k, int H, int I, int E) {
    moe_ffn_args a;
    std::memset(&a, 0, sizeof a);
    a.T = T, a.k = k, a.H = H, a.I = I, a.E = E;
    a.xq = fp<uint8_t>();
    a.xs = fp<uint8_t>();
    a.expert_counts = fp<int32_t>();
    a.expert_offsets = fp<int32_t>();
    a.sorted_assign = fp<int32_t>();
    a.w13 = fp<uint8_t>();
    a.w13_scale = fp<uint8_t>();
    a.w2 = fp<uint8_t>();
    a.w2_scale = fp<uint8_t>();
    a.expert_out = fake();
    a.workspace = fake();
    a.workspace_bytes = (size_t)1 << 40;
    return a;
}

static moe_fused_args fused(int T, int H, int I, int E, int k) {
    moe_fused_args a;
    std::memset(&a, 0, sizeof a);
    a.T = T, a.H = H, a.I = I;
    a.route = rp(E, k);
    a.hidden_states = fp<uint16_t>();
    a.router_logits = fp<float>();
    a.w13 = fp<uint8_t>();
    a.w13_scale = fp<uint8_t>();
    a.w2 = fp<uint8_t>();
    a.w2_scale = fp<uint8_t>();
    a.y = fp<uint16_t>();
    a.workspace = fake();
    a.workspace_bytes = (size_t)1 << 40;
    return a;
}

static void layouts() {
    const int shapes[][5] = {{64, 256, 512, 8, 2},      {32, 2816, 768, 128, 8}, {2048, 768, 1152, 256, 8},
                             {4096, 7168, 2048, 256, 8}, {16384, 4096, 1536, 128, 8}, {1, 128, 128, 1, 1},
                             {300, 128, 128, 1024, 8}};
    for (auto& s : shapes) {
        const int T = s[0], H = s[1], I = s[2], E = s[3], k = s[4];
        for (int q = 0; q < 4; ++q) {
            const FfnPlan p = ffn_plan(T, k, E, q, H);
            CHECK(p.BM == 16 || p.BM == 128);
            // the MX schemes take 128-row tiles (and pairs) only with 256-column down blocks, and
            // pairs for both GEMMs or neither; W8A16 stays on 16-row tiles
            CHECK(q == kQuantFp8Block128 || p.pairs == p.pairs_down);
            CHECK(q != kQuantW8A16 || p.BM == 16);
            CHECK(!(q == kQuantMxfp8 || q == kQuantW4A8) || p.BM == 16 || H % 256 == 0);
            CHECK((int64_t)p.ntiles_max * p.BM >= (int64_t)T * k);   // every row has a tile slot
            CHECK(!p.pairs || p.pairs_down);
            const FfnWsLayout l = ffn_ws_layout(T, H, I, E, k, q);
            const size_t r[] = {l.tiles, l.ntiles, l.hq, l.hs, l.bs, l.pairs, l.npairs, l.end};
            for (size_t i = 0; i + 1 < sizeof r / sizeof r[0]; ++i) CHECK(r[i] <= r[i + 1] && r[i] % 256 == 0);
            const size_t rows = (size_t)p.ntiles_max * p.BM;
            CHECK(l.hs - l.hq >= rows * I * (q == kQuantW8A16 ? 2 : 1));
            CHECK(l.bs - l.hs >= rows * (I / 32));
            CHECK(l.pairs - l.bs >= (p.BM == 128 ? ffn_rb_scale_table_bytes(H, I, E) : 0));
            CHECK(l.npairs - l.pairs >= (size_t)p.npairs_max * 16);
            CHECK(ffn_workspace_bytes(T, H, I, E, k) >= l.end);
        }
        for (int eo = 2; eo <= 4; eo += 2) {
            const FusedWsLayout f = fused_ws_layout(T, H, I, E, k, eo);
            const size_t A = (size_t)T * k;
            CHECK(f.wts - f.ids >= A * 4 && f.counts - f.wts >= A * 4 && f.offsets - f.counts >= (size_t)E * 4);
            CHECK(f.sorted - f.offsets >= (size_t)(E + 1) * 4 && f.pos - f.sorted >= A * 4 && f.route - f.pos >= A * 4);
            CHECK(f.xq - f.route >= route_ws_bytes(T, E, k, 1) && f.xs - f.xq >= (size_t)T * H);
            CHECK(f.ffn - f.xs >= (size_t)T * (H / 32) && f.eo - f.ffn >= ffn_workspace_bytes(T, H, I, E, k));
            CHECK(f.end - f.eo >= A * H * eo && f.end % 256 == 0);
        }
        CHECK(route_ws_bytes(T, E, k, 1) >= route_ws_bytes(T, E, k, 0) + (size_t)T * E * 4);
    }
}

static void route_checks() {
    const void* outs[6] = {fake(), fake(), fake(), fake(), fake(), fake()};
    moe_route_params p = rp(8, 2);
    CHECK(host::check_route(&p, 4, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), 1 << 20) == MOE_OK);
    CHECK(host::check_route(nullptr, 4, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), 1 << 20) == MOE_ERR_INVALID);
    CHECK(host::check_route(&p, 0, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), 1 << 20) == MOE_ERR_INVALID);
    CHECK(host::check_route(&p, 4, nullptr, nullptr, 0, nullptr, 0, outs, fake(), 1 << 20) == MOE_ERR_INVALID);
    CHECK(host::check_route(&p, 4, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), 16) == MOE_ERR_WORKSPACE);
    CHECK(host::check_route(&p, 4, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(4), 1 << 20) == MOE_ERR_INVALID);
    CHECK(host::check_route(&p, 4, fp<float>(), nullptr, 0, nullptr, 8, outs, fake(), 1 << 20) == MOE_ERR_INVALID);
    CHECK(host::check_route(&p, 1 << 28, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), 1 << 20) ==
          MOE_ERR_UNSUPPORTED);
    const void* bad[6] = {fake(), nullptr, fake(), fake(), fake(), fake()};
    CHECK(host::check_route(&p, 4, fp<float>(), nullptr, 0, nullptr, 0, bad, fake(), 1 << 20) == MOE_ERR_INVALID);
    moe_gate_prelude g{fp<float>(), fp<float>(), nullptr, 1e-6f};
    CHECK(host::check_route(&p, 4, nullptr, fp<uint16_t>(), 64, &g, 0, outs, fake(), 1 << 20) == MOE_OK);
    CHECK(host::check_route(&p, 4, nullptr, fp<uint16_t>(), 66, &g, 0, outs, fake(), 1 << 20) == MOE_ERR_UNSUPPORTED);
    CHECK(host::check_route(&p, 1 << 20, nullptr, fp<uint16_t>(), 4096, &g, 0, outs, fake(), (size_t)1 << 40) ==
          MOE_ERR_UNSUPPORTED);
    g.rms_eps = -1.f;
    CHECK(host::check_route(&p, 4, nullptr, fp<uint16_t>(), 64, &g, 0, outs, fake(), 1 << 20) == MOE_ERR_INVALID);
    const int bad_params[][5] = {{8, 9, 1, 1, 0}, {8, 0, 1, 1, 0}, {0, 1, 1, 1, 0}, {2048, 1, 1, 1, 0},
                                 {12, 2, 5, 1, 0}, {16, 2, 4, 5, 0}, {16, 5, 4, 1, 0}, {8, 2, 8, 2, 1},
                                 {8, 2, 2, 1, 3}};
    for (auto& b : bad_params) {
        moe_route_params q = rp(b[0], b[1]);
        q.group_count = b[2];
        q.k_group = b[3];
        q.group_select_mode = b[4];
        CHECK(host::check_route(&q, 4, fp<float>(), nullptr, 0, nullptr, 0, outs, fake(), (size_t)1 << 30) != MOE_OK);
    }
}

static void ffn_checks() {
    moe_ffn_args a = ffn(8, 2, 256, 256, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);
    CHECK(host::check_grouped_ffn(nullptr) == MOE_ERR_INVALID);
    a = ffn(8, 2, 200, 256, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_UNSUPPORTED);
    a = ffn(8, 5, 256, 256, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_INVALID);
    // the 32-bit products
    a = ffn((int)((1LL << 31) / 256), 2, 256, 256, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_UNSUPPORTED && std::strstr(host::last_error(), "T * H"));
    a = ffn((int)((1LL << 31) / 256 - 1), 2, 256, 256, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);
    a = ffn(8, 2, 32768, 32768, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_UNSUPPORTED && std::strstr(host::last_error(), "2 * I * H"));
    a = ffn(8, 2, 32768, 32640, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);
    a = ffn(1 << 28, 2, 128, 128, 4);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_UNSUPPORTED);
    a = ffn(8, 2, 256, 256, 4);
    a.workspace_bytes = 10;
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_WORKSPACE);
    a = ffn(8, 2, 256, 256, 4);
    a.quant = 4;
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_INVALID);
    a.quant = MOE_QUANT_W8A16;
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_INVALID);   // x missing
    a.x = fp<uint16_t>(8);
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_UNSUPPORTED);
    a.x = fp<uint16_t>();
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);
    a.debug_h = fp<float>();
    a.debug_hq = fp<uint8_t>();
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);   // W8A16 takes no debug_hs
    a.quant = 0;
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_INVALID);
    a.debug_hs = fp<uint8_t>();
    CHECK(host::check_grouped_ffn(&a) == MOE_OK);
    a.debug_h = nullptr;
    CHECK(host::check_grouped_ffn(&a) == MOE_ERR_INVALID);
}

static void fused_checks() {
    moe_fused_args a = fused(4, 256, 256, 8, 2);
    CHECK(host::check_fused(&a) == MOE_OK);
    CHECK(host::check_fused(nullptr) == MOE_ERR_INVALID);
    a.flags = 4;
    CHECK(host::check_fused(&a) == MOE_ERR_INVALID);
    a = fused(4, 100, 256, 8, 2);
    CHECK(host::check_fused(&a) == MOE_ERR_UNSUPPORTED);
    a = fused(4, 256, 256, 8, 2);
    a.router_logits = nullptr;
    CHECK(host::check_fused(&a) == MOE_ERR_INVALID);
    a = fused(4, 256, 256, 8, 2);
    a.hidden_states = fp<uint16_t>(4);
    CHECK(host::check_fused(&a) == MOE_ERR_UNSUPPORTED);
    a = fused(4, 256, 256, 8, 2);
    a.workspace_bytes = 1000;
    CHECK(host::check_fused(&a) == MOE_ERR_WORKSPACE);
    a = fused((int)((1LL << 31) / 256), 256, 256, 8, 2);
    CHECK(host::check_fused(&a) == MOE_ERR_UNSUPPORTED);
    a = fused(4, 256, 256, 1024, 8);
    a.flags = MOE_FUSED_SHARED_EXPERT;
    CHECK(host::check_fused(&a) == MOE_ERR_UNSUPPORTED);
    a = fused(4, 256, 256, 8, 2);
    a.quant = MOE_QUANT_W8A16;
    a.act_q = fp<uint8_t>();
    CHECK(host::check_fused(&a) == MOE_ERR_INVALID);
    a.quant = 0;
    a.act_q = fp<uint8_t>(8);
    CHECK(host::check_fused(&a) == MOE_ERR_INVALID);
}

static void static_checks() {
    // the scratch-array variant: no workspace, and steps above the scratch size are rejected
    const size_t lim = (size_t)64 << 20;
    moe_fused_args a = fused(32, 2816, 768, 128, 8);
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    CHECK(host::check_fused_static(&a, lim) == MOE_OK);
    CHECK(host::check_fused(&a) == MOE_ERR_WORKSPACE);
    a.workspace = fake();
    CHECK(host::check_fused_static(&a, lim) == MOE_ERR_INVALID);
    a.workspace = nullptr;
    a.workspace_bytes = 16;
    CHECK(host::check_fused_static(&a, lim) == MOE_ERR_INVALID);
    a = fused(2048, 768, 1152, 256, 8);
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    CHECK(host::check_fused_static(&a, lim) == MOE_ERR_UNSUPPORTED && std::strstr(host::last_error(), "scratch"));
    CHECK(fused_ws_layout(2048, 768, 1152, 256, 8, 4).end > lim);
    a = fused(4, 100, 256, 8, 2);   // the other checks still apply
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    CHECK(host::check_fused_static(&a, lim) == MOE_ERR_UNSUPPORTED);
}

static void helper_checks() {
    CHECK(host::check_quant_act("q", fp<uint16_t>(), 4, 128, 128, fp<uint8_t>(), fp<uint8_t>(), 128) == MOE_OK);
    CHECK(host::check_quant_act("q", fp<uint16_t>(), 4, 100, 128, fp<uint8_t>(), fp<uint8_t>(), 128) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(host::check_quant_act("q", fp<uint16_t>(), 4, 256, 128, fp<uint8_t>(), fp<uint8_t>(), 128) ==
          MOE_ERR_INVALID);
    CHECK(host::check_quant_act("q", fp<uint16_t>(), 4, 64, 64, fp<uint8_t>(), fp<uint8_t>(), 32) == MOE_OK);
    CHECK(host::check_quant_weight_blocks(fp<float>(), 2, 100, 128, fp<uint8_t>(), fp<uint8_t>()) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(host::check_prepack(fp<uint8_t>(), 1, 128, 32, fp<uint8_t>(16)) == MOE_ERR_INVALID);
    CHECK(host::check_prepack(fp<uint8_t>(), 1, 128, 32, fp<uint8_t>(1 << 20)) == MOE_OK);
    CHECK(host::check_quant_weight_mx(fp<float>(), 1, 64, 64, 2, fp<uint8_t>(), fp<uint8_t>()) == MOE_ERR_INVALID);
    CHECK(host::check_prepack_mx(fp<uint8_t>(), fp<uint8_t>(1 << 24), 1, 128, 64, 1, fp<uint8_t>(16),
                                 fp<uint8_t>(3 << 24)) == MOE_ERR_INVALID);
    CHECK(host::check_combine(fake(), 0, fp<int32_t>(), fp<float>(), 4, 2, 132, fp<uint16_t>()) == MOE_OK);
    CHECK(host::check_combine(fake(), 1, fp<int32_t>(), fp<float>(), 4, 2, 130, fp<uint16_t>()) ==
          MOE_ERR_UNSUPPORTED);
    CHECK(host::check_combine(fake(), 0, fp<int32_t>(), fp<float>(), 1 << 27, 4, 128, fp<uint16_t>()) ==
          MOE_ERR_UNSUPPORTED);
}

int main() {
    layouts();
    route_checks();
    ffn_checks();
    fused_checks();
    static_checks();
    helper_checks();
    // the message buffer is bounded: an overlong message is truncated, never overrun
    std::vector<char> big(4096, 'x');
    big.back() = 0;
    host::fail(MOE_ERR_INVALID, "%s", big.data());
    CHECK(std::strlen(host::last_error()) < 512);
    host::ok();
    CHECK(host::last_error()[0] == 0);
    std::printf("host checks ok: %d\n", g_checks);
    return 0;
}
