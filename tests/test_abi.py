"""The C ABI without a GPU: the library loads, exports every function include/moe_fp8.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import mixture_experts_fp8_amd as M
from mixture_experts_fp8_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")

FAKE = 0x10000000   # a non-NULL, 256-aligned pointer value; never dereferenced on error paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for f in ["moe_route", "moe_quant_act", "moe_grouped_ffn", "moe_combine", "moe_fused",
              "moe_workspace_size", "moe_last_error", "moe_prepack_weights", "moe_quant_weight_blocks",
              "moe_quant_act_mx", "moe_quant_weight_mx", "moe_prepack_weights_mx"]:
        assert f in fns


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    for f in declared_functions():
        assert hasattr(lib, f), f
    assert sorted(declared_functions()) == sorted(B.EXPORTED)


def _route(p, T=4, logits=FAKE, flags=0, ws=FAKE, ws_bytes=1 << 20, prelude=None, hidden=None, H=0, outs=FAKE):
    return M.lib().moe_route(ctypes.byref(p), T, logits, hidden, H, prelude, flags, outs, outs, outs, outs, outs,
                             outs, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(num_experts=8, top_k=9), B.MOE_ERR_INVALID, "top_k"),
    (dict(num_experts=8, top_k=0), B.MOE_ERR_INVALID, "top_k"),
    (dict(num_experts=0, top_k=1), B.MOE_ERR_INVALID, "num_experts"),
    (dict(num_experts=2048, top_k=1), B.MOE_ERR_UNSUPPORTED, "exceeds max"),
    (dict(num_experts=12, top_k=2, group_count=5), B.MOE_ERR_INVALID, "divisible"),
    (dict(num_experts=16, top_k=2, group_count=4, k_group=5), B.MOE_ERR_INVALID, "k_group"),
    (dict(num_experts=16, top_k=5, group_count=4, k_group=1), B.MOE_ERR_INVALID, "kept groups"),
    (dict(num_experts=8, top_k=2, group_count=8, k_group=2, group_select_mode=1), B.MOE_ERR_INVALID, "at least 2"),
    (dict(num_experts=8, top_k=2, group_count=2, k_group=1, group_select_mode=3), B.MOE_ERR_INVALID, "group_select_mode"),
    (dict(num_experts=8, top_k=2, routed_scaling_factor=float("inf")), B.MOE_ERR_INVALID, "finite"),
])
def test_route_param_validation(kw, code, needle):
    p = M.route_params(**kw)
    assert _route(p) == code
    assert needle in M.moe_last_error()


def test_route_other_errors():
    p = M.route_params(8, 2)
    assert _route(p, T=0) == B.MOE_ERR_INVALID
    assert _route(p, logits=None) == B.MOE_ERR_INVALID and "router_logits" in M.moe_last_error()
    assert _route(p, outs=None) == B.MOE_ERR_INVALID
    assert _route(p, ws_bytes=16) == B.MOE_ERR_WORKSPACE and "workspace too small" in M.moe_last_error()
    assert _route(p, ws=FAKE + 4) == B.MOE_ERR_INVALID and "aligned" in M.moe_last_error()
    assert _route(p, flags=8) == B.MOE_ERR_INVALID
    pre = B.GatePrelude(None, None, None, 1e-6)
    assert _route(p, logits=None, prelude=ctypes.byref(pre), hidden=FAKE, H=64) == B.MOE_ERR_INVALID
    pre = B.GatePrelude(FAKE, FAKE, None, -1.0)
    assert _route(p, logits=None, prelude=ctypes.byref(pre), hidden=FAKE, H=64) == B.MOE_ERR_INVALID
    pre = B.GatePrelude(FAKE, FAKE, None, 1e-6)
    assert _route(p, logits=None, prelude=ctypes.byref(pre), hidden=FAKE, H=66) == B.MOE_ERR_UNSUPPORTED
    assert "multiple of 4" in M.moe_last_error()
    pre = B.GatePrelude(FAKE + 4, FAKE, None, 1e-6)
    assert _route(p, logits=None, prelude=ctypes.byref(pre), hidden=FAKE, H=64) == B.MOE_ERR_UNSUPPORTED


def test_quant_act_validation():
    L = M.lib()
    assert L.moe_quant_act(None, 4, 128, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert L.moe_quant_act(FAKE, 4, 100, 128, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_act(FAKE, 4, 256, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID     # ld < cols
    assert L.moe_quant_act(FAKE + 2, 4, 128, 128, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_act(FAKE, 0, 128, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID


def test_weight_helpers_validation():
    L = M.lib()
    assert L.moe_quant_weight_blocks(FAKE, 2, 100, 128, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_weight_blocks(None, 2, 128, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert L.moe_prepack_weights(FAKE, 1, 128, 24, FAKE + (1 << 20), None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_prepack_weights(FAKE, 1, 128, 32, FAKE + 16, None) == B.MOE_ERR_INVALID   # overlap
    assert "overlap" in M.moe_last_error()


def test_mx_helpers_validation():
    L = M.lib()
    assert L.moe_quant_act_mx(FAKE, 4, 48, 48, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED   # cols % 32
    assert L.moe_quant_act_mx(None, 4, 64, 64, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert L.moe_quant_act_mx(FAKE, 4, 64, 32, FAKE, FAKE, None) == B.MOE_ERR_INVALID      # ld < cols
    assert L.moe_quant_weight_mx(FAKE, 1, 64, 64, 2, FAKE, FAKE, None) == B.MOE_ERR_INVALID  # wfmt
    assert L.moe_quant_weight_mx(FAKE, 1, 48, 64, 0, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_weight_mx(FAKE, 1, 64, 63, 1, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_prepack_weights_mx(FAKE, FAKE + (1 << 24), 1, 96, 64, 0, FAKE + (2 << 24), FAKE + (3 << 24),
                                    None) == B.MOE_ERR_UNSUPPORTED   # K % 128
    assert L.moe_prepack_weights_mx(FAKE, FAKE + (1 << 24), 1, 128, 64, 1, FAKE + 16, FAKE + (3 << 24),
                                    None) == B.MOE_ERR_INVALID and "overlap" in M.moe_last_error()


def _ffn(**over):
    a = dict(T=8, k=2, H=256, I=256, E=4, xq=FAKE, xs=FAKE, expert_counts=FAKE, expert_offsets=FAKE,
             sorted_assign=FAKE, w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE, expert_out=FAKE,
             out_dtype=0, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(over)
    s = B.FfnArgs(**a)
    return M.lib().moe_grouped_ffn(ctypes.byref(s))


def test_grouped_ffn_validation():
    assert _ffn(H=200) == B.MOE_ERR_UNSUPPORTED and "multiple of 128" in M.moe_last_error()
    assert _ffn(I=1000) == B.MOE_ERR_UNSUPPORTED
    assert _ffn(k=5) == B.MOE_ERR_INVALID
    assert _ffn(w2=None) == B.MOE_ERR_INVALID
    assert _ffn(w13=FAKE + 8) == B.MOE_ERR_INVALID
    assert _ffn(out_dtype=7) == B.MOE_ERR_INVALID
    assert _ffn(workspace_bytes=10) == B.MOE_ERR_WORKSPACE
    assert _ffn(quant=4) == B.MOE_ERR_INVALID and "quant" in M.moe_last_error()
    # W8A16 takes the bf16 hidden states in x (xq / xs unused), 16-byte aligned
    assert _ffn(quant=3) == B.MOE_ERR_INVALID and "x must not be NULL" in M.moe_last_error()
    assert _ffn(quant=3, x=FAKE + 8) == B.MOE_ERR_UNSUPPORTED and "aligned" in M.moe_last_error()
    assert _ffn(quant=0, xq=None) == B.MOE_ERR_INVALID
    assert M.lib().moe_grouped_ffn(None) == B.MOE_ERR_INVALID
    # the test outputs come as a set: debug_h with debug_hq (and debug_hs except for W8A16)
    assert _ffn(debug_hq=FAKE) == B.MOE_ERR_INVALID and "only with debug_h" in M.moe_last_error()
    assert _ffn(debug_h=FAKE, debug_hq=FAKE) == B.MOE_ERR_INVALID and "debug_hs" in M.moe_last_error()
    assert _ffn(debug_h=FAKE, debug_hq=FAKE, debug_hs=FAKE, workspace_bytes=10) == B.MOE_ERR_WORKSPACE
    # the optional float32 biases: 4-byte aligned; valid ones pass on to the workspace check
    assert _ffn(w13_bias=FAKE + 2) == B.MOE_ERR_INVALID and "w13_bias" in M.moe_last_error()
    assert _ffn(w2_bias=FAKE + 1) == B.MOE_ERR_INVALID
    assert _ffn(w13_bias=FAKE + 4, w2_bias=FAKE, workspace_bytes=10) == B.MOE_ERR_WORKSPACE


def test_32bit_offset_limits():
    # products the kernels address with 32-bit offsets are bounded before any launch
    assert _ffn(T=(1 << 31) // 256, H=256) == B.MOE_ERR_UNSUPPORTED and "T * H" in M.moe_last_error()
    # just below the bounds the shapes pass (a too-small workspace then stops the call)
    assert _ffn(T=(1 << 31) // 256 - 1, H=256, workspace_bytes=10) == B.MOE_ERR_WORKSPACE
    assert _ffn(H=32768, I=32768) == B.MOE_ERR_UNSUPPORTED and "2 * I * H" in M.moe_last_error()
    assert _ffn(H=32768, I=32640, workspace_bytes=10) == B.MOE_ERR_WORKSPACE
    assert _ffn(T=1 << 28, k=2) == B.MOE_ERR_UNSUPPORTED and "2^29" in M.moe_last_error()
    assert _fused(T=(1 << 31) // 256) == B.MOE_ERR_UNSUPPORTED and "T * H" in M.moe_last_error()
    p = M.route_params(8, 8)
    assert _route(p, T=1 << 26) == B.MOE_ERR_UNSUPPORTED and "2^29" in M.moe_last_error()
    L = M.lib()
    assert L.moe_combine(FAKE, 0, FAKE, FAKE, 1 << 27, 4, 128, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    pre = B.GatePrelude(FAKE, FAKE, None, 1e-6)
    assert _route(M.route_params(8, 2), T=1 << 20, logits=None, prelude=ctypes.byref(pre), hidden=FAKE,
                  H=4096) == B.MOE_ERR_UNSUPPORTED


def test_combine_validation():
    L = M.lib()
    assert L.moe_combine(FAKE, 0, FAKE, FAKE, 4, 2, 130, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(FAKE, 1, FAKE, FAKE, 4, 2, 130, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(FAKE, 0, FAKE, FAKE, 4, 2, 128, FAKE + 4, None) == B.MOE_ERR_UNSUPPORTED   # y alignment
    assert L.moe_combine(FAKE, 3, FAKE, FAKE, 4, 2, 128, FAKE, None) == B.MOE_ERR_INVALID
    assert L.moe_combine(None, 0, FAKE, FAKE, 4, 2, 128, FAKE, None) == B.MOE_ERR_INVALID


def _fused(**over):
    p = over.pop("route", M.route_params(8, 2))
    a = dict(T=4, H=256, I=256, route=p, hidden_states=FAKE, router_logits=FAKE, prelude=None, w13=FAKE,
             w13_scale=FAKE, w2=FAKE, w2_scale=FAKE, y=FAKE, topk_ids=None, topk_weights=None,
             expert_counts=None, flags=0, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(over)
    return M.lib().moe_fused(ctypes.byref(B.FusedArgs(**a)))


def test_fused_validation():
    assert _fused(route=M.route_params(8, 9)) == B.MOE_ERR_INVALID
    assert _fused(H=100) == B.MOE_ERR_UNSUPPORTED
    assert _fused(router_logits=None) == B.MOE_ERR_INVALID
    assert _fused(y=None) == B.MOE_ERR_INVALID
    assert _fused(flags=4) == B.MOE_ERR_INVALID
    assert _fused(workspace_bytes=1000) == B.MOE_ERR_WORKSPACE
    assert _fused(hidden_states=FAKE + 4) == B.MOE_ERR_UNSUPPORTED
    assert _fused(quant=-1) == B.MOE_ERR_INVALID
    assert _fused(quant=4) == B.MOE_ERR_INVALID
    # the optional quantised-activation outputs: 16-byte aligned, and none for W8A16
    assert _fused(act_q=FAKE + 8) == B.MOE_ERR_INVALID
    assert _fused(act_scales=FAKE + 4) == B.MOE_ERR_INVALID
    assert _fused(quant=B.MOE_QUANT_W8A16, act_q=FAKE) == B.MOE_ERR_INVALID
    assert "W8A16" in M.moe_last_error()
    assert _fused(w13_bias=FAKE + 2) == B.MOE_ERR_INVALID and "bias" in M.moe_last_error()
    assert _fused(w2_bias=FAKE + 6, workspace_bytes=1000) == B.MOE_ERR_INVALID
    assert _fused(w13_bias=FAKE, w2_bias=FAKE + 4, workspace_bytes=1000) == B.MOE_ERR_WORKSPACE
    # 1024 routed experts plus the shared one exceed the dispatch's expert limit
    assert _fused(route=M.route_params(1024, 8), flags=B.MOE_FUSED_SHARED_EXPERT) == B.MOE_ERR_UNSUPPORTED
    assert "exceeds max" in M.moe_last_error()
    assert M.lib().moe_fused(None) == B.MOE_ERR_INVALID


def test_fused_static_validation():
    # the scratch-array entry point: a workspace is an error; a step above the scratch size is
    # unsupported (both rejected before any launch, so the fake pointers are never used)
    L = M.lib()
    a = B.FusedArgs(T=4, H=256, I=256, route=M.route_params(8, 2), hidden_states=FAKE, router_logits=FAKE,
                    prelude=None, w13=FAKE, w13_scale=FAKE, w2=FAKE, w2_scale=FAKE, y=FAKE, topk_ids=None,
                    topk_weights=None, expert_counts=None, flags=0, workspace=FAKE, workspace_bytes=1 << 20,
                    stream=None)
    assert L.moe_fused_static(ctypes.byref(a)) == B.MOE_ERR_INVALID and "NULL" in M.moe_last_error()
    a.workspace, a.workspace_bytes = None, 0
    a.T, a.H, a.I, a.route = 2048, 768, 1152, M.route_params(256, 8)
    assert L.moe_fused_static(ctypes.byref(a)) == B.MOE_ERR_UNSUPPORTED and "scratch" in M.moe_last_error()
    assert L.moe_fused_static(None) == B.MOE_ERR_INVALID


def test_workspace_sizes_are_monotone_and_cover_parts():
    L = M.lib()
    for (T, H, I, E, k) in [(64, 256, 512, 8, 2), (32, 2816, 768, 128, 8), (4096, 7168, 2048, 256, 8)]:
        full = L.moe_workspace_size(T, H, I, E, k, 0)
        assert full >= L.moe_ffn_workspace_size(T, H, I, E, k) + L.moe_route_workspace_size(T, E, k, H, 1)
        assert L.moe_workspace_size(T, H, I, E, k, B.MOE_FUSED_EXPERT_OUT_BF16) < full
        # the shared expert adds one expert and one slot per token
        assert L.moe_workspace_size(T, H, I, E, k, B.MOE_FUSED_SHARED_EXPERT) > full
        assert L.moe_workspace_size(2 * T, H, I, E, k, 0) > full
    assert L.moe_workspace_size(0, 256, 256, 8, 2, 0) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libmoe_fp8.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
