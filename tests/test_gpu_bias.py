"""GPU parity of the optional per-expert biases (w13_bias on the gate/up sums before SwiGLU,
w2_bias on each expert's output before its routing weight; the interface table of the "Fused
MoE" page) against the oracle, through every gate/up and down kernel: the hand-worked case
of tests/golden/ffn_bias_hand.txt bit for bit, the SwiGLU + re-quantisation unit check on the
biased sums, and the whole step with the bar of the unbiased step.
"""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import moe as omoe, mx as omx, w8a16 as ow

import harness as HN
import test_gpu_requant as RQ

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"

# one case per kernel pair the planner picks (rows per expert on average in brackets)
FP8_CASES = {
    "decode_tiles": W.Workload(160, "bdec", T=40, H=256, I=256, E=8, k=2, ffn_bias=True),           # 10
    "plain_128_H384": W.Workload(161, "bplain", T=600, H=384, I=256, E=8, k=3, ffn_bias=True),     # 225, H % 256
    "persistent_gate_rb_down": W.Workload(162, "brb", T=600, H=256, I=256, E=32, k=2, ffn_bias=True),  # 37
    "persistent_gate_pair_down": W.Workload(163, "bpd", T=640, H=512, I=256, E=16, k=2, ffn_bias=True),  # 80
    "tile_pairs": W.Workload(164, "bp2", T=1500, H=256, I=256, E=8, k=4, bias="normal1.5", ffn_bias=True),
    "per_tile_kb1": W.Workload(165, "bkb1", T=800, H=128, I=256, E=16, k=2, ffn_bias=True),        # 100, KB 1
}


def _hand_weights(scheme):
    H = I = 128
    w13 = torch.cat([torch.full((1, H, I), 2.0 ** -7), torch.full((1, H, I), 2.0 ** -6)], dim=2).to(DEV)
    w2 = torch.full((1, I, H), 2.0 ** -7, device=DEV)
    b13 = torch.cat([torch.ones(1, I), -torch.ones(1, I)], dim=1).to(DEV)
    b2 = torch.full((1, H), 0.25, device=DEV)
    if scheme in ("mxfp8", "w4a8"):
        w = M.pack_weights_mx(w13, w2, M.QUANT_SCHEMES[scheme])
    else:
        q13, s13 = M.moe_quant_weight_blocks(w13)
        q2, s2 = M.moe_quant_weight_blocks(w2)
        w = M.PackedWeights.from_logical(q13, s13, q2, s2)
        if scheme == "w8a16":
            w = w.with_quant(M.MOE_QUANT_W8A16)
    return w.with_biases(b13, b2)


@pytest.mark.parametrize("scheme,y_exp", [("fp8", 2.0), ("mxfp8", 2.0), ("w4a8", 2.0), ("w8a16", 2.0078125)])
def test_bias_hand_case_through_device(scheme, y_exp):
    # tests/golden/ffn_bias_hand.txt: x = 1, gate 2^-7 + 1, up 2^-6 - 1, down 2^-7 + 0.25:
    # h = silu(2) -> E4M3 1.75 at scale 2^-7 (its 32-column groups give the same scale), so
    # y = 1.75 + 0.25 = 2; under W8A16 h rounds to the bf16 1.7578125 and o = 2.0078125, which
    # lies halfway between the bf16 neighbours 2 and 2.015625 of the output and rounds to even,
    # 2.  Every weight is a power of two that E2M1 also holds exactly.
    H = 128
    x = torch.ones(1, H, dtype=torch.bfloat16, device=DEV)
    logits = torch.zeros(1, 1, dtype=torch.float32, device=DEV)
    y = M.moe_fused(M.route_params(1, 1), x, _hand_weights(scheme), router_logits=logits)
    y_bf16 = torch.tensor(y_exp, dtype=torch.float64).to(torch.bfloat16).item()
    assert torch.all(y.float() == y_bf16), y.float().unique()
    # the float32 expert output holds o itself
    w = _hand_weights(scheme)
    r = M.moe_route(M.route_params(1, 1), 1, router_logits=logits)
    if scheme == "w8a16":
        eo = M.moe_grouped_ffn(None, None, r, w, 1, x=x)
    else:
        xq, xs = M.moe_quant_act(x) if scheme == "fp8" else M.moe_quant_act_mx(x)
        eo = M.moe_grouped_ffn(xq, xs, r, w, 1)
    assert torch.all(eo == y_exp), eo.unique()
    # and both biases off gives the unbiased hand value (1.5, 1.4609375 under W8A16)
    w0 = _hand_weights(scheme).with_biases(None, None)
    y0 = M.moe_fused(M.route_params(1, 1), x, w0, router_logits=logits)
    assert torch.all(y0.float() == (1.4609375 if scheme == "w8a16" else 1.5))


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_bias_requant_unit_fp8(name):
    RQ._check(FP8_CASES[name], "fp8")


@pytest.mark.parametrize("scheme", ["mxfp8", "w4a8", "w8a16"])
def test_bias_requant_unit_mx_w8a16(scheme):
    RQ._check(W.Workload(166, "bmx", T=48, H=512, I=256, E=8, k=3, ffn_bias=True), scheme)


def _fused_check(wl, scheme="fp8", tokens=None, eo_bf16=False):
    x, logits, pre = HN.device_inputs(wl)
    if scheme == "fp8":
        w = HN.device_weights(wl)
    elif scheme == "w8a16":
        w = HN.device_weights(wl).with_quant(M.MOE_QUANT_W8A16)
    else:
        w = HN.device_weights_mx(wl, M.QUANT_SCHEMES[scheme])
    assert w.w13_bias is not None and w.w2_bias is not None
    y, ids, _, _ = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, prelude=pre, return_routing=True,
                               shared_expert=bool(wl.shared), expert_out_bf16=eo_bf16)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=None if wl.prelude else W.router_logits(wl))
    ok = margin >= 1e-5
    assert np.array_equal(ids[:, :wl.k][ok], ids_ref[ok])
    tok = np.arange(wl.T) if tokens is None else tokens(ids_ref)
    tok = tok[ok[tok]]
    fm = {"fp8": omoe.forward, "w8a16": ow.forward}.get(scheme, omx.forward)
    if wl.shared:
        ids_ref = np.concatenate([ids_ref, np.full((wl.T, 1), wl.E, dtype=ids_ref.dtype)], axis=1)
        w_ref = np.concatenate([np.asarray(w_ref, dtype=np.float64), np.ones((wl.T, 1))], axis=1)
    ref = fm(xf, ids_ref, w_ref, None, tokens=tok, ffn_map=HN.oracle_ffn_map(wl, scheme),
             biases=HN.oracle_biases(wl))
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[tok], ref["y"], wl.name, ref["y_bound"])
    print(f"  {scheme} {W.describe(wl)}: rel fro {fro:.2e} rel max {mx:.2e}", flush=True)
    # the biases are not lost in the noise: without them the output is far off
    y0 = M.moe_fused(HN.device_params(wl), x, w.with_biases(None, None), router_logits=logits, prelude=pre,
                     shared_expert=bool(wl.shared), expert_out_bf16=eo_bf16)
    f0, _ = HN.rel_errors(HN.bf16_to_f64(y0)[tok], ref["y"])
    assert f0 > 20 * max(fro, 1e-4), (f0, fro)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_bias_fused_fp8(name):
    _fused_check(FP8_CASES[name])


@pytest.mark.parametrize("scheme", ["mxfp8", "w4a8", "w8a16"])
def test_bias_fused_mx_w8a16(scheme):
    _fused_check(W.Workload(167, "bfmx", T=70, H=384, I=256, E=8, k=3, bias="normal1.5", ffn_bias=True), scheme)


@pytest.mark.parametrize("scheme", ["mxfp8", "w4a8"])
@pytest.mark.parametrize("wl", [W.Workload(169, "bmxp", T=400, H=512, I=256, E=4, k=2, ffn_bias=True),
                                W.Workload(170, "bmxt", T=200, H=512, I=256, E=16, k=4, ffn_bias=True)],
                         ids=["pairs", "tiles128"])
def test_bias_mx_prefill_tiles(scheme, wl):
    # the larger MX tiles (H % 256 == 0): 256-row items, and 128-row tiles below 128 rows per expert
    RQ._check(wl, scheme)
    _fused_check(wl, scheme)


def test_bias_fused_decode_gemma4_full():
    # the Gemma-4-shaped decode step (RMSNorm + router prelude, 128 experts, top-8) with biases
    _fused_check(W.CONFIGS[2].replace(ffn_bias=True))


def test_bias_fused_shared_expert_and_bf16_expert_out():
    # the shared expert's biases are row E of each table
    wl = W.Workload(168, "bsh", T=300, H=256, I=256, E=8, k=2, shared=1, ffn_bias=True)
    _fused_check(wl)
    _fused_check(wl, eo_bf16=True)


def test_bias_separate_entry_points_match_fused():
    wl = FP8_CASES["persistent_gate_pair_down"]
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    xq, xs = M.moe_quant_act(x)
    eo = M.moe_grouped_ffn(xq, xs, r, w, wl.k)
    y = M.moe_combine(eo, r["assign_pos"], r["topk_weights"])
    yf = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits)
    assert torch.equal(y, yf)
    # a down bias alone adds exactly b2[e] to every expert-output row of expert e
    w_d = w.with_biases(None, w.w2_bias)
    w_n = w.with_biases(None, None)
    eo_d = M.moe_grouped_ffn(xq, xs, r, w_d, wl.k)
    eo_n = M.moe_grouped_ffn(xq, xs, r, w_n, wl.k)
    counts = r["expert_counts"].cpu().numpy()
    e_of_row = torch.from_numpy(np.repeat(np.arange(wl.E), counts)).to(DEV)
    assert torch.equal(eo_d, eo_n + w.w2_bias[e_of_row])
