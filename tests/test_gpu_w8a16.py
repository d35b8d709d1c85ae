"""GPU parity of the W8A16 scheme (E4M3 block-scaled weights, bf16 activations) against the
oracle (oracle.w8a16): routing bit for bit, the output with the bar of the FP8 step (relative
Frobenius <= 5e-3, max |err| <= 2e-2 max |y|).  The weights are the FP8 step's packed E4M3
blocks, read under MOE_QUANT_W8A16.
"""

import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import w8a16 as ow

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"

CASES = {
    "cfg1": W.CONFIGS[1],
    "T1_E1_k1": W.Workload(150, "w16one", T=1, H=128, I=128, E=1, k=1),
    "ragged": W.Workload(151, "w16ragged", T=37, H=256, I=384, E=5, k=3),
    "k_equals_E": W.Workload(152, "w16kE", T=19, H=128, I=256, E=4, k=4, renormalize=False),
    "many_tiles_skewed": W.Workload(153, "w16skew", T=300, H=384, I=256, E=8, k=3, bias="normal1.5"),
    "prelude_small": W.Workload(154, "w16pre", T=9, H=512, I=256, E=16, k=4, prelude=True),
}


def _weights(wl):
    return HN.device_weights(wl).with_quant(M.MOE_QUANT_W8A16)


def _check(wl, tokens=None):
    x, logits, pre = HN.device_inputs(wl)
    w = _weights(wl)
    y, ids, _, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, prelude=pre,
                                    return_routing=True)
    torch.cuda.synchronize()
    ids, counts = ids.cpu().numpy(), counts.cpu().numpy()
    assert counts.sum() == wl.T * wl.k
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=None if wl.prelude else W.router_logits(wl))
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    tok = np.arange(wl.T) if tokens is None else (tokens(ids_ref) if callable(tokens) else np.asarray(tokens))
    tok = tok[ok[tok]]
    ref = ow.forward(xf, ids_ref, w_ref, None, tokens=tok, ffn_map=HN.oracle_ffn_map(wl, "w8a16"))
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[tok], ref["y"], wl.name, ref["y_bound"])
    print(f"  rel fro {fro:.2e} rel max {mx:.2e}", flush=True)
    return y


@pytest.mark.parametrize("name", list(CASES))
def test_w8a16_fused_small(name):
    wl = CASES[name]
    print("w8a16 fused", name, W.describe(wl), flush=True)
    _check(wl)


def test_w8a16_decode_gemma4_full():
    wl = W.CONFIGS[2]
    print("w8a16 fused full", W.describe(wl), flush=True)
    _check(wl)


@pytest.mark.timeout(900)
def test_w8a16_dsv3_prefill_sampled():
    # the DeepSeek-V3-shaped prefill (H/128 = 56 K blocks, 256 experts) on the 16-row tiles:
    # tokens covering every 128 rows of every expert, plus every 64th
    wl = W.CONFIGS[4]
    print("w8a16 fused sampled", W.describe(wl), flush=True)
    _check(wl, tokens=lambda ids: HN.item_sample_tokens(ids, wl.E))


def test_w8a16_hand_ffn_through_device():
    # tests/golden/ffn_w8a16_hand.txt: x = 1, gate 2^-7, up 2^-6, down 2^-7 -> y = 1.4609375
    H = I = 128
    x = torch.ones(1, H, dtype=torch.bfloat16, device=DEV)
    w13 = torch.cat([torch.full((1, H, I), 2.0 ** -7), torch.full((1, H, I), 2.0 ** -6)], dim=2).to(DEV)
    w2 = torch.full((1, I, H), 2.0 ** -7, device=DEV)
    q13, s13 = M.moe_quant_weight_blocks(w13)
    q2, s2 = M.moe_quant_weight_blocks(w2)
    w = M.PackedWeights.from_logical(q13, s13, q2, s2).with_quant(M.MOE_QUANT_W8A16)
    logits = torch.zeros(1, 1, dtype=torch.float32, device=DEV)
    y = M.moe_fused(M.route_params(1, 1), x, w, router_logits=logits)
    assert torch.all(y.float() == 1.4609375)


def test_w8a16_separate_entry_points_match_fused():
    wl = CASES["many_tiles_skewed"]
    x, logits, _ = HN.device_inputs(wl)
    w = _weights(wl)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    eo = M.moe_grouped_ffn(None, None, r, w, wl.k, x=x)
    y = M.moe_combine(eo, r["assign_pos"], r["topk_weights"])
    yf = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits)
    assert torch.equal(y, yf)
    eob = M.moe_grouped_ffn(None, None, r, w, wl.k, out_dtype=torch.bfloat16, x=x)
    assert torch.equal(eob, eo.to(torch.bfloat16))


def test_w8a16_bf16_expert_out_and_shared_expert():
    wl = W.Workload(155, "w16sh", T=40, H=256, I=256, E=8, k=2, shared=1)
    x, logits, _ = HN.device_inputs(wl)
    w = _weights(wl)
    p = HN.device_params(wl)
    y32 = M.moe_fused(p, x, w, router_logits=logits, shared_expert=True)
    y16 = M.moe_fused(p, x, w, router_logits=logits, shared_expert=True, expert_out_bf16=True)
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=W.router_logits(wl))
    T = wl.T
    ids_all = np.concatenate([ids_ref, np.full((T, 1), wl.E, dtype=ids_ref.dtype)], axis=1)
    w_all = np.concatenate([np.asarray(w_ref, dtype=np.float64), np.ones((T, 1))], axis=1)
    ref = ow.forward(xf, ids_all, w_all, None, ffn_map=HN.oracle_ffn_map(wl, "w8a16"))
    ok = margin >= 1e-5
    for y in (y32, y16):
        HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], "w8a16 shared", ref["y_bound"][ok])


def test_w8a16_rejects_missing_activations():
    wl = CASES["ragged"]
    x, logits, _ = HN.device_inputs(wl)
    w = _weights(wl)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    with pytest.raises(ValueError):
        M.moe_grouped_ffn(None, None, r, w, wl.k)
