"""Unit check of the SwiGLU + E4M3 re-quantisation step of the gate+up epilogue (the SiLU
products quantised to E4M3 per (row, 128 group) of the fp8_grouped_tc_w8a8.rs module doc).

moe_grouped_ffn's test outputs expose the float32 h the epilogue computed and the re-quantised
hq / hs copied out of the down GEMM's operand layout.  The oracle's quantiser applied to that
same float32 h must give the device's bytes exactly (float32 values are exact in float64, so
both sides quantise identical numbers); h itself is compared with the oracle's float64 h, and
the share of hq codes that match the oracle's own (from its float64 h) is reported.  Every
gate+up kernel is covered: 16-row decode tiles, the persistent and per-tile 128-row kernels,
256-row items, the plain 128-row kernels, the MX kernels and the W8A16 kernel.
"""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import codec, moe as omoe, mx as omx, w8a16 as ow

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"

FP8_CASES = {
    "cfg1_decode_tiles": W.CONFIGS[1],
    "cfg2_decode_gemma4": W.CONFIGS[2],
    "cfg3_persistent_128": W.CONFIGS[3],
    "I128_tile_pairs": W.Workload(130, "bm128kb1", T=700, H=256, I=128, E=4, k=2),
    "plain_128_H384": W.Workload(128, "bm128p", T=600, H=384, I=256, E=8, k=3),
    "per_tile_128_kb1": W.Workload(135, "pfkb1", T=800, H=128, I=256, E=16, k=2),
    "tile_pairs_skewed": W.Workload(131, "p2s", T=1500, H=256, I=256, E=8, k=4, bias="normal1.5"),
}


def _device(wl, scheme):
    """Route, quantise the activations and run the grouped FFN with and without the test
    outputs; returns (routing dict on the host, h, hq, hs (host arrays))."""
    x, logits, pre = HN.device_inputs(wl)
    if scheme == "fp8":
        w = HN.device_weights(wl)
    elif scheme == "w8a16":
        w = HN.device_weights(wl).with_quant(M.MOE_QUANT_W8A16)
    else:
        w = HN.device_weights_mx(wl, M.QUANT_SCHEMES[scheme])
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits, hidden_states=x if pre else None,
                    prelude=pre)
    if scheme == "fp8":
        xq, xs = M.moe_quant_act(x)
        args = (xq, xs, r, w, wl.k)
        kw = {}
    elif scheme == "w8a16":
        args = (None, None, r, w, wl.k)
        kw = {"x": x}
    else:
        xq, xs = M.moe_quant_act_mx(x)
        args = (xq, xs, r, w, wl.k)
        kw = {}
    eo, h, hq, hs = M.moe_grouped_ffn(*args, debug=True, **kw)
    eo0 = M.moe_grouped_ffn(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(eo, eo0), "the kernels that store h must compute the same expert outputs"
    return {k: v.cpu().numpy() for k, v in r.items()}, h, hq, hs


def _check(wl, scheme, tokens=None, extra_rows=()):
    print("requant", scheme, W.describe(wl), flush=True)
    r, h, hq, hs = _device(wl, scheme)
    A = wl.T * wl.k
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=None if wl.prelude else W.router_logits(wl))
    ok = margin >= 1e-5
    assert np.array_equal(r["topk_ids"][ok], ids_ref[ok])
    tok = np.arange(wl.T) if tokens is None else tokens(ids_ref)
    tok = tok[ok[tok]]
    slots = r["assign_pos"].reshape(wl.T, wl.k)[tok].reshape(-1).astype(np.int64)   # oracle row order
    rows = np.unique(np.concatenate([slots, np.asarray(extra_rows, dtype=np.int64)])) if A > 65536 else np.arange(A)
    ridx = torch.from_numpy(rows).to(DEV)
    h_rows = h[ridx].cpu().numpy().astype(np.float64)
    hq_rows = hq[ridx].cpu()
    # 1. the device's bytes are the oracle's quantisation of the device's own float32 h
    if scheme == "w8a16":
        assert np.array_equal(ow.bf16_rne(h_rows), hq_rows.float().numpy().astype(np.float64))
    else:
        q_ref, s_ref = codec.quant_rows_128(h_rows) if scheme == "fp8" else omx.quant_rows_32(h_rows)
        hs_rows = hs[ridx].cpu().numpy()
        bad = np.nonzero((q_ref != hq_rows.numpy()).any(axis=1) | (s_ref != hs_rows).any(axis=1))[0]
        assert len(bad) == 0, f"{len(bad)} rows differ, first sorted rows {rows[bad[:8]]}"
    # 2. h against the oracle's float64 h on the sampled tokens' rows
    fm = {"fp8": omoe.forward, "w8a16": ow.forward}.get(scheme, omx.forward)
    ref = fm(xf, ids_ref, w_ref, None, tokens=tok, ffn_map=HN.oracle_ffn_map(wl, scheme), biases=HN.oracle_biases(wl))
    h_dev = h[torch.from_numpy(slots).to(DEV)].cpu().numpy().astype(np.float64)
    d = np.abs(h_dev - ref["h"])
    ratio = d / np.maximum(ref["h_err"], 1e-300)
    rowmax = np.maximum(np.abs(ref["h"]).max(axis=1, keepdims=True), 1e-300)
    print(f"  {len(rows)} rows byte-checked; |h - h_oracle|: max {(d / rowmax).max():.2e} of the row max, "
          f"max {ratio.max():.3f} of the oracle's error bound h_err", flush=True)
    assert ratio.max() <= 1.0, "the device's h is outside the oracle's error bound"
    # 3. the device's codes differ from the oracle's own re-quantisation only at decisions that
    #    lie within h_err of a tie (the allowance of the output bar)
    if scheme != "w8a16":
        hq_dev = hq[torch.from_numpy(slots).to(DEV)].cpu().numpy()
        grp = 128 if scheme == "fp8" else 32
        elem, scale = codec.near_tie_flips(ref["h"], grp, ref["h_err"])
        allowed = elem != 0
        for r_, c0, _ in scale:
            allowed[r_, c0:c0 + grp] = True
        # compared as values: a tiny h whose sign differs rounds to +0 on one side and -0 on
        # the other, two codes of the same value
        if scheme == "fp8":
            hs_dev = hs[torch.from_numpy(slots).to(DEV)].cpu().numpy()
            diff = codec.dequant_rows_128(hq_dev, hs_dev) != codec.dequant_rows_128(ref["hq"], ref["hs"])
        else:
            hs_dev = hs[torch.from_numpy(slots).to(DEV)].cpu().numpy()
            diff = omx.dequant_rows_32(hq_dev, hs_dev) != omx.dequant_rows_32(ref["hq"], ref["hs"])
        print(f"  hq values equal to the oracle's: {1 - diff.mean():.6f}; {diff.sum()} differ, "
              f"{allowed.sum()} decisions within h_err of a tie", flush=True)
        assert not (diff & ~allowed).any(), "a value differs from the oracle's away from any near tie"


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_requant_unit_fp8(name):
    _check(FP8_CASES[name], "fp8")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [4, 5])
def test_requant_unit_fp8_prefill_sampled(cfg):
    # every row of the first and the last 256-row item, and the rows of the tokens covering
    # every 128-row tile of every expert
    wl = W.CONFIGS[cfg]
    A = wl.T * wl.k
    _check(wl, "fp8", tokens=lambda ids: HN.item_sample_tokens(ids, wl.E, every=256),
           extra_rows=np.concatenate([np.arange(256), np.arange(A - 256, A)]))


@pytest.mark.parametrize("scheme", ["mxfp8", "w4a8"])
@pytest.mark.parametrize("wl", [W.CONFIGS[2], W.Workload(131, "p2s", T=1500, H=256, I=256, E=8, k=4, bias="normal1.5"),
                                W.Workload(138, "mxt", T=700, H=512, I=384, E=8, k=3),
                                W.Workload(141, "mxpf", T=300, H=512, I=384, E=16, k=4)],
                         ids=["decode_gemma4", "skewed_prefill_pairs", "pairs_I384", "tiles128_I384"])
def test_requant_unit_mx(scheme, wl):
    _check(wl, scheme)


def test_requant_unit_w8a16():
    _check(W.CONFIGS[2], "w8a16")
