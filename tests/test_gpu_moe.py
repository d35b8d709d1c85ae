"""GPU parity of the grouped FFN and of the fused step against the oracle.

Small shapes compare every output; the full workload sizes run in the same launch
configuration the benchmark times and compare a sample of tokens that the oracle
computes one by one (a row of y depends only on its own token).
"""

import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import codec, moe as omoe, routing as orouting

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"

SMALL = {
    "cfg1": W.CONFIGS[1],
    "T1_E1_k1": W.Workload(120, "one", T=1, H=128, I=128, E=1, k=1),
    "ragged": W.Workload(121, "ragged", T=37, H=256, I=384, E=5, k=3),
    "k_equals_E": W.Workload(122, "kE", T=19, H=128, I=256, E=4, k=4, renormalize=False),
    "staged_tiles_skewed": W.Workload(123, "bm128s", T=640, H=256, I=256, E=16, k=6, bias="normal1.5"),
    "plain_tiles_H384": W.Workload(128, "bm128p", T=600, H=384, I=256, E=8, k=3),
    "staged_tiles_K_not_multiple_of_3": W.Workload(129, "bm128k", T=700, H=512, I=640, E=8, k=2),
    "bm128_path": W.Workload(124, "bm128", T=1100, H=256, I=384, E=8, k=2),
    "staged_tiles_single_k_block": W.Workload(130, "bm128kb1", T=700, H=256, I=128, E=4, k=2),
    # experts averaging >= 256 rows: 256-row items (tile pairs), with single-tile pairs and
    # ragged second tiles from the skew
    "tile_pairs_skewed": W.Workload(131, "p2s", T=1500, H=256, I=256, E=8, k=4, bias="normal1.5"),
    "tile_pairs_zipf_kb6": W.Workload(132, "p2z", T=900, H=768, I=384, E=6, k=2, bias="zipf"),
    # experts averaging 25..127 rows: 128-row tiles, the persistent gate/up kernel for
    # 2 <= H/128 <= 32 (several tiles per workgroup on this few-item grid only when skewed)
    # and the per-tile kernel for a single K block
    "persistent_tiles_skewed": W.Workload(133, "ppS", T=900, H=512, I=384, E=32, k=3, bias="normal1.5"),
    "persistent_tiles_kb12": W.Workload(134, "pp12", T=700, H=1536, I=256, E=16, k=2),
    # two or three items in all: most XCD shares of the persistent kernel's work queues are empty
    "persistent_tiles_few_items": W.Workload(171, "ppfew", T=200, H=256, I=128, E=2, k=1),
    "staged_tiles_kb1": W.Workload(135, "pfkb1", T=800, H=128, I=256, E=16, k=2),
    "sigmoid_groups": W.Workload(125, "grp", T=96, H=384, I=256, E=32, k=4, scoring="sigmoid", group_count=4,
                                 k_group=2, group_select_mode=1, routed_scaling_factor=2.5),
    "prelude_small": W.Workload(126, "pre", T=9, H=512, I=256, E=16, k=4, prelude=True),
    # the largest expert count the routing and dispatch kernels take (E = 1024), through the
    # single-workgroup dispatch (A <= 4096) and the chunked one
    "E1024_single_wg_dispatch": W.Workload(138, "e1k", T=300, H=128, I=128, E=1024, k=8),
    "E1024_chunked_dispatch": W.Workload(139, "e1kc", T=1200, H=128, I=256, E=1024, k=8, bias="normal1.5"),
}


def _run_fused(wl, weights=None, expert_out_bf16=False, x=None, logits=None, pre=None):
    if x is None:
        x, logits, pre = HN.device_inputs(wl)
    w = weights or HN.device_weights(wl)
    y, ids, wts, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, prelude=pre,
                                      expert_out_bf16=expert_out_bf16, return_routing=True)
    torch.cuda.synchronize()
    return y, ids.cpu().numpy(), wts.cpu().numpy(), counts.cpu().numpy(), w


def _oracle(wl, tokens=None):
    x = W.hidden_bf16(wl)
    xf = W.bf16_to_f64(x)
    logits = None if wl.prelude else W.router_logits(wl)
    ids, w, margin = HN.oracle_route(wl, x_f64=xf, logits=logits)
    tok = np.arange(wl.T) if tokens is None else np.asarray(tokens)
    out = omoe.forward(xf, ids, w, None, tokens=tok, ffn_map=HN.oracle_ffn_map(wl))
    return out, ids, w, margin


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_small(name):
    wl = SMALL[name]
    print("fused", name, W.describe(wl), flush=True)
    y, ids, wts, counts, _ = _run_fused(wl)
    ref, ids_ref, w_ref, margin = _oracle(wl)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    assert counts.sum() == wl.T * wl.k
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], name, ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mx:.2e}", flush=True)


def test_grouped_ffn_unit_cfg1():
    wl = W.CONFIGS[1]
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    xq, xs = M.moe_quant_act(x)
    eo = M.moe_grouped_ffn(xq, xs, r, w, wl.k)
    ref, ids_ref, _, _ = _oracle(wl)
    assert np.array_equal(r["topk_ids"].cpu().numpy(), ids_ref)
    pos = r["assign_pos"].cpu().numpy().astype(np.int64)
    got = eo.cpu().numpy().astype(np.float64)[pos]          # back to flat (t, j) order
    HN.assert_output_close(got, ref["o"], "expert_out", ref["o_bound"])
    eob = M.moe_grouped_ffn(xq, xs, r, w, wl.k, out_dtype=torch.bfloat16)
    HN.assert_output_close(HN.bf16_to_f64(eob)[pos], ref["o"], "expert_out bf16", ref["o_bound"])
    y = M.moe_combine(eo, r["assign_pos"], r["topk_weights"])
    HN.assert_output_close(HN.bf16_to_f64(y), ref["y"], "combine", ref["y_bound"])


@pytest.mark.parametrize("name", ["tile_pairs_skewed", "persistent_tiles_kb12"])
def test_separate_entry_points_match_fused(name):
    # moe_route -> moe_quant_act -> moe_grouped_ffn -> moe_combine on the 256-row-item and
    # persistent-tile paths (the grouped FFN builds its own tile / pair lists here): the same
    # bits as the fused call, and the oracle's expert outputs
    wl = SMALL[name]
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    xq, xs = M.moe_quant_act(x)
    eo = M.moe_grouped_ffn(xq, xs, r, w, wl.k)
    y = M.moe_combine(eo, r["assign_pos"], r["topk_weights"])
    yf = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits)
    assert torch.equal(y, yf)
    ref, ids_ref, _, margin = _oracle(wl)
    ok = margin >= 1e-5
    assert np.array_equal(r["topk_ids"].cpu().numpy()[ok], ids_ref[ok])
    pos = r["assign_pos"].cpu().numpy().astype(np.int64)
    got = eo.cpu().numpy().astype(np.float64)[pos]          # back to flat (t, j) order
    okf = np.repeat(ok, wl.k)
    HN.assert_output_close(got[okf], ref["o"][okf], "expert_out", ref["o_bound"][okf])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_fused_activation_quant_bit_exact(cfg):
    # the fused call quantises the activations inside its routing kernel (one wave per token);
    # its E4M3 codes and UE8M0 scales must be the oracle's per-(row, 128) quantisation exactly,
    # and taking them in caller buffers must not change y
    wl = W.CONFIGS[cfg]
    print("fused act quant", W.describe(wl), flush=True)
    x, logits, pre = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    p = HN.device_params(wl)
    xq = torch.empty(wl.T, wl.H, dtype=torch.uint8, device=DEV)
    xs = torch.empty(wl.T, wl.H // 128, dtype=torch.uint8, device=DEV)
    y = M.moe_fused(p, x, w, router_logits=logits, prelude=pre, act_q=xq, act_scales=xs)
    y0 = M.moe_fused(p, x, w, router_logits=logits, prelude=pre)
    torch.cuda.synchronize()
    q_ref, s_ref = codec.quant_rows_128(W.bf16_to_f64(W.hidden_bf16(wl)))
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert torch.equal(y, y0)


def test_golden_hand_ffn_through_device():
    # x = 1, gate weights 2^-7, up 2^-6, down 2^-7 -> y = 1.5 exactly (tests/golden/ffn_hand.txt)
    H = I = 128
    x = torch.ones(1, H, dtype=torch.bfloat16, device=DEV)
    w13 = torch.cat([torch.full((1, H, I), 2.0 ** -7), torch.full((1, H, I), 2.0 ** -6)], dim=2).to(DEV)
    w2 = torch.full((1, I, H), 2.0 ** -7, device=DEV)
    q13, s13 = M.moe_quant_weight_blocks(w13)
    q2, s2 = M.moe_quant_weight_blocks(w2)
    assert s13.cpu().flatten().tolist() == [112, 113] and s2.item() == 112
    w = M.PackedWeights.from_logical(q13, s13, q2, s2)
    logits = torch.zeros(1, 1, dtype=torch.float32, device=DEV)
    y = M.moe_fused(M.route_params(1, 1), x, w, router_logits=logits)
    assert torch.all(y.float() == 1.5)


def test_all_tokens_on_one_expert_and_empty_experts():
    wl = W.Workload(127, "skew", T=300, H=256, I=256, E=16, k=2, bias="none")
    x, _, _ = HN.device_inputs(wl)
    logits = W.router_logits(wl)
    logits[:, 5] += 100.0           # expert 5 first for every token
    logits[:, 8:] -= 100.0          # experts 8..15 never chosen
    w = HN.device_weights(wl)
    y, ids, _, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits.to(DEV), return_routing=True)
    ids = ids.cpu().numpy()
    counts = counts.cpu().numpy()
    assert counts[5] == 300 and counts[8:].sum() == 0
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, _ = omoe.route_workload({"logits": logits.numpy()}, HN.oracle_params(wl))
    assert np.array_equal(ids, ids_ref)
    ref = omoe.forward(xf, ids_ref, w_ref, None, ffn_map=HN.oracle_ffn_map(wl))
    HN.assert_output_close(HN.bf16_to_f64(y), ref["y"], "skew", ref["y_bound"])


def test_determinism_and_row_independence():
    wl = W.CONFIGS[3]
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    p = HN.device_params(wl)
    y1 = M.moe_fused(p, x, w, router_logits=logits)
    y2 = M.moe_fused(p, x, w, router_logits=logits)
    assert torch.equal(y1, y2)
    # a row's bits do not depend on the other rows: rerun on a subset of tokens
    sub = torch.arange(5, wl.T, 7, device=DEV)
    ys = M.moe_fused(p, x[sub].contiguous(), w, router_logits=logits[sub].contiguous())
    assert torch.equal(ys, y1[sub])


@pytest.mark.parametrize("cfg", [2, 3])
def test_fused_workload_full(cfg):
    wl = W.CONFIGS[cfg]
    print("fused full", cfg, W.describe(wl), flush=True)
    y, ids, _, counts, w = _run_fused(wl)
    yb, ids_b, _, _, _ = _run_fused(wl, weights=w, expert_out_bf16=True)
    ref, ids_ref, _, margin = _oracle(wl)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok]) and np.array_equal(ids_b, ids)
    for out, eo in ((y, "fp32"), (yb, "bf16")):
        fro, mx = HN.assert_output_close(HN.bf16_to_f64(out)[ok], ref["y"][ok], f"cfg{cfg} {eo} expert_out",
                                         ref["y_bound"][ok])
        print(f"  {eo} expert_out: rel fro {fro:.2e} rel max {mx:.2e} active experts {(counts > 0).sum()}", flush=True)


def _fused_routing(wl):
    """The fused call with every routing output: y (with float32 and with bf16 expert outputs),
    ids, counts and the dispatch (offsets, sorted_assign, assign_pos) re-derived by moe_route
    from the fused call's ids."""
    x, logits, pre = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    p = HN.device_params(wl)
    y, ids, wts, counts = M.moe_fused(p, x, w, router_logits=logits, prelude=pre, return_routing=True)
    yb = M.moe_fused(p, x, w, router_logits=logits, prelude=pre, expert_out_bf16=True)
    r = M.moe_route(p, wl.T, topk_ids=ids, topk_weights=wts, device=DEV)
    torch.cuda.synchronize()
    return (y, yb), ids.cpu().numpy(), counts.cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


# The prefill shapes at full size, in the launch configuration the benchmark times: the
# oracle computes the tokens whose rows cover every 128-row tile of every expert (so every
# 256-row item and every position of the super-tile work order holds a checked row) plus
# every 64th token.  The dispatch is compared with the oracle's stable permutation of the
# same ids, bit for bit, over the whole batch.  Both expert-output dtypes are checked (the
# benchmark keeps them in bf16 for these shapes).
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [4, 5, 6])
def test_fused_workload_sampled(cfg):
    wl = W.CONFIGS[cfg]
    print("fused sampled", cfg, W.describe(wl), flush=True)
    ys, ids, counts, r = _fused_routing(wl)
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=None if wl.prelude else W.router_logits(wl))
    ok = margin >= 1e-6
    assert np.array_equal(ids[ok], ids_ref[ok]), "routing differs from the oracle on an unambiguous token"
    c_ref, o_ref, sa_ref, ap_ref = orouting.permute(ids, wl.E)
    assert np.array_equal(counts, c_ref) and np.array_equal(r["expert_counts"], c_ref)
    assert np.array_equal(r["expert_offsets"], o_ref)
    assert np.array_equal(r["sorted_assign"], sa_ref) and np.array_equal(r["assign_pos"], ap_ref)
    tokens = HN.item_sample_tokens(ids_ref, wl.E)
    tokens = tokens[ok[tokens]]
    print(f"  {len(tokens)} of {wl.T} tokens, {(~ok).sum()} near-tie routings", flush=True)
    ref = omoe.forward(xf, ids_ref, w_ref, None, tokens=tokens, ffn_map=HN.oracle_ffn_map(wl))
    for y, eo in zip(ys, ("fp32", "bf16")):
        fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[tokens], ref["y"], f"cfg{cfg} {eo} expert_out",
                                         ref["y_bound"])
        print(f"  {eo} expert_out: rel fro {fro:.2e} rel max {mx:.2e}", flush=True)


# Tile pairs at H/128 = 16 and 32 with a few hundred 256-row items over a few skewed experts:
# full pairs, ragged second tiles and single-tile pairs, several items per expert and column
# block.  Every 8th token is compared: sorted rows follow token order within an expert, so
# every 256-row item holds sampled rows.
MEDIUM = {
    "persistent_tile_pairs_kb16": W.Workload(136, "p2pk16", T=4096, H=2048, I=2048, E=4, k=2, bias="normal1.5"),
    "persistent_tile_pairs_kb32": W.Workload(137, "p2pk32", T=6144, H=4096, I=1024, E=4, k=2, bias="normal1.5"),
    # at least 512 tiles of experts averaging under 128 rows: the persistent gate/up kernel on
    # the super-tile work order (a fixed item list per workgroup), then the 256-row down items
    # (64 rows per expert on average) or the persistent 128-row down kernel (32)
    "persistent_tiles_super_order": W.Workload(172, "ppso", T=4096, H=256, I=256, E=512, k=8, bias="normal1.5"),
    "persistent_tiles_super_order_rb_down": W.Workload(173, "ppsorb", T=2048, H=256, I=256, E=512, k=8),
}


@pytest.mark.parametrize("name", list(MEDIUM))
def test_fused_medium_sampled(name):
    wl = MEDIUM[name]
    print("fused medium", name, W.describe(wl), flush=True)
    y, ids, _, counts, _ = _run_fused(wl)
    tokens = np.arange(0, wl.T, 8)
    ref, ids_ref, _, margin = _oracle(wl, tokens=tokens)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    assert counts.sum() == wl.T * wl.k
    sel = ok[tokens]
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[tokens][sel], ref["y"][sel], name, ref["y_bound"][sel])
    print(f"  rel fro {fro:.2e} rel max {mx:.2e}", flush=True)


# ---- one shared expert (weights of expert index E) run on every token in the same launches
SHARED = {
    "shared_small": W.Workload(140, "sh", T=96, H=256, I=256, E=8, k=2, shared=1),
    "shared_prelude_decode_tiles": W.Workload(141, "shd", T=9, H=512, I=256, E=16, k=4, prelude=True, shared=1),
    "shared_tile_pairs": W.Workload(142, "shp", T=700, H=256, I=384, E=4, k=2, shared=1),
    "shared_persistent_tiles": W.Workload(143, "shpp", T=600, H=512, I=256, E=32, k=3, bias="normal1.5", shared=1),
    "shared_decode_gemma4": W.CONFIGS[2].replace(cfg=144, shared=1),
}


def _check_shared(wl, tokens=None):
    x, logits, pre = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    y, ids, wts, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, prelude=pre,
                                      return_routing=True, shared_expert=True)
    torch.cuda.synchronize()
    ids, wts, counts = ids.cpu().numpy(), wts.cpu().numpy(), counts.cpu().numpy()
    E, k = wl.E, wl.k
    # column k holds the shared expert with weight 1 for every token; it has T rows
    assert ids.shape == (wl.T, k + 1) and (ids[:, k] == E).all() and (wts[:, k] == 1.0).all()
    assert counts.shape == (E + 1,) and counts[E] == wl.T and counts.sum() == wl.T * (k + 1)
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=None if wl.prelude else W.router_logits(wl))
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok, :k], ids_ref[ok])
    tok = np.arange(wl.T) if tokens is None else (tokens(ids_ref) if callable(tokens) else np.asarray(tokens))
    tok = tok[ok[tok]]
    ref = omoe.forward_shared(xf, ids_ref, w_ref, None, shared=E, tokens=tok, ffn_map=HN.oracle_ffn_map(wl))
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[tok], ref["y"], wl.name, ref["y_bound"])
    print(f"  rel fro {fro:.2e} rel max {mx:.2e}", flush=True)


@pytest.mark.parametrize("name", list(SHARED))
def test_fused_shared_expert(name):
    wl = SHARED[name]
    print("fused shared", name, W.describe(wl), flush=True)
    _check_shared(wl)


@pytest.mark.timeout(900)
def test_fused_shared_expert_dsv3_prefill_sampled():
    # the DeepSeek-V3-shaped prefill with its one shared expert (same I; the routed experts'
    # inputs and weights are the workload's own): tokens covering every 128-row tile of the
    # routed experts, and with them the shared expert's tiles at every 64th
    wl = W.CONFIGS[4].replace(shared=1)
    print("fused shared sampled", W.describe(wl), flush=True)
    _check_shared(wl, tokens=lambda ids: HN.item_sample_tokens(ids, wl.E))


# ---- seeded shape sweep: every GEMM path (16-row tiles, persistent and staged 128-row tiles,
# 256-row pairs), both scorings with and without group limits, k from 1 to 8, expert_out in
# fp32 and bf16.  The shapes come from a fixed seed, so the list is the same on every run.
def _sweep_shapes(n=14):
    r = np.random.default_rng(4242)
    out = []
    for i in range(n):
        regime = i % 4   # 0: decode tiles, 1: 128-row tiles, 2: tile pairs, 3: single K block / odd sizes
        E = int(r.choice([4, 8, 16, 32, 64]))
        k = int(r.integers(1, min(8, E) + 1))
        H = 128 * int(r.integers(1, 13))
        I = 128 * int(r.integers(1, 9))
        avg = {0: r.integers(1, 20), 1: r.integers(30, 120), 2: r.integers(140, 400), 3: r.integers(1, 300)}[regime]
        T = max(1, int(avg * E // k))
        if regime == 3:
            H = 128
        scoring = "sigmoid" if r.random() < 0.4 else "softmax"
        G = int(r.choice([g for g in (1, 2, 4) if E % g == 0 and E // g >= 2])) if scoring == "sigmoid" else 1
        kg = int(r.integers(1, G + 1)) if G > 1 else 1
        if G > 1 and kg * (E // G) < k:
            kg = G
        out.append(W.Workload(160 + i, f"sweep{i}", T=T, H=H, I=I, E=E, k=k, scoring=scoring,
                              renormalize=bool(r.random() < 0.7), group_count=G, k_group=kg,
                              group_select_mode=int(r.integers(0, 2)), routed_scaling_factor=float(r.choice([1.0, 2.5])),
                              bias=str(r.choice(["none", "normal1.5", "zipf"]))))
    return out


SWEEP = _sweep_shapes()


@pytest.mark.parametrize("i", range(len(SWEEP)))
def test_fused_shape_sweep(i):
    wl = SWEEP[i]
    bf = i % 2 == 1
    print("fused sweep", i, W.describe(wl), "expert_out bf16" if bf else "", flush=True)
    y, ids, _, counts, _ = _run_fused(wl, expert_out_bf16=bf)
    ref, ids_ref, _, margin = _oracle(wl)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    assert counts.sum() == wl.T * wl.k
    fro, mx = HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], wl.name, ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mx:.2e}", flush=True)
