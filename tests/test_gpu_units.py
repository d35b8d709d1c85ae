"""GPU parity of each entry point against the oracle, on the same seeded inputs.

Bit-exact: quantised bytes and scales, routing ids, counts, offsets and the permutation.
Tolerance: routing weights (relative 1e-5), expert outputs and y (the output bar).
"""
import numpy as np
import pytest
import torch

from gen import rng, workloads as W
from oracle import codec, moe as omoe, routing as orouting

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"


def _finite_bf16_patterns() -> np.ndarray:
    p = np.arange(65536, dtype=np.uint32)
    exp = (p >> 7) & 0xFF
    p = p[exp != 0xFF]
    return (p << 16).view(np.float32).astype(np.float64)


def _anchored_groups() -> np.ndarray:
    """Every finite bf16 value, in groups of 127 neighbours by magnitude plus an anchor
    448 * 2^(e + s) that sets the group's scale s binades above its own (s = 0..12 by 3),
    so each value is rounded in the normal and in the subnormal E4M3 range."""
    v = _finite_bf16_patterns()
    v = v[np.argsort(np.abs(v), kind="stable")]
    rs = np.random.default_rng(0)
    groups = []
    for c in range(0, len(v), 127):
        chunk = v[c:c + 127]
        e0 = int(codec.scale_exponent(np.array([np.abs(chunk).max()]))[0])
        for s in (0, 3, 6, 9, 12):
            anchor = 448.0 * 2.0 ** (e0 + s) if (e0 + s) <= 119 and np.abs(chunk).max() > 0 else 0.0
            g = np.concatenate([chunk, [anchor]])
            g = np.pad(g, (0, 128 - len(g)))
            groups.append(rs.permutation(g))
    groups.append(np.zeros(128))
    groups.append(-np.zeros(128))
    while len(groups) % 4:
        groups.append(np.zeros(128))
    return np.stack(groups).reshape(-1, 512)


def test_quant_act_all_bf16_values_bit_exact():
    x = torch.from_numpy(_anchored_groups()).to(torch.float32).to(torch.bfloat16)
    print("quant_act exhaustive rows", x.shape, flush=True)
    xq, xs = M.moe_quant_act(x.to(DEV))
    q_ref, s_ref = codec.quant_rows_128(W.bf16_to_f64(x))
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_quant_act_workload_bit_exact(cfg):
    wl = W.CONFIGS[cfg]
    x = W.hidden_bf16(wl)
    xq, xs = M.moe_quant_act(x.to(DEV))
    q_ref, s_ref = codec.quant_rows_128(W.bf16_to_f64(x))
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


def test_quant_weight_blocks_bit_exact():
    wl = W.CONFIGS[1]
    w = torch.stack([W.expert_weight_f32(wl, "w13", e) for e in range(3)])
    w[1, :128, :128] *= 1e-30          # a block near the bottom of the scale range
    w[2, 128:, 256:384] = 0.0          # an all-zero block
    q, s = M.moe_quant_weight_blocks(w.to(DEV))
    for e in range(3):
        q_ref, s_ref = codec.quant_blocks_128(w[e].double().numpy())
        assert np.array_equal(s[e].cpu().numpy(), s_ref)
        assert np.array_equal(q[e].cpu().numpy(), q_ref)


def test_prepack_layout():
    g = torch.Generator().manual_seed(0)
    E, K, N = 2, 256, 48
    w = torch.randint(0, 256, (E, K, N), dtype=torch.uint8, generator=g)
    p = M.moe_prepack_weights(w.to(DEV)).cpu().numpy()
    wn = w.numpy()
    # expected: byte (e, n16, kb, h, lane, b) = W[e][kb*128 + (lane//16)*32 + h*16 + b][n16*16 + lane%16]
    e, n16, kb, h, lane, b = np.meshgrid(np.arange(E), np.arange(N // 16), np.arange(K // 128), np.arange(2),
                                         np.arange(64), np.arange(16), indexing="ij")
    exp = wn[e, kb * 128 + (lane // 16) * 32 + h * 16 + b, n16 * 16 + lane % 16]
    assert np.array_equal(p, exp.reshape(-1))


ROUTE_CASES = {
    "cfg1": W.CONFIGS[1],
    "cfg3": W.CONFIGS[3],
    "cfg4": W.CONFIGS[4],
    "cfg5": W.CONFIGS[5],
    "softmax_no_renorm": W.CONFIGS[1].replace(cfg=101, T=300, E=64, k=6, renormalize=False,
                                              routed_scaling_factor=1.7),
    "sigmoid_flat": W.CONFIGS[1].replace(cfg=102, T=257, E=200, k=5, scoring="sigmoid", renormalize=False),
    "group_mode0": W.CONFIGS[1].replace(cfg=103, T=200, E=96, k=4, group_count=8, k_group=3,
                                        group_select_mode=0, routed_scaling_factor=0.5),
    "grouped_example": W.CONFIGS[1].replace(cfg=104, T=64, E=16, k=2, scoring="sigmoid", renormalize=False,
                                            group_count=4, k_group=1, group_select_mode=1,
                                            routed_scaling_factor=0.5),
    "softmax_group_mode1": W.CONFIGS[1].replace(cfg=105, T=128, E=256, k=8, group_count=16, k_group=5,
                                                group_select_mode=1),
    "E1024_k1": W.CONFIGS[1].replace(cfg=106, T=70, E=1024, k=1),
    "k_equals_E": W.CONFIGS[1].replace(cfg=107, T=33, E=8, k=8),
    "T1": W.CONFIGS[1].replace(cfg=108, T=1, E=5, k=3),
    # group-limited sigmoid routing on 256 experts for a decode-sized batch, 4 experts per
    # lane without renormalisation, and an odd batch past a multiple of the 4 tokens per
    # workgroup
    "small_dsv3_like": W.CONFIGS[4].replace(cfg=109, T=48),
    "small_E200_no_renorm": W.CONFIGS[1].replace(cfg=110, T=64, E=200, k=6, renormalize=False,
                                                 routed_scaling_factor=1.3),
    "T65_odd_batch": W.CONFIGS[2].replace(cfg=111, T=65, prelude=False),
}


def _check_routing(wl, got, ids_ref, w_ref, margin, tau):
    ids = got["topk_ids"].cpu().numpy()
    wts = got["topk_weights"].cpu().numpy()
    ambiguous = margin < tau
    ok = ~ambiguous
    assert np.array_equal(ids[ok], ids_ref[ok])
    np.testing.assert_allclose(wts[ok], w_ref[ok], rtol=1e-5, atol=1e-7)
    # dispatch of the device's own ids must be the stable counting sort, bit for bit
    counts, offsets, sa, ap = orouting.permute(ids, wl.E)
    assert np.array_equal(got["expert_counts"].cpu().numpy(), counts)
    assert np.array_equal(got["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(got["sorted_assign"].cpu().numpy(), sa)
    assert np.array_equal(got["assign_pos"].cpu().numpy(), ap)
    return int(ambiguous.sum())


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_and_dispatch(name):
    wl = ROUTE_CASES[name]
    print("route", name, W.describe(wl), flush=True)
    logits = W.router_logits(wl)
    ids_ref, w_ref, margin = HN.oracle_route(wl, logits=logits)
    got = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits.to(DEV))
    n_amb = _check_routing(wl, got, ids_ref, w_ref, margin, tau=1e-6)
    assert n_amb == 0


def test_route_rows_independent_of_batch():
    # a token's ids and weights do not depend on the batch around it: the first 64 tokens of
    # a 65-token batch against the same 64 tokens alone, bit for bit
    wl = W.CONFIGS[4].replace(cfg=112, T=65)
    logits = W.router_logits(wl).to(DEV)
    big = M.moe_route(HN.device_params(wl), 65, router_logits=logits)
    small = M.moe_route(HN.device_params(wl), 64, router_logits=logits[:64].contiguous())
    assert torch.equal(big["topk_ids"][:64], small["topk_ids"])
    assert torch.equal(big["topk_weights"][:64], small["topk_weights"])


def test_route_gate_prelude():
    wl = W.CONFIGS[2]
    x = W.hidden_bf16(wl)
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=W.bf16_to_f64(x))
    xd, _, pre = HN.device_inputs(wl)
    got = M.moe_route(HN.device_params(wl), wl.T, hidden_states=xd, prelude=pre)
    n_amb = _check_routing(wl, got, ids_ref, w_ref, margin, tau=1e-5)
    assert n_amb == 0


def test_route_gate_prelude_golden_hand_cases():
    # the hand-worked prelude cases of tests/golden/prelude_hand.txt through the device's
    # RMSNorm + router + top-k + softmax-over-selected kernels (x exact in bf16)
    import test_oracle_routing as tor
    for name, x, nw, eps, W_r, pe, k, ids_exp, w_exp in tor._golden_prelude():
        E, H = W_r.shape
        xd = torch.from_numpy(x[None]).to(torch.bfloat16).to(DEV)
        assert np.array_equal(xd.float().cpu().numpy()[0], x)
        pre = M.Prelude(torch.from_numpy(nw).float().to(DEV), torch.from_numpy(W_r).float().contiguous().to(DEV),
                        torch.from_numpy(pe).float().to(DEV), float(eps))
        got = M.moe_route(M.route_params(E, k), 1, hidden_states=xd, prelude=pre)
        assert got["topk_ids"].cpu().numpy()[0].tolist() == ids_exp, name
        np.testing.assert_allclose(got["topk_weights"].cpu().numpy()[0], w_exp, rtol=2e-6, err_msg=name)


def test_dispatch_of_given_ids_with_skew_and_empty_experts():
    # every token on expert 3 first, most experts empty; more than one dispatch chunk
    T, k, E = 3000, 4, 40
    r = np.random.default_rng(1)
    print("dispatch skew", T, k, E, flush=True)
    ids = np.stack([np.concatenate([[3], r.choice([e for e in range(E) if e != 3], k - 1, replace=False)])
                    for _ in range(T)]).astype(np.int32)
    ids[ids > 30] = 7                     # experts 31..39 empty
    ids[:, 1:] = np.where(ids[:, 1:] == 3, 8, ids[:, 1:])
    w = r.uniform(0, 1, (T, k)).astype(np.float32)
    got = M.moe_route(M.route_params(E, k), T, topk_ids=torch.from_numpy(ids).to(DEV),
                      topk_weights=torch.from_numpy(w).to(DEV), device=DEV)
    counts, offsets, sa, ap = orouting.permute(ids, E)
    assert np.array_equal(got["expert_counts"].cpu().numpy(), counts)
    assert np.array_equal(got["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(got["sorted_assign"].cpu().numpy(), sa)
    assert np.array_equal(got["assign_pos"].cpu().numpy(), ap)


# the scatter that forms its own bases takes up to 256 chunks of 1024 assignments and up to
# 32768 chunk counts: (32768, 8, 128) and (16384, 8, 256) sit at those limits, (32769, 8, 128)
# is one chunk past them (the three-kernel path, as the other large cases)
@pytest.mark.parametrize("T,k,E", [(75000, 4, 100), (20000, 8, 1024), (5000, 1, 3), (40000, 6, 256),
                                   (32768, 8, 128), (16384, 8, 256), (32769, 8, 128)])
def test_dispatch_many_chunks(T, k, E):
    # hundreds of dispatch chunks, expert counts that are not powers of two, E = 1024, k = 1:
    # the chunk-parallel scan and the scatter must still give the stable counting sort
    print("dispatch chunks", T, k, E, flush=True)
    r = np.random.default_rng(T + E)
    p = r.zipf(1.3, size=E).astype(np.float64)
    p /= p.sum()
    ids = np.stack([r.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0, 1, (T, k)).astype(np.float32)
    got = M.moe_route(M.route_params(E, k), T, topk_ids=torch.from_numpy(ids).to(DEV),
                      topk_weights=torch.from_numpy(w).to(DEV), device=DEV)
    counts, offsets, sa, ap = orouting.permute(ids, E)
    assert np.array_equal(got["expert_counts"].cpu().numpy(), counts)
    assert np.array_equal(got["expert_offsets"].cpu().numpy(), offsets)
    assert np.array_equal(got["sorted_assign"].cpu().numpy(), sa)
    assert np.array_equal(got["assign_pos"].cpu().numpy(), ap)


# (T, k, H): fp32 rows take 1, 2 or 4 column groups per thread at H = 384, 2816, 4096 and
# bf16 rows 1, 2, 4 at H = 2816, 4096, 8192; k = 9 runs the slot loop twice; H = 132 takes
# 8-byte column groups for bf16 rows (a length that is not a multiple of 8)
@pytest.mark.parametrize("T,k,H", [(37, 3, 384), (5, 8, 2816), (4, 9, 4096), (3, 2, 8192), (6, 3, 132)])
def test_combine_parity_on_generated_expert_out(T, k, H):
    eo = rng.normal_f32(rng.stream_key(0, 200, 0), T * k * H, 1.0).view(T * k, H)
    w = rng.uniform_f32(rng.stream_key(0, 200, 1), T * k, 0.0, 1.0).view(T, k)
    perm = torch.from_numpy(np.random.default_rng(2).permutation(T * k).astype(np.int32))
    y = M.moe_combine(eo.to(DEV), perm.to(DEV), w.to(DEV)).float().cpu().numpy()
    o_flat = eo.double().numpy()[perm.numpy().astype(np.int64)]
    y_ref = omoe.combine(o_flat, w.double().numpy())
    # float32 accumulation then one bf16 rounding: half a bf16 ulp plus the fp32 sum's error
    mag = omoe.combine(np.abs(o_flat), w.double().numpy())
    assert np.all(np.abs(y - y_ref) <= np.abs(y_ref) * 2.0 ** -8 + 1e-6 * mag)
    eob = eo.to(torch.bfloat16)
    yb = M.moe_combine(eob.to(DEV), perm.to(DEV), w.to(DEV)).float().cpu().numpy()
    ob = eob.double().numpy()[perm.numpy().astype(np.int64)]
    y_ref_b = omoe.combine(ob, w.double().numpy())
    assert np.all(np.abs(yb - y_ref_b) <= np.abs(y_ref_b) * 2.0 ** -8 + 1e-6 * omoe.combine(np.abs(ob), w.double().numpy()))


# bf16 expert outputs against the float32 ones of the same call rounded to nearest even on the
# host, bit for bit: the conversion and the lane exchange of every down kernel's bf16 store
# (256-row items FP8 and MX, 128-row tiles, 16-row decode tiles, W8A16)
BF16_OUT_CASES = {
    "fp8_pairs": (W.Workload(190, "bo_p2", T=1500, H=512, I=256, E=8, k=4, bias="normal1.5"), "fp8"),
    "fp8_tiles128": (W.Workload(191, "bo_t128", T=600, H=256, I=384, E=32, k=2), "fp8"),
    "fp8_decode": (W.Workload(192, "bo_dec", T=24, H=512, I=256, E=16, k=4), "fp8"),
    "mxfp8_pairs": (W.Workload(193, "bo_mxp2", T=600, H=512, I=384, E=8, k=3), "mxfp8"),
    "w4a8_pairs_ragged": (W.Workload(194, "bo_w4p2", T=700, H=512, I=256, E=4, k=2, bias="zipf"), "w4a8"),
    "w4a8_tiles128": (W.Workload(195, "bo_w4t", T=300, H=512, I=384, E=16, k=4), "w4a8"),
    "w8a16": (W.Workload(196, "bo_w16", T=40, H=256, I=384, E=8, k=3), "w8a16"),
}


@pytest.mark.parametrize("name", list(BF16_OUT_CASES))
def test_bf16_expert_out_is_rounded_float32(name):
    wl, scheme = BF16_OUT_CASES[name]
    print("bf16 expert_out", name, scheme, W.describe(wl), flush=True)
    x, logits, _ = HN.device_inputs(wl)
    if scheme == "fp8":
        w = HN.device_weights(wl)
    elif scheme == "w8a16":
        w = HN.device_weights(wl).with_quant(M.MOE_QUANT_W8A16)
    else:
        w = HN.device_weights_mx(wl, M.QUANT_SCHEMES[scheme])
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    xq = xs = None
    kw = {}
    if scheme == "w8a16":
        kw["x"] = x
    else:
        xq, xs = (M.moe_quant_act if scheme == "fp8" else M.moe_quant_act_mx)(x)
    e32 = M.moe_grouped_ffn(xq, xs, r, w, wl.k, out_dtype=torch.float32, **kw)
    e16 = M.moe_grouped_ffn(xq, xs, r, w, wl.k, out_dtype=torch.bfloat16, **kw)
    ref = e32.to(torch.bfloat16)
    diff = (e16.view(torch.int16) != ref.view(torch.int16)).sum().item()
    ties = ((e32.view(torch.int32) & 0xFFFF) == 0x8000).sum().item()
    print(f"  {e16.numel()} values, {ties} exact ties in float32, {diff} differ", flush=True)
    assert diff == 0
