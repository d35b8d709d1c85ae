"""Pins of the oracle's expert FFN and combine (CPU only)."""
import os

import numpy as np
import torch

from oracle import codec, moe, routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _experts_from_dense(w13s, w2s):
    return moe.QuantizedExperts(lambda e: (w13s[e], w2s[e]), cache=64)


def test_golden_hand_ffn():
    g = {}
    with open(os.path.join(GOLDEN, "ffn_hand.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, val = ln.split()
                g[key] = val
    H = I = 128
    x = np.full((1, H), float(g["x"]))
    w13 = np.concatenate([np.full((H, I), float(g["w13_gate"])), np.full((H, I), float(g["w13_up"]))], axis=1)
    w2 = np.full((I, H), float(g["w2"]))
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1))
    out = moe.forward(x, ids, w, _experts_from_dense([w13], [w2]))
    assert (out["xq"] == int(g["xq"], 16)).all() and (out["xs"] == int(g["xs"])).all()
    assert (out["hq"] == int(g["hq"], 16)).all() and (out["hs"] == int(g["hs"])).all()
    assert (out["y"] == float(g["y"])).all()
    q13, s13 = codec.quant_blocks_128(w13)
    assert list(s13[0]) == [112, 113]


def test_single_token_single_expert_is_dense_swiglu_mlp():
    rng = np.random.default_rng(20)
    H, I = 256, 384
    x = torch.randn(1, H, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).double().numpy()
    w13 = rng.normal(0, 0.02, (H, 2 * I))
    w2 = rng.normal(0, 0.02, (I, H))
    ex = _experts_from_dense([w13], [w2])
    out = moe.forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), ex)
    # textbook dense SwiGLU MLP in torch float64 on the dequantised operands
    q13, s13, q2, s2 = ex.get(0)
    xd = torch.from_numpy(codec.dequant_rows_128(out["xq"], out["xs"]))
    w13d = torch.from_numpy(codec.dequant_blocks_128(q13, s13))
    w2d = torch.from_numpy(codec.dequant_blocks_128(q2, s2))
    gu = xd @ w13d
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    hq, hs = codec.quant_rows_128(h.numpy())
    assert np.array_equal(hq, out["hq"]) and np.array_equal(hs, out["hs"])
    y = torch.from_numpy(codec.dequant_rows_128(hq, hs)) @ w2d
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-15)
    # and the quantised input really is the per-128 quantisation of x
    q, s = codec.quant_rows_128(x)
    assert np.array_equal(q, out["xq"]) and np.array_equal(s, out["xs"])


def _random_case(T=12, H=256, I=256, E=4, k=2, seed=0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.normal(0, 1, (T, H))).to(torch.bfloat16).double().numpy()
    w13 = [rng.normal(0, 0.02, (H, 2 * I)) for _ in range(E)]
    w2 = [rng.normal(0, 0.02, (I, H)) for _ in range(E)]
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    return x, logits, _experts_from_dense(w13, w2)


def test_combine_k1_w1_is_gather():
    x, logits, ex = _random_case(k=1)
    ids = np.argmax(logits, axis=1).astype(np.int32)[:, None]
    out = moe.forward(x, ids, np.ones_like(ids, dtype=np.float64), ex)
    assert np.array_equal(out["y"], out["o"])


def test_routed_scaling_factor_is_linear():
    x, logits, ex = _random_case()
    p1 = routing.RouteParams(4, 2, "softmax", True, routed_scaling_factor=1.0)
    p2 = routing.RouteParams(4, 2, "softmax", True, routed_scaling_factor=2.5)
    ids1, w1, _ = routing.route(logits, p1)
    ids2, w2, _ = routing.route(logits, p2)
    assert np.array_equal(ids1, ids2)
    y1 = moe.forward(x, ids1, w1, ex)["y"]
    y2 = moe.forward(x, ids2, w2, ex)["y"]
    np.testing.assert_allclose(y2, 2.5 * y1, rtol=1e-12, atol=1e-14)


def test_token_permutation_equivariance_and_row_independence():
    x, logits, ex = _random_case(T=10, seed=3)
    p = routing.RouteParams(4, 2, "softmax", True)
    ids, w, _ = routing.route(logits, p)
    y = moe.forward(x, ids, w, ex)["y"]
    perm = np.random.default_rng(4).permutation(10)
    idsP, wP, _ = routing.route(logits[perm], p)
    yP = moe.forward(x[perm], idsP, wP, ex)["y"]
    assert np.array_equal(yP, y[perm])
    # a sample of rows equals the same rows of the full batch, bit for bit
    ys = moe.forward(x, ids, w, ex, tokens=np.array([7, 2]))["y"]
    assert np.array_equal(ys, y[[7, 2]])


def test_combine_matches_explicit_sum():
    rng = np.random.default_rng(5)
    o = rng.normal(0, 1, (6 * 3, 16))
    w = rng.uniform(0, 1, (6, 3))
    y = moe.combine(o, w)
    for t in range(6):
        ref = sum(w[t, j] * o[t * 3 + j] for j in range(3))
        np.testing.assert_allclose(y[t], ref, rtol=1e-15, atol=1e-15)


def _dense_swiglu_mlp(ex, e, xq, xs):
    """Textbook dense SwiGLU MLP in torch float64 on the dequantised operands of expert e,
    with the re-quantisation of h between the projections."""
    q13, s13, q2, s2 = ex.get(e)
    xd = torch.from_numpy(codec.dequant_rows_128(xq, xs))
    gu = xd @ torch.from_numpy(codec.dequant_blocks_128(q13, s13))
    I = gu.shape[1] // 2
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    hq, hs = codec.quant_rows_128(h.numpy())
    return (torch.from_numpy(codec.dequant_rows_128(hq, hs)) @ torch.from_numpy(codec.dequant_blocks_128(q2, s2))).numpy()


def test_shared_expert_alone_is_dense_swiglu_mlp():
    # all routed weights zero: y is the shared expert's dense MLP of every token
    T, E, k = 7, 4, 2
    x, logits, ex = _random_case(T=T, E=E + 1, k=k, seed=5)
    ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    out = moe.forward_shared(x, ids, np.zeros((T, k)), ex, shared=E)
    ref = _dense_swiglu_mlp(ex, E, out["xq"], out["xs"])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-15)
    assert out["o"].shape == (T * (k + 1), x.shape[1])


def test_shared_expert_adds_its_mlp_to_the_routed_output():
    T, E, k = 9, 6, 3
    x, logits, ex = _random_case(T=T, E=E + 1, k=k, seed=6)
    p = routing.RouteParams(num_experts=E, top_k=k, scoring="softmax", renormalize=True)
    ids, w, _ = routing.route(logits[:, :E], p)
    routed = moe.forward(x, ids, w, ex)
    both = moe.forward_shared(x, ids, w, ex, shared=E)
    ref = _dense_swiglu_mlp(ex, E, routed["xq"], routed["xs"])
    np.testing.assert_allclose(both["y"] - routed["y"], ref, rtol=1e-9, atol=1e-12)
    # the routed slots are untouched: same per-assignment outputs in slots 0..k-1
    np.testing.assert_array_equal(both["o"].reshape(T, k + 1, -1)[:, :k], routed["o"].reshape(T, k, -1))


def _golden(name):
    g = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, val = ln.split()
                g[key] = val
    return g


def test_golden_hand_ffn_with_biases():
    # tests/golden/ffn_bias_hand.txt: gate bias +1, up bias -1, down bias 0.25, worked by hand
    g = _golden("ffn_bias_hand.txt")
    H = I = 128
    x = np.full((1, H), float(g["x"]))
    w13 = np.concatenate([np.full((H, I), float(g["w13_gate"])), np.full((H, I), float(g["w13_up"]))], axis=1)
    w2 = np.full((I, H), float(g["w2"]))
    b13 = np.concatenate([np.full(I, float(g["b13_gate"])), np.full(I, float(g["b13_up"]))])[None]
    b2 = np.full((1, H), float(g["b2"]))
    out = moe.forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), _experts_from_dense([w13], [w2]),
                      biases=(b13, b2))
    np.testing.assert_allclose(out["h"], float(g["h_exact"]), rtol=1e-15)
    assert (out["hq"] == int(g["hq"], 16)).all() and (out["hs"] == int(g["hs"])).all()
    assert (out["y"] == float(g["y"])).all()


def test_biased_expert_is_torch_linear_swiglu_linear():
    # the dense biased SwiGLU MLP written with torch.nn.functional.linear (bias argument) on
    # the dequantised operands, with h re-quantised between the projections
    rng = np.random.default_rng(21)
    T, H, I, E, k = 6, 256, 128, 3, 2
    x, logits, ex = _random_case(T=T, H=H, I=I, E=E, k=k, seed=21)
    b13 = rng.normal(0, 0.3, (E, 2 * I))
    b2 = rng.normal(0, 0.3, (E, H))
    ids, w, _ = routing.route(logits, routing.RouteParams(E, k, "softmax", True))
    out = moe.forward(x, ids, w, ex, biases=(b13, b2))
    F = torch.nn.functional
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            q13, s13, q2, s2 = ex.get(e)
            xd = torch.from_numpy(codec.dequant_rows_128(out["xq"][t:t + 1], out["xs"][t:t + 1]))
            w13d = torch.from_numpy(codec.dequant_blocks_128(q13, s13))
            gu = F.linear(xd, w13d.T, torch.from_numpy(b13[e]))
            h = F.silu(gu[:, :I]) * gu[:, I:]
            hq, hs = codec.quant_rows_128(h.numpy())
            o = F.linear(torch.from_numpy(codec.dequant_rows_128(hq, hs)),
                         torch.from_numpy(codec.dequant_blocks_128(q2, s2)).T, torch.from_numpy(b2[e]))
            y[t] += w[t, j] * o.numpy()[0]
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-14)


def test_down_bias_adds_weighted_sum_and_zero_biases_change_nothing():
    # y with a down bias alone = y without biases + sum_j w_j * b2[e_j] (the bias is taken
    # before the routing weight); zero biases reproduce the unbiased result bit for bit
    rng = np.random.default_rng(22)
    T, H, I, E, k = 8, 256, 256, 4, 2
    x, logits, ex = _random_case(T=T, H=H, I=I, E=E, k=k, seed=22)
    ids, w, _ = routing.route(logits, routing.RouteParams(E, k, "softmax", True, routed_scaling_factor=1.7))
    y0 = moe.forward(x, ids, w, ex)
    z = moe.forward(x, ids, w, ex, biases=(np.zeros((E, 2 * I)), np.zeros((E, H))))
    assert np.array_equal(z["y"], y0["y"]) and np.array_equal(z["hq"], y0["hq"])
    b2 = rng.normal(0, 1, (E, H))
    yb = moe.forward(x, ids, w, ex, biases=(np.zeros((E, 2 * I)), b2))["y"]
    np.testing.assert_allclose(yb - y0["y"], (w[:, :, None] * b2[ids]).sum(1), rtol=1e-10, atol=1e-12)
    # a gate/up bias moves h exactly as adding it to the sums does: with x = 0 the sums are the
    # biases alone, h = silu(b_gate) * b_up
    zq = np.zeros((1, H))
    b13 = rng.normal(0, 1, (E, 2 * I))
    r = moe.forward(zq, np.zeros((1, 1), np.int32), np.ones((1, 1)), ex, biases=(b13, np.zeros((E, H))))
    hb = b13[0, :I] / (1 + np.exp(-b13[0, :I])) * b13[0, I:]
    np.testing.assert_allclose(r["h"][0], hb, rtol=1e-14)
