"""Pins of the W8A16 oracle (oracle.w8a16; CPU only)."""
import os

import numpy as np
import torch

from oracle import codec, moe
from oracle import w8a16 as ow

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _experts_from_dense(w13s, w2s):
    return moe.QuantizedExperts(lambda e: (w13s[e], w2s[e]), cache=64)


def test_bf16_rne_is_torch_float32_to_bfloat16():
    # torch's float32 -> bfloat16 conversion (round to nearest even) on float32 values
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 100, 20000))).astype(np.float32)
    one = np.float32(1.0)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -9, 2.0 ** -130 * 1.5,
                     2.0 ** -133 * 2.5, 2.0 ** -133 * 0.5, 255.5, 1.9990234375, 0.0, -0.0], dtype=np.float32)
    v = np.concatenate([v, ties, np.nextafter(ties, one), np.nextafter(ties, -one)])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = ow.bf16_rne(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def _golden():
    g = {}
    with open(os.path.join(GOLDEN, "ffn_w8a16_hand.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, val = ln.split()
                g[key] = float(val)
    return g


def test_golden_hand_ffn_w8a16():
    g = _golden()
    H = I = 128
    x = np.full((1, H), g["x"])
    w13 = np.concatenate([np.full((H, I), g["w13_gate"]), np.full((H, I), g["w13_up"])], axis=1)
    w2 = np.full((I, H), g["w2"])
    out = ow.forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), _experts_from_dense([w13], [w2]))
    assert (out["hb"] == g["hb"]).all()
    assert (out["y"] == g["y"]).all()
    assert abs(2.0 / (1.0 + np.exp(-1.0)) - g["h_exact"]) < 1e-15


def test_single_token_single_expert_is_dense_swiglu_mlp_with_bf16_h():
    rng = np.random.default_rng(21)
    H, I = 256, 384
    x = torch.randn(1, H, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).double()
    w13 = rng.normal(0, 0.02, (H, 2 * I))
    w2 = rng.normal(0, 0.02, (I, H))
    ex = _experts_from_dense([w13], [w2])
    out = ow.forward(x.numpy(), np.zeros((1, 1), np.int32), np.ones((1, 1)), ex)
    # textbook dense SwiGLU MLP in torch float64 on the dequantised weights, the bf16 input as
    # is, h rounded by the (separately pinned) bf16 rounding
    q13, s13, q2, s2 = ex.get(0)
    gu = x @ torch.from_numpy(codec.dequant_blocks_128(q13, s13))
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    hb = ow.bf16_rne(h.numpy())
    assert np.array_equal(hb, out["hb"])
    assert np.all(np.abs(hb - h.numpy()) <= np.abs(h.numpy()) * 2.0 ** -8)
    y = torch.from_numpy(hb) @ torch.from_numpy(codec.dequant_blocks_128(q2, s2))
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-15)


def test_equals_w8a8_step_when_activations_are_exact_in_both():
    # x = 1 and h from a small set of values that E4M3 (at the row's scale) and bf16 both hold
    # exactly; silu(g) == g in float64 for these g >= 40 (e^-g below half an ulp), so both
    # schemes see the same activations and must give the same y
    rng = np.random.default_rng(5)
    H, I, E, T, k = 128, 128, 2, 3, 2
    w13s, w2s = [], []
    for _ in range(E):
        gate = np.tile(rng.choice([40.0, 48.0, 56.0, 64.0], I) / H, (H, 1))
        up = np.tile(rng.choice([0.25, 0.5, 1.0, 2.0], I) / H, (H, 1))
        w13s.append(np.concatenate([gate, up], axis=1))
        w2s.append(rng.normal(0, 0.02, (I, H)))
    ex = _experts_from_dense(w13s, w2s)
    x = np.ones((T, H))
    ids = np.array([[0, 1], [1, 0], [0, 1]], np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    a = ow.forward(x, ids, w, ex)
    b = moe.forward(x, ids, w, ex)
    # preconditions: h is exact in bf16 and in E4M3 at its row scale
    assert np.array_equal(ow.bf16_rne(a["hb"]), a["hb"])
    assert np.array_equal(codec.dequant_rows_128(b["hq"], b["hs"]), a["hb"])
    assert np.array_equal(a["y"], b["y"])


def test_biased_expert_hand_values_and_torch_linear():
    # the hand case of tests/golden/ffn_bias_hand.txt under W8A16: h = silu(2) = 1.76159...
    # rounds to the bf16 value 225 * 2^-7 = 1.7578125 (step 2^-7 in [1, 2)), so
    # o = 128 * 1.7578125 * 2^-7 + 0.25 = 2.0078125
    H = I = 128
    w13 = np.concatenate([np.full((H, I), 2.0 ** -7), np.full((H, I), 2.0 ** -6)], axis=1)
    w2 = np.full((I, H), 2.0 ** -7)
    b13 = np.concatenate([np.ones(I), -np.ones(I)])[None]
    b2 = np.full((1, H), 0.25)
    out = ow.forward(np.ones((1, H)), np.zeros((1, 1), np.int32), np.ones((1, 1)),
                     _experts_from_dense([w13], [w2]), biases=(b13, b2))
    assert (out["hb"] == 1.7578125).all() and (out["y"] == 2.0078125).all()
    # random biased case against torch.nn.functional.linear with its bias argument
    rng = np.random.default_rng(23)
    H, I = 256, 128
    x = torch.randn(3, H, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).double()
    w13 = rng.normal(0, 0.02, (H, 2 * I))
    w2 = rng.normal(0, 0.02, (I, H))
    b13 = rng.normal(0, 0.5, (1, 2 * I))
    b2 = rng.normal(0, 0.5, (1, H))
    ex = _experts_from_dense([w13], [w2])
    out = ow.forward(x.numpy(), np.zeros((3, 1), np.int32), np.ones((3, 1)), ex, biases=(b13, b2))
    q13, s13, q2, s2 = ex.get(0)
    F = torch.nn.functional
    gu = F.linear(x, torch.from_numpy(codec.dequant_blocks_128(q13, s13)).T, torch.from_numpy(b13[0]))
    hb = ow.bf16_rne((F.silu(gu[:, :I]) * gu[:, I:]).numpy())
    assert np.array_equal(hb, out["hb"])
    o = F.linear(torch.from_numpy(hb), torch.from_numpy(codec.dequant_blocks_128(q2, s2)).T, torch.from_numpy(b2[0]))
    np.testing.assert_allclose(out["y"], o.numpy(), rtol=1e-12, atol=1e-14)
