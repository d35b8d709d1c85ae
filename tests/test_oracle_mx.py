"""Pins of the oracle's micro-scaled (32-element) formats: E2M1 codec, the 32-group scale
rule, the MX quantisers and the MXFP8 / W4A8 expert FFN (CPU only)."""
import os

import numpy as np
import torch

from oracle import codec, moe, mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                rows.append(ln.split())
    return rows


def test_e2m1_hand_table():
    for kind, a, b in _golden("e2m1_hand.txt"):
        if kind == "decode":
            v = mx.e2m1_decode(np.array([int(a, 16)]))[0]
            assert v == float(b) and np.signbit(v) == b.startswith("-")
        elif kind == "encode":
            assert mx.e2m1_encode(np.array([float(a)]))[0] == int(b, 16), a
        else:
            assert mx.scale_exponent(np.array([float(a)]), mx.FMT_E2M1)[0] == int(b), a


def test_e2m1_table_from_bit_fields():
    t = mx.e2m1_decode_table()
    assert list(t[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.array_equal(t[8:], -t[:8])
    # every code round-trips (negative zero included)
    assert np.array_equal(mx.e2m1_encode(t), np.arange(16, dtype=np.uint8))


def test_e2m1_encode_matches_bruteforce_on_midpoints_and_neighbours():
    mags = mx.e2m1_decode_table()[:8]
    mids = (mags[1:] + mags[:-1]) / 2
    pts = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 10), [6.5, 7, 1e9]])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(mx.e2m1_encode(pts), mx.e2m1_encode_bruteforce(pts))
    r = np.random.default_rng(3).uniform(-8, 8, 5000)
    assert np.array_equal(mx.e2m1_encode(r), mx.e2m1_encode_bruteforce(r))


def test_scale_rule_invariant_both_formats():
    r = np.random.default_rng(4)
    amax = np.ldexp(r.uniform(0.5, 1.0, 20000), r.integers(-60, 60, 20000))
    for fmt in (mx.FMT_E4M3, mx.FMT_E2M1):
        M = mx.fmt_max(fmt)
        e = mx.scale_exponent(amax, fmt)
        s = amax / np.ldexp(1.0, e)
        assert np.all((s > M / 2) & (s <= M))
    # E4M3 with 32-groups uses the same rule as the 128 path
    assert np.array_equal(mx.scale_exponent(amax, mx.FMT_E4M3), codec.scale_exponent(amax))


def test_round_trip_on_representable_groups():
    r = np.random.default_rng(5)
    for fmt, ncode in ((mx.FMT_E4M3, 127), (mx.FMT_E2M1, 8)):
        M = mx.fmt_max(fmt)
        mags = (codec.e4m3_decode_table()[:127] if fmt == mx.FMT_E4M3 else mx.e2m1_decode_table()[:8])
        for _ in range(20):
            e = int(r.integers(-20, 20))
            v = r.choice(mags, size=(3, 64)) * np.where(r.random((3, 64)) < 0.5, -1, 1)
            v[:, 0] = M
            v[:, 32] = -M
            x = np.ldexp(v, e)
            q, s = mx.quant_rows_32(x, fmt)
            assert np.array_equal(mx.dequant_rows_32(q, s, fmt), x)
            assert np.all(s == e + 127)


def test_32_groups_agree_with_128_groups_when_every_subgroup_has_the_group_max():
    r = np.random.default_rng(6)
    x = r.normal(size=(5, 256))
    g = np.abs(x).reshape(5, 2, 128).max(axis=2)
    for j in range(4):            # each 32-subgroup carries its 128-group's amax
        x[:, j * 32] = np.repeat(g[:, :1], 1, axis=1)[:, 0]
        x[:, 128 + j * 32] = -g[:, 1]
    q32, s32 = mx.quant_rows_32(x)
    q128, s128 = codec.quant_rows_128(x)
    assert np.array_equal(q32, q128)
    assert np.array_equal(s32, np.repeat(s128, 4, axis=1))
    # weights: every (32 x 1) group holds its 128 x 128 block's amax
    w = r.normal(0, 0.02, (256, 128))
    for kb in range(2):
        c = np.abs(w[kb * 128:(kb + 1) * 128]).max() * 1.01
        w[kb * 128 + np.arange(4) * 32, :] = c
    qw, sw = mx.quant_weight_k32(w, mx.FMT_E4M3)
    qb, sb = codec.quant_blocks_128(w)
    assert np.array_equal(qw, qb)
    assert np.array_equal(sw, np.repeat(np.repeat(sb, 4, axis=0), 128, axis=1))


def test_mx_single_token_single_expert_is_dense_swiglu_mlp():
    H, I = 192, 160
    g = torch.Generator().manual_seed(7)
    x = torch.randn(1, H, generator=g).to(torch.bfloat16).double().numpy()
    w13 = (torch.randn(H, 2 * I, generator=g) * 0.05).double().numpy()
    w2 = (torch.randn(I, H, generator=g) * 0.05).double().numpy()
    for fmt in (mx.FMT_E4M3, mx.FMT_E2M1):
        ex = mx.QuantizedExpertsMX(lambda e: (w13, w2), fmt)
        out = mx.forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), ex)
        q13, s13, q2, s2 = ex.get(0)
        xd = torch.from_numpy(mx.dequant_rows_32(out["xq"], out["xs"]))
        gu = xd @ torch.from_numpy(mx.dequant_weight_k32(q13, s13, fmt))
        h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        hq, hs = mx.quant_rows_32(h.numpy())
        assert np.array_equal(hq, out["hq"]) and np.array_equal(hs, out["hs"])
        y = torch.from_numpy(mx.dequant_rows_32(hq, hs)) @ torch.from_numpy(mx.dequant_weight_k32(q2, s2, fmt))
        np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-14)
        # and the dequantised weights are within the format's step of the float weights
        rel = 2.0 ** -3 if fmt == mx.FMT_E4M3 else 0.25
        wd = mx.dequant_weight_k32(q13, s13, fmt)
        s = codec.ue8m0_decode(s13).repeat(32, axis=0)
        assert np.all(np.abs(wd - w13) <= np.maximum(rel * np.abs(w13), 0.5 * 2.0 ** (-9 if fmt == mx.FMT_E4M3 else -1) * s * (8 if fmt == mx.FMT_E4M3 else 1)) + 1e-300)


def test_mx_combine_and_routing_structure():
    # k = 2: y is the weighted sum of the two experts' outputs, each one the single-expert FFN
    H, I = 64, 96
    r = np.random.default_rng(8)
    w13s = [r.normal(0, 0.05, (H, 2 * I)) for _ in range(3)]
    w2s = [r.normal(0, 0.05, (I, H)) for _ in range(3)]
    x = r.normal(size=(4, H))
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1]], np.int32)
    w = r.uniform(0.1, 1, (4, 2))
    ex = mx.QuantizedExpertsMX(lambda e: (w13s[e], w2s[e]), mx.FMT_E2M1, cache=8)
    out = mx.forward(x, ids, w, ex)
    for t in range(4):
        acc = 0
        for j in range(2):
            one = mx.forward(x[t:t + 1], ids[t:t + 1, j:j + 1], np.ones((1, 1)), ex)
            acc = acc + w[t, j] * one["y"][0]
        np.testing.assert_allclose(out["y"][t], acc, rtol=1e-13, atol=1e-15)


def test_mx_decision_margin_hand_values_and_perturbations():
    row = np.ones(64)
    row[0] = 256.0
    row[32] = 256.0
    assert mx.decision_margin_rows_32(row[None])[0] == 2.0 ** -5
    mid = row.copy()
    mid[40] = 1.0625                       # halfway between 1.0 and 1.125
    assert mx.decision_margin_rows_32(mid[None])[0] == 0.0
    b = row / 256.0 * 448.0 * 4             # amax on a scale boundary
    assert mx.decision_margin_rows_32(b[None])[0] == 0.0
    assert mx.decision_margin_rows_32(np.zeros((1, 64)))[0] == np.inf
    # brute force: no single element moved by a relative amount just below the margin changes
    # a code or a scale
    r = np.random.default_rng(9)
    v = r.standard_normal((3, 64)) * np.exp2(r.integers(-6, 7, size=(3, 1)))
    m = mx.decision_margin_rows_32(v)
    q0, s0 = mx.quant_rows_32(v)
    for i in range(3):
        for j in range(64):
            for sgn in (-1.0, 1.0):
                w = v[i].copy()
                w[j] *= 1 + sgn * m[i] * (1 - 1e-6)
                q, s_ = mx.quant_rows_32(w[None])
                assert np.array_equal(q[0], q0[i]) and np.array_equal(s_[0], s0[i])


def test_mx_biased_expert_is_torch_linear_swiglu_linear():
    # biases as in the FP8 step: w13_bias before SwiGLU, w2_bias on o before the routing weight
    H, I = 128, 96
    g = torch.Generator().manual_seed(9)
    x = torch.randn(2, H, generator=g).to(torch.bfloat16).double().numpy()
    w13 = (torch.randn(H, 2 * I, generator=g) * 0.05).double().numpy()
    w2 = (torch.randn(I, H, generator=g) * 0.05).double().numpy()
    b13 = (torch.randn(1, 2 * I, generator=g) * 0.5).double().numpy()
    b2 = (torch.randn(1, H, generator=g) * 0.5).double().numpy()
    F = torch.nn.functional
    for fmt in (mx.FMT_E4M3, mx.FMT_E2M1):
        ex = mx.QuantizedExpertsMX(lambda e: (w13, w2), fmt)
        w = np.array([[0.75], [1.5]])
        out = mx.forward(x, np.zeros((2, 1), np.int32), w, ex, biases=(b13, b2))
        q13, s13, q2, s2 = ex.get(0)
        xd = torch.from_numpy(mx.dequant_rows_32(out["xq"], out["xs"]))
        gu = F.linear(xd, torch.from_numpy(mx.dequant_weight_k32(q13, s13, fmt)).T, torch.from_numpy(b13[0]))
        h = F.silu(gu[:, :I]) * gu[:, I:]
        hq, hs = mx.quant_rows_32(h.numpy())
        assert np.array_equal(hq, out["hq"]) and np.array_equal(hs, out["hs"])
        o = F.linear(torch.from_numpy(mx.dequant_rows_32(hq, hs)),
                     torch.from_numpy(mx.dequant_weight_k32(q2, s2, fmt)).T, torch.from_numpy(b2[0]))
        np.testing.assert_allclose(out["y"], w * o.numpy(), rtol=1e-12, atol=1e-14)
