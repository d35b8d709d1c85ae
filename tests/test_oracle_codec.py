"""Pins of the oracle's E4M3 / UE8M0 codecs and scale rule (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_all_codes():
    ours = codec.e4m3_decode_table()
    ref = torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert nan.sum() == 2 and ours[0x7E] == 448.0


def test_golden_hand_encodings():
    with open(os.path.join(GOLDEN, "e4m3_hand.txt")) as f:
        rows = [ln.split()[:2] for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for val, code in rows:
        assert int(codec.e4m3_encode(np.array([float(val)]))[0]) == int(code, 16), val


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(codec.e4m3_encode(codec.e4m3_decode(codes)), codes)


def _midpoint_set():
    mags = codec.e4m3_decode_table()[:127]
    mids = (mags[:-1] + mags[1:]) / 2
    v = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), mags])
    return np.concatenate([v, -v])


def test_encode_matches_bruteforce():
    rng = np.random.default_rng(0)
    v = np.concatenate([_midpoint_set(), rng.normal(0, 100, 2000), rng.normal(0, 0.01, 2000),
                        [0.0, -0.0, 448.0, 449.0, 1e9, -1e9, 1e-30, -1e-30]])
    assert np.array_equal(codec.e4m3_encode(v), codec.e4m3_encode_bruteforce(v))


def test_encode_matches_torch_cast_in_range():
    # every bfloat16 bit pattern times 2^s, plus all midpoints; torch saturates differently
    # above 448 (NaN), so compare only |v| <= 448 -- the scale rule never exceeds it.
    # torch casts float64 through float32 (rounding twice), so only float32 values are used.
    pats = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    pats = pats[np.isfinite(pats) & (np.abs(pats) < 1e30)].astype(np.float64)
    vals = [pats * 2.0 ** s for s in (-8, 0, 6)] + [_midpoint_set()]
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    v = v[v.astype(np.float32).astype(np.float64) == v]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3_encode(v), ref)


def test_ue8m0_exhaustive():
    b = np.arange(255)
    vals = codec.ue8m0_decode(b)
    assert np.array_equal(vals, np.ldexp(1.0, b - 127))
    assert np.array_equal(codec.ue8m0_encode(b - 127), b.astype(np.uint8))
    assert np.isnan(codec.ue8m0_decode(np.array([255]))[0])
    with pytest.raises(ValueError):
        codec.ue8m0_encode(np.array([128]))


def test_scale_exponent_hand_values():
    cases = {448.0: 0, np.nextafter(448.0, 1e9): 1, 224.0: -1, np.nextafter(224.0, 1e9): 0,
             1.0: -8, 1.75: -8, np.nextafter(1.75, 9): -7, 0.0: 0, 1e-300: -127, 1e300: 127,
             2.0 ** -7: -15, 2.0 ** -6: -14}
    for a, e in cases.items():
        assert int(codec.scale_exponent(np.array([a]))[0]) == e, a


def test_scale_exponent_invariant():
    rng = np.random.default_rng(1)
    amax = np.exp(rng.uniform(-60, 60, 100000))
    e = codec.scale_exponent(amax)
    r = amax / np.ldexp(1.0, e)
    assert ((r > 224.0) & (r <= 448.0)).all()


def test_quant_rows_roundtrip_on_representable_groups():
    rng = np.random.default_rng(2)
    R, C = 37, 384
    codes = rng.integers(0, 256, (R, C)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    e = rng.integers(-20, 20, (R, C // 128))
    vals = codec.e4m3_decode(codes).reshape(R, C // 128, 128)
    vals[:, :, 5] = 448.0            # force amax = 448 * 2^e
    x = (vals * np.ldexp(1.0, e)[:, :, None]).reshape(R, C)
    q, s = codec.quant_rows_128(x)
    assert np.array_equal(codec.dequant_rows_128(q, s), x)
    assert np.array_equal(s.astype(np.int64) - 127, e)


def test_quant_rows_group_max_in_expected_set():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (64, 512))
    q, s = codec.quant_rows_128(x)
    mx = np.abs(codec.e4m3_decode(q)).reshape(64, 4, 128).max(axis=2)
    # amax / 2^e lies in (224, 448]; E4M3 values there are 224 (reached from (224, 232)),
    # 240, 256, then steps of 32 up to 448
    assert set(np.unique(mx)) <= {224.0, 240.0, 256.0, 288.0, 320.0, 352.0, 384.0, 416.0, 448.0}


def test_quant_blocks_scales_per_block():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, (256, 384))
    w[128:, :128] *= 16.0
    q, s = codec.quant_blocks_128(w)
    assert s.shape == (2, 3)
    assert int(s[1, 0]) - int(s[0, 0]) in (3, 4, 5)
    # each block's largest |code value| is in the [224, 448] band
    d = np.abs(codec.e4m3_decode(q)).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert ((d >= 224) & (d <= 448)).all()
    rt = codec.dequant_blocks_128(q, s)
    assert np.abs(rt - w).max() <= np.abs(w).max() * 2.0 ** -3


def test_negative_underflow_keeps_sign():
    q = codec.e4m3_encode(np.array([-1e-6, 1e-6, -0.0, 0.0]))
    assert list(q) == [0x80, 0x00, 0x80, 0x00]


def test_decision_margin_hand_values():
    # 256 and 1.0 sit 2^-5 (relative) below the midpoints 248 and 0.96875 to their lower
    # neighbours 240 and 0.9375; the scale boundaries 224 and 448 are farther away
    row = np.ones(128)
    row[0] = 256.0
    assert codec.decision_margin_rows_128(row[None])[0] == 2.0 ** -5
    mid = row.copy()
    mid[5] = 1.0625                       # halfway between 1.0 and 1.125
    assert codec.decision_margin_rows_128(mid[None])[0] == 0.0
    for amax in (448.0, 448.0 * 8, 448.0 * 2.0 ** -20):   # amax on a scale boundary
        b = row / 256.0 * amax
        assert codec.decision_margin_rows_128(b[None])[0] == 0.0
    zero = np.zeros((1, 256))
    assert codec.decision_margin_rows_128(zero)[0] == np.inf
    two = np.concatenate([np.zeros(128), row])[None]     # the zero group takes no decision
    assert codec.decision_margin_rows_128(two)[0] == 2.0 ** -5
    assert codec.decision_margin_rows_128(np.concatenate([row, mid])[None])[0] == 0.0


def test_decision_margin_bounds_single_element_perturbations():
    # brute force: no single element moved by a relative amount just below the margin
    # changes a code or a scale; some element moved just above it does
    rng = np.random.default_rng(7)
    R, C = 6, 128
    v = rng.standard_normal((R, C)) * np.exp2(rng.integers(-6, 7, size=(R, 1)))
    m = codec.decision_margin_rows_128(v)
    q0, s0 = codec.quant_rows_128(v)
    for r in range(R):
        changed_above = False
        for f in (1 - 1e-6, 1 + 1e-6):
            t = m[r] * f
            for i in range(C):
                for sign in (-1.0, 1.0):
                    w = v[r].copy()
                    w[i] *= 1 + sign * t
                    q, s = codec.quant_rows_128(w[None])
                    same = np.array_equal(q[0], q0[r]) and np.array_equal(s[0], s0[r])
                    if f < 1:
                        assert same, (r, i, sign)
                    elif not same:
                        changed_above = True
        assert changed_above, r


def _dq(v, group):
    """dequant(quant(v)) per (row, group) through the pinned quantisers."""
    if group == 128:
        return codec.dequant_rows_128(*codec.quant_rows_128(v))
    from oracle import mx
    return mx.dequant_rows_32(*mx.quant_rows_32(v))


def test_near_tie_flips_hand_values():
    # 1.0625 sits on the midpoint of 1.0 and 1.125 (group amax 320, e = 0, no scale tie):
    # round to nearest even takes 1.0 (code 0x38), the other way is 1.125; a negative copy
    # flips to -1.125
    row = np.ones(128)
    row[0] = 320.0
    row[5] = 1.0625
    row[9] = -1.0625
    elem, scale = codec.near_tie_flips(row[None], 128, 3e-5)
    assert elem[0, 5] == 0.125 and elem[0, 9] == -0.125
    assert np.count_nonzero(elem) == 2 and scale == []
    # amax on the scale boundary 448 * 2^3: the other way is e + 1 = 4 (every code re-chosen)
    b = row * 8.0
    b[0] = 448.0 * 8.0
    b[5] = b[9] = 8.0
    elem, scale = codec.near_tie_flips(b[None], 128, 3e-5)
    assert np.count_nonzero(elem) == 0 and len(scale) == 1
    r, c0, d = scale[0]
    assert (r, c0) == (0, 0)
    cur = _dq(b[None], 128)[0]
    alt = codec.e4m3_decode(codec.e4m3_encode(b / 16.0)) * 16.0
    assert np.array_equal(d, alt - cur)


@pytest.mark.parametrize("group", [128, 32])
def test_near_tie_flips_against_perturbations(group):
    # brute force through the pinned quantiser (tolerance tol * |v|, i.e. relative): every
    # flagged element decision flips when its element alone moves by a relative amount below
    # tol (in the direction of its midpoint),
    # and the dequantised row then changes by exactly the reported delta; no unflagged element
    # changes its code under any single-element move of relative size below tol
    tol = 1e-3     # wide, so that random rows hold near ties
    rng = np.random.default_rng(11)
    R, C = 4, 256
    v = rng.standard_normal((R, C)) * np.exp2(rng.integers(-4, 5, size=(R, 1)))
    elem, scale = codec.near_tie_flips(v, group, tol * np.abs(v))
    assert np.count_nonzero(elem) > 5
    base = _dq(v, group)
    scale_groups = {(r, c0) for r, c0, _ in scale}
    for r in range(R):
        for i in range(C):
            if (r, i - i % group) in scale_groups:
                continue
            flips = []
            for f in (1 - tol * 0.999, 1 + tol * 0.999):
                w = v[r].copy()
                w[i] *= f
                d = _dq(w[None], group)[0] - base[r]
                if np.any(d != 0):
                    flips.append(d)
            if elem[r, i] != 0:
                assert flips, (r, i)
                for d in flips:   # only the element itself moved, by the reported delta
                    assert d[i] == elem[r, i] and np.count_nonzero(d) == 1
            else:
                # a move may change the group's scale only if that is a flagged scale tie
                assert not flips, (r, i)


def test_flip_bound_covers_every_subset_and_is_exact_for_one():
    # brute force over all subsets of a row's near-tie element decisions: the change of
    # dequant(quant(v)) @ w never exceeds the bound, and with a single decision it equals it
    tol = 2e-3
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 128)) * 3.0
    w = rng.standard_normal((128, 6))
    elem, scale = codec.near_tie_flips(v, 128, tol * np.abs(v))
    idx = np.nonzero(elem[0])[0]
    assert scale == [] and 2 <= len(idx) <= 10
    bound = codec.flip_bound(v, w, 128, tol * np.abs(v))[0]
    base = _dq(v, 128)[0] @ w
    import itertools
    for n in range(1, len(idx) + 1):
        for sub in itertools.combinations(idx, n):
            hq = _dq(v, 128)[0].copy()
            hq[list(sub)] += elem[0, list(sub)]
            assert np.all(np.abs(hq @ w - base) <= bound * (1 + 1e-12))
    one = v.copy()
    keep = idx[0]
    one[0, idx[1:]] = np.round(one[0, idx[1:]])          # move the other ties away
    e1, s1 = codec.near_tie_flips(one, 128, tol * np.abs(one))
    assert np.count_nonzero(e1) == 1 and not s1
    assert np.allclose(codec.flip_bound(one, w, 128, tol * np.abs(one))[0], np.abs(e1[0, keep] * w[keep]))
