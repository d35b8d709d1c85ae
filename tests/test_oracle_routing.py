"""Pins of the oracle's routing, gate prelude and permutation (CPU only)."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import routing
from oracle.routing import RouteParams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_logit(tok):
    assert tok.startswith("ln")
    a = tok[2:]
    if "/" in a:
        n, d = a.split("/")
        return math.log(float(n) / float(d))
    return math.log(float(a))


def test_golden_hand_routing_cases():
    with open(os.path.join(GOLDEN, "routing_hand.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 9
    for ln in rows:
        name, scoring, ren, G, kg, mode, rsf, k, logits, ids, w = [c.strip() for c in ln.split("|")]
        lg = np.array([[_parse_logit(t) for t in logits.split()]], dtype=np.float32)
        p = RouteParams(num_experts=lg.shape[1], top_k=int(k), scoring=scoring,
                        renormalize=bool(int(ren)), group_count=int(G), k_group=int(kg),
                        group_select_mode=int(mode), routed_scaling_factor=float(rsf))
        got_ids, got_w, _ = routing.route(lg, p)
        assert list(got_ids[0]) == [int(i) for i in ids.split()], name
        np.testing.assert_allclose(got_w[0], [float(x) for x in w.split()], rtol=1e-6, err_msg=name)


def brute_topk(l, k, allowed=None):
    """Enumerate every k-subset; the top-k is the one whose members all beat every
    non-member under the order (value desc, id asc)."""
    E = len(l)
    allowed = np.ones(E, bool) if allowed is None else allowed
    cand = [i for i in range(E) if allowed[i]]
    better = lambda a, b: (l[a] > l[b]) or (l[a] == l[b] and a < b)
    for S in itertools.combinations(cand, k):
        rest = [i for i in cand if i not in S]
        if all(better(a, b) for a in S for b in rest):
            return sorted(S, key=lambda i: (-l[i], i))
    raise AssertionError("no subset")


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 3), (10, 4), (10, 10)])
def test_topk_bruteforce(E, k):
    rng = np.random.default_rng(E * 31 + k)
    # coarse values make ties frequent
    l = rng.integers(-3, 4, (50, E)).astype(np.float32)
    ids, _, _ = routing.route(l, RouteParams(E, k))
    for t in range(50):
        assert list(ids[t]) == brute_topk(l[t], k)


def test_softmax_matches_page_definition_with_torch():
    # the custom routing function example: softmax -> topk -> divide by the sum
    rng = np.random.default_rng(5)
    l = rng.normal(0, 1, (200, 16)).astype(np.float32)
    for renorm in (False, True):
        ids, w, _ = routing.route(l, RouteParams(16, 4, "softmax", renorm))
        t = torch.from_numpy(l).double()
        r = t.softmax(dim=-1).topk(4, dim=-1)
        tw = r.values
        if renorm:
            tw = tw / tw.sum(dim=-1, keepdim=True)
        assert np.array_equal(ids, r.indices.numpy())
        np.testing.assert_allclose(w, tw.numpy(), rtol=1e-12)


def test_renormalized_softmax_is_softmax_over_selected():
    rng = np.random.default_rng(6)
    l = rng.normal(0, 2, (100, 32)).astype(np.float32)
    ids, w, _ = routing.route(l, RouteParams(32, 5, "softmax", True, routed_scaling_factor=2.5))
    sel = np.take_along_axis(l.astype(np.float64), ids, axis=1)
    ref = np.exp(sel) / np.exp(sel).sum(axis=1, keepdims=True) * 2.5
    np.testing.assert_allclose(w, ref, rtol=1e-12)


def test_sigmoid_k1_weight_is_rsf():
    rng = np.random.default_rng(7)
    l = rng.normal(0, 1, (20, 8)).astype(np.float32)
    _, w, _ = routing.route(l, RouteParams(8, 1, "sigmoid", False, routed_scaling_factor=0.5))
    assert np.all(w == 0.5)


def test_sigmoid_weights_normalised_even_without_renormalize():
    rng = np.random.default_rng(8)
    l = rng.normal(0, 1, (20, 8)).astype(np.float32)
    ids, w, _ = routing.route(l, RouteParams(8, 3, "sigmoid", False))
    s = 1 / (1 + np.exp(-np.take_along_axis(l.astype(np.float64), ids, 1)))
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True), rtol=1e-12)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("mode", [0, 1])
def test_group_degenerate_cases_reduce_to_ungrouped(scoring, mode):
    rng = np.random.default_rng(9)
    l = rng.normal(0, 1, (100, 16)).astype(np.float32)
    base = routing.route(l, RouteParams(16, 4, scoring, True))
    g1 = routing.route(l, RouteParams(16, 4, scoring, True, group_count=1, k_group=1, group_select_mode=mode))
    gall = routing.route(l, RouteParams(16, 4, scoring, True, group_count=4, k_group=4, group_select_mode=mode))
    for other in (g1, gall):
        assert np.array_equal(base[0], other[0])
        np.testing.assert_allclose(base[1], other[1], rtol=1e-15)


def brute_group_route(l, E, G, kg, mode, k, scoring):
    s = [1 / (1 + math.exp(-v)) for v in l] if scoring == "sigmoid" else None
    if scoring == "softmax":
        m = max(l)
        z = [math.exp(v - m) for v in l]
        s = [v / sum(z) for v in z]
    per = E // G
    gs = []
    for g in range(G):
        vals = sorted(s[g * per:(g + 1) * per], reverse=True)
        gs.append(vals[0] if mode == 0 else vals[0] + vals[1])
    best = None
    for keep in itertools.combinations(range(G), kg):
        rest = [g for g in range(G) if g not in keep]
        if all((gs[a] > gs[b]) or (gs[a] == gs[b] and a < b) for a in keep for b in rest):
            best = keep
    allowed = np.zeros(E, bool)
    for g in best:
        allowed[g * per:(g + 1) * per] = True
    return brute_topk(np.asarray(l), k, allowed)


@pytest.mark.parametrize("scoring,mode,kg", [("sigmoid", 1, 1), ("sigmoid", 0, 2), ("softmax", 1, 2), ("softmax", 0, 1)])
def test_group_selection_bruteforce(scoring, mode, kg):
    # the fused_moe grouped example's parameters: E=16, G=4, k_group=1, mode 1, sigmoid, rsf 0.5
    rng = np.random.default_rng(10 + mode + 2 * kg)
    l = rng.normal(0, 1, (60, 16)).astype(np.float32)
    p = RouteParams(16, 2, scoring, False, group_count=4, k_group=kg, group_select_mode=mode,
                    routed_scaling_factor=0.5)
    ids, w, _ = routing.route(l, p)
    for t in range(60):
        assert list(ids[t]) == brute_group_route([float(v) for v in l[t]], 16, 4, kg, mode, 2, scoring)
    if scoring == "sigmoid":
        np.testing.assert_allclose(w.sum(axis=1), 0.5, rtol=1e-12)


def test_prelude_matches_torch_rmsnorm_and_matmul():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (8, 256))
    nw = 1 + rng.normal(0, 0.1, 256)
    W = rng.normal(0, 0.02, (32, 256))
    l = routing.gate_prelude_logits(x, nw, W, 1e-6)
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.rms_norm(xt, (256,), torch.from_numpy(nw), eps=1e-6) @ torch.from_numpy(W).T
    np.testing.assert_allclose(l, ref.numpy(), rtol=1e-12, atol=1e-14)
    pe = rng.uniform(0.5, 1.5, 32)
    ids, w, l2, margin = routing.route_prelude(x, nw, W, pe, 1e-6, 4)
    assert np.array_equal(l, l2)
    for t in range(len(x)):
        assert list(ids[t]) == brute_topk(l[t], 4), t
    # the weights through torch: the page's softmax over all experts, top-k, divide by the
    # selected sum (equal to the softmax over the selected logits), times the scale
    p_all = torch.softmax(torch.from_numpy(l), dim=1)
    v, i = torch.topk(p_all, 4, dim=1)
    assert np.array_equal(i.numpy(), ids)
    np.testing.assert_allclose(w, (v / v.sum(1, keepdim=True)).numpy() * pe[ids], rtol=1e-12)
    assert (margin > 0).all()


def test_permute_invariants_and_stable_sort():
    rng = np.random.default_rng(12)
    for T, k, E in [(50, 2, 8), (300, 8, 64), (1, 1, 1), (17, 4, 4)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, sa, ap = routing.permute(ids, E)
        flat = ids.reshape(-1)
        assert counts.sum() == T * k and offsets[-1] == T * k
        assert np.array_equal(np.sort(sa), np.arange(T * k))
        assert np.array_equal(ap[sa], np.arange(T * k))
        assert np.array_equal(sa, np.argsort(flat, kind="stable"))
        assert np.array_equal(sa, np.array(sorted(range(T * k), key=lambda f: (flat[f], f))))
        for e in range(E):
            seg = sa[offsets[e]:offsets[e + 1]]
            assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def _golden_prelude():
    def val(tok):
        return float(np.log(float(tok[2:]))) if tok.startswith("ln") else float(tok)
    cases = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "prelude_hand.txt")) as f:
        for ln in f:
            if not ln.strip() or ln.startswith("#"):
                continue
            name, x, nw, eps, rows, pe, k, ids, w = [c.strip() for c in ln.split("|")]
            cases.append((name, np.array([val(t) for t in x.split()]), np.array([val(t) for t in nw.split()]),
                          float(eps), np.array([[val(t) for t in r.split()] for r in rows.split(";")]),
                          np.array([val(t) for t in pe.split()]), int(k), [int(t) for t in ids.split()],
                          [float(t) for t in w.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_prelude(), ids=lambda c: c[0])
def test_prelude_golden_hand_cases(case):
    # tests/golden/prelude_hand.txt: RMSNorm, router rows, top-k with the lower-id tie rule,
    # softmax over the selected logits and the per-expert scale, all worked by hand
    name, x, nw, eps, W_r, pe, k, ids_exp, w_exp = case
    ids, w, l, margin = routing.route_prelude(x[None], nw, W_r, pe, eps, k)
    assert ids[0].tolist() == ids_exp, name
    assert np.allclose(w[0], w_exp, rtol=1e-12, atol=0), (name, w[0])
