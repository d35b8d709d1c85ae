"""Top-k routing, the gate prelude and the stable expert permutation (CPU, float64).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Definitions (restated from the pages, readings marked):

* Softmax routing -- MindIE-SD ``fused_moe``, parameter table (``routing_method``,
  ``renormalize``, ``routed_scaling_factor``), section "路由选择" (routing selection)
  and the custom routing function example, which spells the plain definition out:
  softmax over all experts, take the k largest, divide by their sum when renormalising.
  ``routed_scaling_factor`` multiplies the routing weights at expert-selection time.
* Sigmoid routing -- same table and section: scores are sigmoids and the selected
  weights always come out normalised over the k selected ("NPU gating top-k semantics").
  Reading: ``renormalize`` only affects softmax; the scaling factor is applied last.
* Group-limited selection -- same table (``group_count``, ``k_group``,
  ``group_select_mode``) and the routing section's constraint list: experts form
  ``group_count`` contiguous id ranges; a group's score is its largest score (mode 0) or
  the sum of its two largest scores (mode 1); the ``k_group`` best groups are kept and
  the top-k is taken inside them.
* Gate prelude (decode shape) -- mlx-native ``moe_gate.rs``, module doc and the
  ``moe_gate`` doc: RMSNorm of the bf16 token, router matmul with float32 weights
  [E, H], top-K, softmax over the selected, times a per-expert scale.
  Reading: the RMSNorm feeds only the router; the expert FFN consumes the
  un-normalised hidden state.
* Static dispatch -- ``fused_moe`` "Dispatcher 策略": the static dispatcher sorts
  tokens by expert and counts tokens per expert.  Reading: a stable counting sort on
  the expert id over the flat assignment index f = t*k + j.

Ordering readings: the k selected experts are listed by descending score, ties going
to the lower expert id; group ties go to the lower group id.  Selection is done on the
float32 logits as given: softmax and sigmoid are strictly increasing, so ranking by
logit is ranking by score, and it is exact.

Pins (tests/test_oracle_routing.py): brute force over all k-subsets on small E; the
torch softmax/topk definition of the custom routing example; the closed form
"renormalised softmax weights = softmax over the selected logits"; G = 1 and
k_group = G reduce to ungrouped routing; brute-force group enumeration; hand cases;
stable argsort for the permutation; the RMSNorm against torch's rms_norm.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class RouteParams:
    num_experts: int
    top_k: int
    scoring: str = "softmax"          # "softmax" | "sigmoid"
    renormalize: bool = False
    group_count: int = 1
    k_group: int = 1
    group_select_mode: int = 0
    routed_scaling_factor: float = 1.0


def softmax_rows(l: np.ndarray) -> np.ndarray:
    l = np.asarray(l, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def sigmoid(l: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(l, dtype=np.float64)))


def _order_desc(keys: np.ndarray) -> np.ndarray:
    """Per row: indices sorted by descending key, ties to the lower index."""
    # a stable sort of the negated keys keeps equal keys in increasing index order
    return np.argsort(-keys, axis=1, kind="stable")


def group_mask(scores: np.ndarray, p: RouteParams):
    """Boolean [T, E] mask of the experts inside each token's k_group best groups, and
    the float64 margin between the k_group-th and the next group score (inf if none)."""
    T, E = scores.shape
    G = p.group_count
    if G == 1:
        return np.ones((T, E), dtype=bool), np.full(T, np.inf)
    per = E // G
    g = scores.reshape(T, G, per)
    if p.group_select_mode == 0:
        gscore = g.max(axis=2)
    else:
        top2 = np.sort(g, axis=2)[:, :, -2:]
        gscore = top2[:, :, 0] + top2[:, :, 1]
    order = _order_desc(gscore)
    keep = order[:, :p.k_group]
    mask_g = np.zeros((T, G), dtype=bool)
    np.put_along_axis(mask_g, keep, True, axis=1)
    srt = np.take_along_axis(gscore, order, axis=1)
    margin = srt[:, p.k_group - 1] - srt[:, p.k_group] if p.k_group < G else np.full(T, np.inf)
    return np.repeat(mask_g, per, axis=1), margin


def route(logits: np.ndarray, p: RouteParams):
    """Route [T, E] logits.

    Returns (ids int32 [T, k], weights float64 [T, k], group_margin float64 [T]).
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    if E != p.num_experts:
        raise ValueError("router logits last dim must equal num_experts")
    if p.scoring == "softmax":
        scores = softmax_rows(l)
    elif p.scoring == "sigmoid":
        scores = sigmoid(l)
    else:
        raise ValueError(p.scoring)
    allowed, gmargin = group_mask(scores, p)
    keys = np.where(allowed, l, -np.inf)
    ids = _order_desc(keys)[:, :p.top_k]
    sel = np.take_along_axis(scores, ids, axis=1)
    if p.scoring == "sigmoid" or p.renormalize:
        w = sel / sel.sum(axis=1, keepdims=True)
    else:
        w = sel
    w = w * p.routed_scaling_factor
    return ids.astype(np.int32), w, gmargin


def gate_prelude_logits(x: np.ndarray, norm_w: np.ndarray, router_w: np.ndarray, eps: float):
    """RMSNorm then router matmul: l = (x * r * w_norm) @ W_r^T with
    r = 1 / sqrt(mean(x^2) + eps); everything float64."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
    xn = x * r * np.asarray(norm_w, dtype=np.float64)[None, :]
    return xn @ np.asarray(router_w, dtype=np.float64).T


def route_prelude(x, norm_w, router_w, pe_scale, eps: float, top_k: int):
    """Gate prelude routing: top-k by logit, softmax over the k selected logits, times
    the selected experts' per-expert scale.

    Returns (ids int32 [T, k], weights float64 [T, k], logits float64 [T, E],
    selection margin float64 [T] = k-th minus (k+1)-th largest logit)."""
    l = gate_prelude_logits(x, norm_w, router_w, eps)
    T, E = l.shape
    order = _order_desc(l)
    ids = order[:, :top_k]
    sel = np.take_along_axis(l, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    w = w * np.asarray(pe_scale, dtype=np.float64)[ids]
    srt = np.take_along_axis(l, order, axis=1)
    margin = srt[:, top_k - 1] - srt[:, top_k] if top_k < E else np.full(T, np.inf)
    return ids.astype(np.int32), w, l, margin


def permute(ids: np.ndarray, num_experts: int):
    """Stable counting sort of the flat assignments f = t*k + j by expert id.

    Returns (counts int32 [E], offsets int32 [E+1], sorted_assign int32 [A] = the flat
    index at each sorted slot, assign_pos int32 [A] = the slot of each flat index)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_assign = np.empty(A, dtype=np.int64)
    cursor = offsets[:-1].copy()
    for f in range(A):                       # in flat order, so equal ids stay in order
        e = flat[f]
        sorted_assign[cursor[e]] = f
        cursor[e] += 1
    assign_pos = np.empty(A, dtype=np.int64)
    assign_pos[sorted_assign] = np.arange(A)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_assign.astype(np.int32), assign_pos.astype(np.int32))
