"""The routed FP8 expert step end to end (CPU, float64).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Steps, in the order of the MindIE-SD ``fused_moe`` execution flow ("执行流程":
select_experts, dispatch, mlp, combine) with the W8A8 expert step of the metrale
``fp8_grouped_tc_w8a8.rs`` page (``run_fp8_grouped_w8a8``: quantise the layer input,
gate+up producing quantised SiLU products, then down):

1. route (``oracle.routing``);
2. quantise each token row of the hidden state to E4M3 per 128 columns (``oracle.codec``);
3. gate+up: gu = dequant(xq row) @ dequant(w13[e]), float64.  w13[e] is [H, 2I] with
   the gate projection in columns [0, I) and the up projection in [I, 2I) (reading of
   the "gate/up" fused weight in the ``fused_moe`` parameter table);
4. SwiGLU: h = silu(g) * u = g / (1 + exp(-g)) * u (the "swiglu" activation of the MATE
   Mega MoE page; no clamp);
5. re-quantise h per (assignment row, 128 columns of I) to E4M3;
6. down: o = dequant(hq) @ dequant(w2[e]), w2[e] is [I, H], float64;
   optional biases (the ``w13_bias`` [experts, 2I] and ``w2_bias`` [experts, H] of the
   ``fused_moe`` parameter table): w13_bias[e] is added to gate+up before SwiGLU (step 3),
   w2_bias[e] to o (step 6), before the routing weight;
7. combine: y[t] = sum_j w[t, j] * o[(t, j)], float64 (the ``combine`` stage; the MATE
   page's contiguous bfloat16 output is the caller-side rounding of this value).

Every product of two E4M3 values and two powers of two is exact in float64, so only
the summation order rounds (relative ~1e-16).

Pins (tests/test_oracle_moe.py): one token, one expert, top-1 equals a dense SwiGLU MLP
computed by torch in float64 on the dequantised tensors, with the re-quantisation step
checked separately; combine reduces to a gather for k = 1, w = 1; scaling the routed
scaling factor scales y; permuting tokens permutes y; a row of y does not depend on the
other rows.  The shared expert (``forward_shared``): with all routed weights zero y is the
dense SwiGLU MLP of the shared weights, and y minus the routed-only y is that MLP's output.
"""
from __future__ import annotations

import numpy as np

from . import codec, routing


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


class QuantizedExperts:
    """Per-expert E4M3 weights with UE8M0 128x128 block scales, produced on demand.

    ``source(e)`` returns (w13_f32 [H, 2I], w2_f32 [I, H]) as arrays; the oracle
    quantises them itself and keeps the last few experts."""

    def __init__(self, source, cache: int = 4):
        self.source = source
        self.cache = cache
        self._mem: dict = {}

    def preload(self, quantized: dict) -> None:
        """Keep already-quantised experts {e: (q13, s13, q2, s2)} (made by this module's
        codec, e.g. in parallel by a caller) for the next forward."""
        self.cache = max(self.cache, len(quantized))
        self._mem.update(quantized)

    def quantize(self, e: int):
        w13, w2 = self.source(e)
        q13, s13 = codec.quant_blocks_128(np.asarray(w13, dtype=np.float64))
        q2, s2 = codec.quant_blocks_128(np.asarray(w2, dtype=np.float64))
        return q13, s13, q2, s2

    def get(self, e: int):
        if e not in self._mem:
            q = self.quantize(e)
            if len(self._mem) >= self.cache:
                self._mem.pop(next(iter(self._mem)))
            self._mem[e] = q
        return self._mem[e]


# Accumulation error of a computed dot product relative to the Euclidean norm of its products
# (the float32 matrix-core accumulation, whose internal sums are not exact float32 sums; the
# rounding errors of a long sum add up like a random walk, so their total scales with the norm
# of the terms rather than with the sum of their magnitudes): the default `acc_err` of the h
# error model below.
ACC_ERR = 2.0 ** -13


def h_error_bound(x, w13, gu, acc_err=ACC_ERR):
    """Per element, how far a computation of h = silu(g) * u is taken to be from the exact
    value: each gate and up sum g, u carries an error up to acc_err * sqrt(sum_i (x_i w_i)^2)
    and the SwiGLU itself a relative acc_err; to first order
    |dh| <= |silu'(g) u| dg + |silu(g)| du + acc_err |h|, silu'(g) = s (1 + g (1 - s)),
    s = 1 / (1 + exp(-g)).  x [R, K], w13 [K, 2I], gu = x @ w13 -> [R, I]."""
    S = np.sqrt((x * x) @ (w13 * w13))
    I = w13.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    s = 1.0 / (1.0 + np.exp(-g))
    return acc_err * (np.abs(s * (1.0 + g * (1.0 - s)) * u) * S[:, :I] + np.abs(g * s) * S[:, I:] + np.abs(g * s * u))


def expert_ffn(xq_rows, xs_rows, q13, s13, q2, s2, acc_err=ACC_ERR, b13=None, b2=None):
    """One expert on a stack of quantised rows.

    Returns (o float64 [R, H], hq uint8 [R, I], hs uint8 [R, I/128], margin float64 [R],
    bound float64 [R, H], h float64 [R, I], h_err float64 [R, I]): margin is the
    re-quantisation's decision margin per row (``codec.decision_margin_rows_128``); h is the
    SwiGLU output before re-quantisation and h_err its error bound (``h_error_bound``); bound is
    the largest change of o that taking the other way any re-quantisation decision lying within
    h_err of a tie can make (``codec.flip_bound``).  b13 [2I] / b2 [H]: optional biases of the
    gate+up sums and of o."""
    x = codec.dequant_rows_128(xq_rows, xs_rows)
    w13 = codec.dequant_blocks_128(q13, s13)
    gu = x @ w13
    if b13 is not None:
        gu = gu + np.asarray(b13, dtype=np.float64)
    I = w13.shape[1] // 2
    h = silu(gu[:, :I]) * gu[:, I:]
    h_err = h_error_bound(x, w13, gu, acc_err)
    hq, hs = codec.quant_rows_128(h)
    w2 = codec.dequant_blocks_128(q2, s2)
    o = codec.dequant_rows_128(hq, hs) @ w2
    if b2 is not None:
        o = o + np.asarray(b2, dtype=np.float64)
    return o, hq, hs, codec.decision_margin_rows_128(h), codec.flip_bound(h, w2, codec.GROUP, h_err), h, h_err


def combine(o_flat: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y[t] = sum_j weights[t, j] * o_flat[t*k + j]."""
    T, k = weights.shape
    o = o_flat.reshape(T, k, -1)
    return (weights[:, :, None] * o).sum(axis=1)


def forward(x_f64, ids, weights, experts: QuantizedExperts, tokens=None, acc_err=ACC_ERR, ffn_map=None,
            biases=None):
    """Expert step for the given routing.

    x_f64 [T, H]: exact values of the bfloat16 hidden state.  ids/weights [T, k].
    tokens: optional array of token indices; only those rows of y are computed.
    Returns a dict with y float64 [len(tokens), H], o [len(tokens)*k, H] in flat
    (t, j) order, hq/hs, h and its error bound h_err by assignment, xq/xs of the tokens, the
    re-quantisation decision margin by assignment ("qmargin") and by token ("qmargin_tok", the
    smallest over its k assignments), and the near-tie flip bounds of o ("o_bound", by
    assignment) and of y ("y_bound" = sum_j |w[t, j]| * o_bound of slot j): the largest change
    of each output element that re-quantisation decisions lying within h_err of a tie could
    make (``expert_ffn``).

    ffn_map: optional callable (jobs, acc_err) -> results that runs ``expert_ffn`` on each job
    (e, xq rows, xs rows, b13 or None, b2 or None) with expert e's weights (e.g. in worker
    processes) and returns the results in job order; by default they run here with
    ``experts.get(e)``.  biases: optional (w13_bias [E, 2I], w2_bias [E, H]) float arrays."""
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    xq, xs = codec.quant_rows_128(x_f64[tok])
    sub_ids = ids[tok]
    n = len(tok)
    H = x_f64.shape[1]
    o = np.zeros((n * k, H))
    ob = np.zeros((n * k, H))
    qm = np.full(n * k, np.inf)
    hq = hs = h = h_err = None
    flat_ids = sub_ids.reshape(-1)
    groups = [(int(e), np.nonzero(flat_ids == e)[0]) for e in np.unique(flat_ids)]   # flat positions
    jobs = [(e, xq[rows // k], xs[rows // k], None if biases is None else biases[0][e],
             None if biases is None else biases[1][e]) for e, rows in groups]
    if ffn_map is None:
        results = [expert_ffn(xr, sr, *experts.get(e), acc_err, b13, b2) for e, xr, sr, b13, b2 in jobs]
    else:
        results = ffn_map(jobs, acc_err)
    for (e, rows), (oe, hqe, hse, qme, obe, he, hee) in zip(groups, results):
        if hq is None:
            hq = np.zeros((n * k, hqe.shape[1]), dtype=np.uint8)
            hs = np.zeros((n * k, hse.shape[1]), dtype=np.uint8)
            h = np.zeros((n * k, he.shape[1]))
            h_err = np.zeros((n * k, he.shape[1]))
        o[rows] = oe
        ob[rows] = obe
        hq[rows] = hqe
        hs[rows] = hse
        h[rows] = he
        h_err[rows] = hee
        qm[rows] = qme
    w = np.asarray(weights, dtype=np.float64)[tok]
    y = combine(o, w)
    return {"y": y, "o": o, "hq": hq, "hs": hs, "h": h, "h_err": h_err, "xq": xq, "xs": xs, "tokens": tok,
            "qmargin": qm, "qmargin_tok": qm.reshape(n, k).min(axis=1),
            "o_bound": ob, "y_bound": combine(ob, np.abs(w))}


def forward_shared(x_f64, ids, weights, experts: QuantizedExperts, shared: int, tokens=None, acc_err=ACC_ERR,
                   ffn_map=None, biases=None):
    """Routed experts plus one shared expert that every token runs through, added with
    weight 1 (the metrale grouped FP8 MoE page: the W8A8 gate_up and down launches also take
    the shared expert's gate/up/down projections and write its activations and output
    beside the routed ones):

        y[t] = sum_j weights[t, j] * o_{ids[t, j]}(t) + o_shared(t),

    o_shared being the same quantised SwiGLU FFN (steps 2-6) with expert ``shared``'s
    weights.  Written as the routed forward over k + 1 slots, slot k holding the shared
    expert with weight 1; the result dict is the routed one over those k + 1 slots."""
    T = ids.shape[0]
    ids_all = np.concatenate([np.asarray(ids), np.full((T, 1), shared, dtype=np.asarray(ids).dtype)], axis=1)
    w_all = np.concatenate([np.asarray(weights, dtype=np.float64), np.ones((T, 1))], axis=1)
    return forward(x_f64, ids_all, w_all, experts, tokens, acc_err, ffn_map, biases)


def route_workload(inputs: dict, p: routing.RouteParams, prelude=None):
    """Routing for either given logits or the gate prelude.

    prelude: None or (norm_w, router_w, pe_scale, eps).  Returns (ids, weights, margin)
    where margin is the near-tie measure for scores the device must compute (group
    scores in mode 1, prelude logits); inf where selection is exact."""
    if prelude is None:
        ids, w, gm = routing.route(inputs["logits"], p)
        margin = gm if p.group_select_mode == 1 and p.group_count > 1 else np.full(len(ids), np.inf)
        return ids, w, margin
    norm_w, router_w, pe_scale, eps = prelude
    ids, w, _, m = routing.route_prelude(inputs["x"], norm_w, router_w, pe_scale, eps, p.top_k)
    return ids, w * p.routed_scaling_factor, m
