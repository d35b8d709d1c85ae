"""The W8A16 expert step (CPU, float64): E4M3 weights with UE8M0 128 x 128 block scales,
bf16 activations.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

The metrale grouped FP8 MoE page (module notes of its W8A8 expert step) keeps the experts
on W8A16 unless FP8 activations are published, and says the W8A8 output differs from the
W8A16 one only by the activation rounding.  Plainest reading, taken here: the W8A8 steps of
``oracle.moe`` with both activation quantisations replaced by bf16 — the layer input is the
bf16 value it already is, and the SiLU product is rounded once to bf16 (round to nearest,
ties to even) before the down projection:

1. route (``oracle.routing``), as for the FP8 step;
2. gate+up: gu = x @ dequant(w13[e]), float64, x the exact values of the bf16 row;
3. SwiGLU: h = silu(g) * u;
4. hb = bf16(h), round to nearest even (``bf16_rne``);
5. down: o = hb @ dequant(w2[e]), float64;
6. combine: y[t] = sum_j w[t, j] * o[(t, j)], float64 (bf16 rounding of y is the caller's).

Pins (tests/test_oracle_w8a16.py): ``bf16_rne`` equals torch's float32 -> bfloat16
conversion on float32 values (ties, subnormals, signs); a hand-worked FFN
(tests/golden/ffn_w8a16_hand.txt); one token, one expert, top-1 equals the dense SwiGLU MLP
computed by torch in float64 on the dequantised tensors with the bf16 rounding of h; and
the step reduces to ``oracle.moe.forward`` when x and h are exactly representable in both
schemes' activation formats.
"""
from __future__ import annotations

import numpy as np

from . import codec, moe


def bf16_rne(v) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    bfloat16 keeps 8 significant bits for normal values (|v| >= 2^-126) and a fixed spacing
    of 2^-133 below them.  Values beyond the bfloat16 range are not handled (the expert
    step stays far inside it)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                              # v = m * 2^e, 0.5 <= |m| < 1
    ulp = np.exp2(np.maximum(e, -125) - 8)
    return np.rint(v / ulp) * ulp                  # rint rounds halves to even


def expert_ffn(x_rows, q13, s13, q2, s2, b13=None, b2=None):
    """One expert on a stack of bf16 activation rows (float64 values).
    Returns (o float64 [R, H], hb float64 [R, I] holding bf16 values, h float64 [R, I] before
    the rounding, h_err float64 [R, I] its error bound (``oracle.moe.h_error_bound``)).
    b13 / b2: optional biases as in ``oracle.moe.expert_ffn``."""
    w13 = codec.dequant_blocks_128(q13, s13)
    x = np.asarray(x_rows, dtype=np.float64)
    gu = x @ w13
    if b13 is not None:
        gu = gu + np.asarray(b13, dtype=np.float64)
    I = w13.shape[1] // 2
    h = moe.silu(gu[:, :I]) * gu[:, I:]
    hb = bf16_rne(h)
    o = hb @ codec.dequant_blocks_128(q2, s2)
    if b2 is not None:
        o = o + np.asarray(b2, dtype=np.float64)
    return o, hb, h, moe.h_error_bound(x, w13, gu)


def forward(x_f64, ids, weights, experts: moe.QuantizedExperts, tokens=None, ffn_map=None, biases=None):
    """W8A16 expert step for the given routing (same experts object and result layout as
    ``oracle.moe.forward``).  There is no activation re-quantisation, so the decision
    margins ("qmargin", "qmargin_tok") are infinite and the flip bounds ("o_bound", "y_bound")
    zero: no output element is excused from the output bar.  ffn_map as in
    ``oracle.moe.forward``, with jobs (e, x rows, None) for this module's ``expert_ffn``."""
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    x = np.asarray(x_f64, dtype=np.float64)[tok]
    n = len(tok)
    H = x.shape[1]
    o = np.zeros((n * k, H))
    hb = h = h_err = None
    flat_ids = np.asarray(ids)[tok].reshape(-1)
    groups = [(int(e), np.nonzero(flat_ids == e)[0]) for e in np.unique(flat_ids)]   # flat positions
    jobs = [(e, x[rows // k], None, None if biases is None else biases[0][e], None if biases is None else biases[1][e])
            for e, rows in groups]
    if ffn_map is None:
        results = [expert_ffn(xr, *experts.get(e), b13, b2) for e, xr, _, b13, b2 in jobs]
    else:
        results = ffn_map(jobs, None)
    for (e, rows), (oe, hbe, he, hee) in zip(groups, results):
        if hb is None:
            hb = np.zeros((n * k, hbe.shape[1]))
            h = np.zeros((n * k, he.shape[1]))
            h_err = np.zeros((n * k, he.shape[1]))
        o[rows] = oe
        hb[rows] = hbe
        h[rows] = he
        h_err[rows] = hee
    y = moe.combine(o, np.asarray(weights, dtype=np.float64)[tok])
    qm = np.full(n * k, np.inf)
    return {"y": y, "o": o, "hb": hb, "h": h, "h_err": h_err, "tokens": tok, "qmargin": qm, "qmargin_tok": qm.reshape(n, k).min(axis=1),
            "o_bound": np.zeros_like(o), "y_bound": np.zeros_like(y)}
