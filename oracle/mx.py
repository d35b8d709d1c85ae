"""Micro-scaled (32-element group) formats of the expert step: MXFP8 and W4A8 (CPU, float64).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Two variants of the routed FP8 expert step that the pages describe next to the
128-block one:

* MXFP8 (MindIE-SD ``fused_moe``, section "MXFP8 dynamic quant MoE", and the MATE Mega MoE
  ``recipe=(1, 1, 32)``): E4M3FN activations and weights with one UE8M0 scale per 32
  elements.  The page's weight preparation quantises ``weight.transpose(1, 2)`` along its
  last axis, i.e. along K, and reshapes the scales to [experts, N, K/64, 2]: one scale per
  (32 consecutive rows of K, one column).
* W4A8 (the FP8 x FP4 Mega MoE path of the DeepGEMM pull request, whose W8A8 variant
  "switches the weights from e2m1 to e4m3" and keeps the UE8M0 scale handling; the
  MATE page's W4A8 mixed-dtype GEMM): the same activations, weights in E2M1 (FP4) with one
  UE8M0 scale per (32 rows of K, one column).

E2M1 (the 4-bit float of the OCP micro-scaling formats): sign bit, 2 exponent bits (bias
1), 1 mantissa bit; exponent field 0 is subnormal (m * 0.5).  Magnitudes of codes 0..7:
0, 0.5, 1, 1.5, 2, 3, 4, 6.  No infinity or NaN.  Code c's low bit is its mantissa bit.

Scale rule (readings; the pages name the UE8M0 scale per 32 elements but not how it is
chosen): the rule of the 128-element path, with the format's largest magnitude M (448 for
E4M3, 6 for E2M1):

    amax = max |v| over the group
    e    = smallest integer with amax <= M * 2^e, clamped to [-127, 127];  e = 0 if amax = 0
    q    = RNE(v / 2^e) onto the format's codes (exact division; |v / 2^e| <= M, so nothing
           saturates); ties go to the code with a zero last bit; the sign of zero is kept
    scale byte = e + 127

Groups: activations and the re-quantised SwiGLU output h per (row, 32 consecutive
columns); weights per (32 consecutive rows of K, one column).  The expert FFN is the
128-path one (``oracle.moe``) with these quantisers: gu = dequant(xq) @ dequant(w13),
h = silu(gu[:I]) * gu[I:], hq = quant_rows_32(h) in E4M3, o = dequant(hq) @ dequant(w2).

Pins (tests/test_oracle_mx.py): the E2M1 table against the bit-field definition and the
hand values of tests/golden/e2m1_hand.txt; encode against a brute-force nearest-code
search on every midpoint and its neighbours; the scale rule's invariant
(amax / 2^e in (M/2, M]); the round trip on groups of representable values; the
re-quantisation decision margin against hand values and single-element perturbations; the FFN
against a dense float64 SwiGLU MLP for one token, one expert; and the 32-group E4M3 FFN
against the 128-group oracle where the two coincide (every 32-group of a 128-group has
the same scale).
"""
from __future__ import annotations

import numpy as np

from . import codec, moe

MX = 32
E2M1_MAX = 6.0
FMT_E4M3, FMT_E2M1 = "e4m3", "e2m1"


def e2m1_decode_table() -> np.ndarray:
    """Float64 value of each 4-bit E2M1 code 0..15, from the bit fields."""
    t = np.empty(16, dtype=np.float64)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        t[c] = -v if s else v
    return t


_E2M1 = e2m1_decode_table()
_E2M1_MAGS = _E2M1[:8].copy()     # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    return _E2M1[np.asarray(c, dtype=np.uint8) & 15]


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto E2M1 codes (uint8, low nibble); |v| > 6 saturates; sign kept."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    sign = np.signbit(v).astype(np.uint8)
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_E2M1_MAGS, a, side="left"), 7)   # mags[hi-1] < a <= mags[hi]
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E2M1_MAGS[lo]
    d_hi = _E2M1_MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E2M1_MAGS[hi], hi, code).astype(np.uint8)
    return code | (sign << 3)


def e2m1_encode_bruteforce(v) -> np.ndarray:
    """Slow reference: distance to all 8 magnitudes, ties to the even code."""
    v = np.atleast_1d(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(v):
        a = min(abs(x), E2M1_MAX)
        best = None
        for c in range(8):
            d = abs(_E2M1_MAGS[c] - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        out[i] = best[1] | (8 if np.signbit(x) else 0)
    return out


def fmt_max(fmt: str) -> float:
    return {FMT_E4M3: codec.E4M3_MAX, FMT_E2M1: E2M1_MAX}[fmt]


def scale_exponent(amax: np.ndarray, fmt: str) -> np.ndarray:
    """Smallest integer e with amax <= M * 2^e (exact float64 tests), clamped to
    [-127, 127]; 0 where amax == 0."""
    M = fmt_max(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    e = np.ceil(np.log2(safe / M)).astype(np.int64)
    for _ in range(2):
        e = np.where(safe > M * np.ldexp(1.0, e), e + 1, e)
        e = np.where(safe <= M * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(pos, e, 0)
    return np.clip(e, -127, 127)


def encode(v: np.ndarray, fmt: str) -> np.ndarray:
    return codec.e4m3_encode(v) if fmt == FMT_E4M3 else e2m1_encode(v)


def decode(c: np.ndarray, fmt: str) -> np.ndarray:
    return codec.e4m3_decode(c) if fmt == FMT_E4M3 else e2m1_decode(c)


def quant_rows_32(v: np.ndarray, fmt: str = FMT_E4M3):
    """Per (row, 32-column group) quantisation of [R, C], C % 32 == 0.
    Returns (codes uint8 [R, C], scale bytes uint8 [R, C/32])."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % MX:
        raise ValueError("columns must be a multiple of 32")
    g = v.reshape(R, C // MX, MX)
    e = scale_exponent(np.abs(g).max(axis=2), fmt)
    q = encode(np.ldexp(g, -e[:, :, None]), fmt).reshape(R, C)
    return q, codec.ue8m0_encode(e)


def dequant_rows_32(q: np.ndarray, s: np.ndarray, fmt: str = FMT_E4M3) -> np.ndarray:
    R, C = q.shape
    return (decode(q, fmt).reshape(R, C // MX, MX) * codec.ue8m0_decode(s)[:, :, None]).reshape(R, C)


def quant_weight_k32(w: np.ndarray, fmt: str):
    """Per (32 rows of K, one column) quantisation of a [K, N] weight, K % 32 == 0.
    Returns (codes uint8 [K, N], scale bytes uint8 [K/32, N])."""
    w = np.asarray(w, dtype=np.float64)
    K, N = w.shape
    if K % MX:
        raise ValueError("K must be a multiple of 32")
    b = w.reshape(K // MX, MX, N)
    e = scale_exponent(np.abs(b).max(axis=1), fmt)
    q = encode(np.ldexp(b, -e[:, None, :]), fmt).reshape(K, N)
    return q, codec.ue8m0_encode(e)


def dequant_weight_k32(q: np.ndarray, s: np.ndarray, fmt: str) -> np.ndarray:
    K, N = q.shape
    return (decode(q, fmt).reshape(K // MX, MX, N) * codec.ue8m0_decode(s)[:, None, :]).reshape(K, N)


def decision_margin_rows_32(v: np.ndarray) -> np.ndarray:
    """How far each row's E4M3 32-group quantisation decisions (``quant_rows_32``) are from
    flipping: for [R, C] returns [R], the smallest relative distance over the row from an
    element's |v| / 2^e to the nearest E4M3 rounding midpoint and from each group's amax to
    its two scale boundaries 448 * 2^(e-1) and 448 * 2^e.  A computation of v with relative
    error below this margin takes every decision the same way; zero elements take none.
    Rows of all-zero groups get +inf."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % MX:
        raise ValueError("columns must be a multiple of 32")
    g = np.abs(v.reshape(R, C // MX, MX))
    amax = g.max(axis=2)
    e = scale_exponent(amax, FMT_E4M3)
    s = np.ldexp(g, -e[:, :, None])
    tab = codec.e4m3_decode_table()
    mags = np.unique(np.abs(tab[np.isfinite(tab)]))
    mids = (mags[1:] + mags[:-1]) / 2
    i = np.clip(np.searchsorted(mids, s), 1, len(mids) - 1)
    d = np.minimum(np.abs(s - mids[i - 1]), np.abs(s - mids[i]))
    rel = np.where(s > 0, d / np.where(s > 0, s, 1.0), np.inf)
    pos = amax > 0
    lo = codec.E4M3_MAX * np.ldexp(1.0, e - 1)
    hi = codec.E4M3_MAX * np.ldexp(1.0, e)
    srel = np.where(pos, np.minimum(np.abs(amax / lo - 1), np.abs(amax / hi - 1)), np.inf)
    return np.minimum(rel.min(axis=(1, 2)), srel.min(axis=1))


class QuantizedExpertsMX(moe.QuantizedExperts):
    """Per-expert weights in the given weight format with (32 x 1) UE8M0 scales."""

    def __init__(self, source, fmt: str, cache: int = 4):
        super().__init__(source, cache)
        self.fmt = fmt

    def quantize(self, e: int):
        w13, w2 = self.source(e)
        q13, s13 = quant_weight_k32(np.asarray(w13, dtype=np.float64), self.fmt)
        q2, s2 = quant_weight_k32(np.asarray(w2, dtype=np.float64), self.fmt)
        return q13, s13, q2, s2


def expert_ffn(xq_rows, xs_rows, q13, s13, q2, s2, fmt: str, acc_err=moe.ACC_ERR, b13=None, b2=None):
    """One expert on a stack of MX-quantised rows; weights in `fmt`.
    Returns (o float64 [R, H], hq uint8 [R, I], hs uint8 [R, I/32], margin float64 [R],
    bound float64 [R, H], h float64 [R, I], h_err float64 [R, I]): margin is the
    re-quantisation's decision margin per row (``decision_margin_rows_32``), h the SwiGLU output
    and h_err its error bound (``oracle.moe.h_error_bound``), bound the largest change of o the
    decisions within h_err of a tie could make (``codec.flip_bound`` on 32-column groups).
    b13 / b2: optional biases as in ``oracle.moe.expert_ffn``."""
    x = dequant_rows_32(xq_rows, xs_rows)
    w13 = dequant_weight_k32(q13, s13, fmt)
    gu = x @ w13
    if b13 is not None:
        gu = gu + np.asarray(b13, dtype=np.float64)
    I = w13.shape[1] // 2
    h = moe.silu(gu[:, :I]) * gu[:, I:]
    h_err = moe.h_error_bound(x, w13, gu, acc_err)
    hq, hs = quant_rows_32(h)
    w2 = dequant_weight_k32(q2, s2, fmt)
    o = dequant_rows_32(hq, hs) @ w2
    if b2 is not None:
        o = o + np.asarray(b2, dtype=np.float64)
    return o, hq, hs, decision_margin_rows_32(h), codec.flip_bound(h, w2, MX, h_err), h, h_err


def forward(x_f64, ids, weights, experts: QuantizedExpertsMX, tokens=None, acc_err=moe.ACC_ERR, ffn_map=None,
            biases=None):
    """Expert step for the given routing with MX activations and `experts.fmt` weights.
    Same contract as ``oracle.moe.forward`` (y float64 over the chosen tokens, o in flat
    (t, j) order, hq/hs and h by assignment, xq/xs of the tokens, margins and the near-tie
    flip bounds o_bound / y_bound; ffn_map as there, running this module's ``expert_ffn``)."""
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    xq, xs = quant_rows_32(x_f64[tok])
    n = len(tok)
    H = x_f64.shape[1]
    o = np.zeros((n * k, H))
    ob = np.zeros((n * k, H))
    qm = np.full(n * k, np.inf)
    hq = hs = h = h_err = None
    flat_ids = ids[tok].reshape(-1)
    groups = [(int(e), np.nonzero(flat_ids == e)[0]) for e in np.unique(flat_ids)]
    jobs = [(e, xq[rows // k], xs[rows // k], None if biases is None else biases[0][e],
             None if biases is None else biases[1][e]) for e, rows in groups]
    if ffn_map is None:
        results = [expert_ffn(xr, sr, *experts.get(e), experts.fmt, acc_err, b13, b2) for e, xr, sr, b13, b2 in jobs]
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
    y = moe.combine(o, w)
    return {"y": y, "o": o, "hq": hq, "hs": hs, "h": h, "h_err": h_err, "xq": xq, "xs": xs, "tokens": tok,
            "qmargin": qm, "qmargin_tok": qm.reshape(n, k).min(axis=1),
            "o_bound": ob, "y_bound": moe.combine(ob, np.abs(w))}
