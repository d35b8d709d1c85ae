"""E4M3 / UE8M0 codecs and the power-of-two group quantiser (CPU, float64).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Formats
-------
* E4M3FN ("FP8 E4M3"), the format named by the metrale ``fp8_grouped_tc_w8a8.rs``
  module doc (layer input and SiLU products quantised to E4M3) and by the MindIE-SD
  ``fused_moe`` MXFP8 example (``torch.float8_e4m3fn``, section "MXFP8 dynamic quant
  MoE").  A byte b has sign s = b>>7, exponent field e = (b>>3)&15, mantissa m = b&7;
  e = 0 is subnormal (m/8 * 2^-6), otherwise (1 + m/8) * 2^(e-7); the two bytes
  0x7F/0xFF are NaN and there is no infinity.  Largest finite value: 448.
* UE8M0, the unsigned power-of-two scale of the DeepGEMM W8A8 Mega MoE pull request
  ("Changes": 4-packed UE8M0 scale factors): byte b means 2^(b-127); 255 is NaN.

Quantiser (the pages name E4M3 values with power-of-two scales per (row, 128-column
group) for activations and per 128x128 block for weights, but give no rule for choosing
the scale; the reading used here is the smallest power of two that makes every element
of the group fit):

    amax = max |v| over the group
    e    = smallest integer with amax <= 448 * 2^e, clamped to [-127, 127];  e = 0 if amax = 0
    q    = E4M3_RNE(v / 2^e)      (v / 2^e is exact; |v / 2^e| <= 448, so nothing saturates)
    scale byte = e + 127

Pins (tests/test_oracle_codec.py): decode agrees with torch.float8_e4m3fn on all 256
codes; encode agrees with a brute-force nearest-code search and with the torch cast on
every representable value, every midpoint and its neighbours; UE8M0 round-trips all
255 finite codes; the scale rule is checked against hand values and its invariant
(amax / 2^e in (224, 448]); quantise-dequantise is the identity on groups built from
representable values; the decision margin matches hand values (0 at a rounding midpoint
and at a scale boundary) and no perturbation below it changes a code, while one just
above it at the closest element does.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GROUP = 128


def e4m3_decode_table() -> np.ndarray:
    """Float64 value of every E4M3FN byte, from the bit fields."""
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[b] = -v if s else v
    return t


_DEC = e4m3_decode_table()
_MAGS = _DEC[:127].copy()          # codes 0..126: the non-negative finite values, increasing


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    return _DEC[np.asarray(b, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto E4M3FN codes; |v| > 448 saturates to 448; sign kept.

    The nearest code is found by binary search in the increasing table of the 127
    non-negative finite values; on an exact tie the code with a zero last bit wins
    (that is "ties to even": the last code bit is the mantissa LSB).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    sign = np.signbit(v).astype(np.uint8)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # _MAGS[hi-1] < a <= _MAGS[hi]
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _MAGS[hi], hi, code).astype(np.uint8)   # exact hits (incl. 0)
    return code | (sign << 7)


def e4m3_encode_bruteforce(v) -> np.ndarray:
    """Slow reference: distance to all 127 magnitudes, ties to the even code."""
    v = np.atleast_1d(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(v):
        a = min(abs(x), E4M3_MAX)
        best = None
        for c in range(127):
            d = abs(_MAGS[c] - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        out[i] = best[1] | (0x80 if np.signbit(x) else 0)
    return out


def ue8m0_decode(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, (b - 127).clip(-127, 127)))


def ue8m0_encode(e: np.ndarray) -> np.ndarray:
    e = np.asarray(e, dtype=np.int64)
    if (e < -127).any() or (e > 127).any():
        raise ValueError("ue8m0_encode: exponent out of [-127, 127]")
    return (e + 127).astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (exact float64 tests), clamped to
    [-127, 127]; 0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # fix up any off-by-one of log2 with exact comparisons against 448 * 2^e
    for _ in range(2):
        e = np.where(safe > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
        e = np.where(safe <= E4M3_MAX * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(pos, e, 0)
    return np.clip(e, -127, 127)


def quantize_group(v: np.ndarray, e: np.ndarray) -> np.ndarray:
    """E4M3 codes of v / 2^e (e broadcast against v)."""
    return e4m3_encode(np.ldexp(np.asarray(v, dtype=np.float64), -np.asarray(e)))


def quant_rows_128(v: np.ndarray):
    """Per (row, 128-column group) quantisation of a [R, C] array, C % 128 == 0.

    Returns (q uint8 [R, C], scale bytes uint8 [R, C/128])."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % GROUP:
        raise ValueError("columns must be a multiple of 128")
    g = v.reshape(R, C // GROUP, GROUP)
    e = scale_exponent(np.abs(g).max(axis=2))
    q = quantize_group(g, e[:, :, None]).reshape(R, C)
    return q, ue8m0_encode(e)


def decision_margin_rows_128(v: np.ndarray) -> np.ndarray:
    """How far each row's quantisation decisions (``quant_rows_128``) are from flipping.

    For a [R, C] array returns [R]: the smallest relative distance, over the row, from an
    element's |v| / 2^e to the nearest E4M3 rounding midpoint (the value halfway between
    two adjacent magnitudes, where round-to-nearest changes code), and from each group's
    amax to the two scale boundaries 448 * 2^(e-1) and 448 * 2^e (where the scale rule
    changes e).  A computation of v carrying relative error below this margin takes every
    decision of the row the same way; zero elements take no rounding decision.  Rows of
    all-zero groups get +inf."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % GROUP:
        raise ValueError("columns must be a multiple of 128")
    g = np.abs(v.reshape(R, C // GROUP, GROUP))
    amax = g.max(axis=2)
    e = scale_exponent(amax)
    s = np.ldexp(g, -e[:, :, None])
    mags = np.unique(np.abs(e4m3_decode_table()[np.isfinite(e4m3_decode_table())]))   # 0 .. 448
    mids = (mags[1:] + mags[:-1]) / 2
    i = np.clip(np.searchsorted(mids, s), 1, len(mids) - 1)
    d = np.minimum(np.abs(s - mids[i - 1]), np.abs(s - mids[i]))
    rel = np.where(s > 0, d / np.where(s > 0, s, 1.0), np.inf)
    pos = amax > 0
    lo = E4M3_MAX * np.ldexp(1.0, e - 1)
    hi = E4M3_MAX * np.ldexp(1.0, e)
    srel = np.where(pos, np.minimum(np.abs(amax / lo - 1), np.abs(amax / hi - 1)), np.inf)
    return np.minimum(rel.min(axis=(1, 2)), srel.min(axis=1))


def _e4m3_magnitudes() -> np.ndarray:
    t = e4m3_decode_table()
    return np.unique(np.abs(t[np.isfinite(t)]))          # 0 .. 448, increasing


def near_tie_flips(v: np.ndarray, group: int, tol):
    """The E4M3 re-quantisation decisions of ``quant`` per (row, `group` columns) of v (scale
    rule above) that a computation of v carrying an absolute error up to `tol` (an array
    broadcastable to v, or a number) could take the other way, and what taking each the other
    way changes in the dequantised row.

    A decision is
      * an element's rounding: |v| within tol of the rounding midpoint (times 2^e) between
        the two magnitudes nearest to |v| / 2^e; the other way is the magnitude across that
        midpoint (same sign; for a zero element, either sign);
      * a group's scale: its amax within the group's largest tol of 448 * 2^(e-1) (the other
        way is e - 1) or of 448 * 2^e (the other way is e + 1); taking it re-quantises the
        whole group.
    Returns (elem, scale): elem [R, C] float64 holding dequant(other code) - dequant(code) at
    the near-tie elements and 0 elsewhere; scale a list of (row, first column, delta [group])
    for the near-tie scales."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % group:
        raise ValueError(f"columns must be a multiple of {group}")
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), v.shape).reshape(R, C // group, group)
    g = v.reshape(R, C // group, group)
    amax = np.abs(g).max(axis=2)
    e = scale_exponent(amax)
    pw = np.ldexp(1.0, e)[:, :, None]
    s = np.abs(g) / pw
    mags = _e4m3_magnitudes()
    mids = (mags[1:] + mags[:-1]) / 2
    # nearest midpoint m: between mags[m] and mags[m + 1]
    j = np.clip(np.searchsorted(mids, s), 1, len(mids) - 1)
    m = np.where(np.abs(s - mids[j - 1]) <= np.abs(s - mids[j]), j - 1, j)
    near = np.abs(s - mids[m]) * pw < tol      # a zero element too: a computed one may not be zero
    chosen = np.abs(e4m3_decode(e4m3_encode(g / pw)))
    other = np.where(chosen == mags[m], mags[m + 1], mags[m])
    sign = np.where(np.signbit(g), -1.0, 1.0)
    elem = np.where(near, sign * (other - chosen) * pw, 0.0).reshape(R, C)
    scale = []
    pos = amax > 0
    gtol = tol.max(axis=2)
    lo = E4M3_MAX * np.ldexp(1.0, e - 1)
    hi = E4M3_MAX * np.ldexp(1.0, e)
    for alt, bound in ((-1, lo), (1, hi)):
        for r, c in zip(*np.nonzero(pos & (np.abs(amax - bound) < gtol))):
            grp = g[r, c]
            cur = e4m3_decode(e4m3_encode(np.ldexp(grp, -e[r, c]))) * np.ldexp(1.0, e[r, c])
            ea = int(np.clip(e[r, c] + alt, -127, 127))
            new = e4m3_decode(e4m3_encode(np.ldexp(grp, -ea))) * np.ldexp(1.0, ea)
            scale.append((int(r), int(c) * group, new - cur))
    return elem, scale


def flip_bound(v: np.ndarray, w: np.ndarray, group: int, tol) -> np.ndarray:
    """Largest change of dequant(quant(v)) @ w, element by element, that taking any set of
    the near-tie decisions of ``near_tie_flips`` (absolute tolerance `tol`) the other way can
    make (each decision's effect added in absolute value).  v [R, C], w [C, N] -> [R, N]."""
    elem, scale = near_tie_flips(v, group, tol)
    w = np.asarray(w, dtype=np.float64)
    out = np.zeros((v.shape[0], w.shape[1]))
    rows, cols = np.nonzero(elem)
    if len(rows):
        np.add.at(out, rows, np.abs(elem[rows, cols])[:, None] * np.abs(w[cols]))
    for r, c0, d in scale:
        out[r] += np.abs(d @ w[c0:c0 + len(d)])
    return out


def dequant_rows_128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    R, C = q.shape
    vals = e4m3_decode(q).reshape(R, C // GROUP, GROUP)
    return (vals * ue8m0_decode(s)[:, :, None]).reshape(R, C)


def quant_blocks_128(w: np.ndarray):
    """Per 128x128 block quantisation of a [K, N] weight (blocks tile (K, N)).

    Returns (q uint8 [K, N], scale bytes uint8 [K/128, N/128])."""
    w = np.asarray(w, dtype=np.float64)
    K, N = w.shape
    if K % GROUP or N % GROUP:
        raise ValueError("weight dims must be multiples of 128")
    b = w.reshape(K // GROUP, GROUP, N // GROUP, GROUP)
    e = scale_exponent(np.abs(b).max(axis=(1, 3)))
    q = quantize_group(b, e[:, None, :, None]).reshape(K, N)
    return q, ue8m0_encode(e)


def dequant_blocks_128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    K, N = q.shape
    vals = e4m3_decode(q).reshape(K // GROUP, GROUP, N // GROUP, GROUP)
    return (vals * ue8m0_decode(s)[:, None, :, None]).reshape(K, N)
