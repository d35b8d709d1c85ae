"""CPU oracle for the routed FP8 MoE expert step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy restatement of what the expert step computes, written
from the pages and checked against closed forms, brute force, library routines and
hand-worked cases (tests/test_oracle_*.py, tests/golden/).  It shares no code with the
HIP path and imports nothing from the product package; only tests/, the smoke check
of __graft_entry__ and the CPU-baseline leg of bench.py may use it.

Modules
-------
codec    E4M3FN and UE8M0 codecs, the power-of-two scale rule, per-(row, 128) and
         per-128x128-block quantisation.
routing  softmax / sigmoid top-k routing, group-limited selection, the RMSNorm +
         router gate prelude, and the stable expert permutation.
moe      the expert FFN (gate+up, SwiGLU, re-quantisation, down) and the weighted
         top-k combine, for all tokens or a sample of them.
mx       the micro-scaled schemes (MXFP8, W4A8): 32-element groups, E2M1.
w8a16    the weight-only scheme: E4M3 block-scaled weights, bf16 activations, h rounded
         once to bf16.

Every function is pinned; none is "parity unpinned".
"""
from . import codec, routing, moe, mx, w8a16  # noqa: F401
