"""Recompute the Zipf bias strength of the large-prefill workload.

The workload asks for a Zipf(s=1.1) per-expert logit bias such that the 8 hottest experts
receive about 40% of the top-8 assignments.  The bias profile is
bias_e = -1.1 * alpha * ln(e + 1); this script finds alpha by bisection, routing the seed-0
logits with the oracle, and prints it.  The value is stored as gen.workloads.ZIPF_ALPHA.

    python tests/golden/calibrate_zipf.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from gen import rng, workloads as W  # noqa: E402
from oracle import routing  # noqa: E402


def top8_share(alpha: float) -> float:
    wl = W.CONFIGS[5]
    noise = rng.normal_f32_chunked(wl.key(W.S_LOGITS), wl.T * wl.E, 1.0).view(wl.T, wl.E).numpy()
    bias = (-W.ZIPF_S * alpha * np.log(np.arange(wl.E) + 1.0)).astype(np.float32)
    ids, _, _ = routing.route(noise + bias[None, :], routing.RouteParams(wl.E, wl.k, "softmax", True))
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    return np.sort(counts)[::-1][:8].sum() / counts.sum()


def main():
    lo, hi = 0.1, 1.5
    for _ in range(30):
        mid = (lo + hi) / 2
        if top8_share(mid) < 0.40:
            lo = mid
        else:
            hi = mid
    a = round((lo + hi) / 2, 3)
    print(f"alpha = {a}  top-8 share = {top8_share(a):.4f}")


if __name__ == "__main__":
    main()
