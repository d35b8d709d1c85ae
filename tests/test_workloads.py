"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import torch

from gen import rng, workloads as W
from oracle import routing


def test_splitmix64_matches_pure_python():
    key = rng.stream_key(0, 3, 4, 17)
    got = rng.raw_u64(key, 64, start=1000)
    for i, v in enumerate(got.tolist()):
        assert (v & rng.MASK64) == rng.mix64_int(key + (1000 + i + 1) * rng.GAMMA)


def test_slices_are_independent_of_chunking():
    key = rng.stream_key(0, 1, 0)
    a = rng.normal_f32_chunked(key, 10000, 1.0, chunk=1 << 20)
    b = rng.normal_f32_chunked(key, 10000, 1.0, chunk=999)
    assert torch.equal(a, b)
    assert torch.equal(rng.normal_f32(key, 100, 1.0, start=500), a[500:600])


def test_normal_moments():
    x = rng.normal_f32(rng.stream_key(0, 9, 0), 1 << 20, 0.02).double()
    assert abs(x.mean().item()) < 1e-4
    assert abs(x.std().item() - 0.02) < 1e-4
    assert x.abs().max().item() <= 0.02 * 2 * 3 ** 0.5 + 1e-9


def test_uniform_range():
    u = rng.uniform_f32(rng.stream_key(0, 9, 1), 100000, 0.5, 1.5)
    assert u.min().item() >= 0.5 and u.max().item() < 1.5


def test_zipf_share_of_large_prefill():
    wl = W.CONFIGS[5]
    ids, _, _ = routing.route(W.router_logits(wl).numpy(), routing.RouteParams(wl.E, wl.k, "softmax", True))
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    share = np.sort(counts)[::-1][:8].sum() / counts.sum()
    assert abs(share - 0.40) < 0.01
    assert counts[0] == counts.max()


def test_config_shapes():
    c = W.CONFIGS
    assert (c[2].T, c[2].H, c[2].I, c[2].E, c[2].k) == (32, 2816, 768, 128, 8)
    assert (c[3].T, c[3].H, c[3].I, c[3].E, c[3].k) == (2048, 768, 1152, 256, 8)
    assert c[4].group_count == 8 and c[4].k_group == 4 and c[4].routed_scaling_factor == 2.5
    for wl in c.values():
        assert wl.H % 128 == 0 and wl.I % 128 == 0
