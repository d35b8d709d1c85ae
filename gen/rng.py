"""Counter-based random numbers that come out bit-identical on the CPU and on a GPU.

The generator is SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): the i-th output of a stream with key
``k`` is ``mix64(k + (i + 1) * GAMMA)`` where ``mix64`` is the 64-bit finaliser of that
paper (Stafford's "variant 13" constants).  Every output is a pure function of
``(key, i)``, so any slice of a tensor can be produced on its own, on any device.

All arithmetic is int64 two's-complement wrap-around (logical right shifts are spelled
as an arithmetic shift plus a mask), followed by conversions that IEEE-754 rounds
exactly the same way everywhere: an integer of at most 24 bits to float32, and one
float32 multiply.  That is what makes a CPU tensor and a GPU tensor of the same
stream bit-identical, which lets the oracle regenerate any expert's weights on the
host without copying them back from device memory.

Normal variates use the Irwin-Hall sum of four 16-bit uniforms (the four 16-bit
quarters of one 64-bit output), centred and scaled to unit variance.  Its support is
bounded at +-2*sqrt(3) standard deviations; the rest of its shape is close to a
Gaussian.  This is a synthetic-input choice, not part of the MoE method.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(v: int) -> int:
    """An unsigned 64-bit constant as the signed int64 with the same bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def mix64_int(z: int) -> int:
    """Pure-Python SplitMix64 finaliser on an unsigned 64-bit integer."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, cfg: int, stream: int, index: int = 0) -> int:
    """Key of one named stream: (seed, workload id, tensor id, expert index)."""
    assert 0 <= seed < 256 and 0 <= cfg < 256 and 0 <= stream < 65536 and 0 <= index < (1 << 32)
    return mix64_int((seed << 56) | (cfg << 48) | (stream << 32) | index)


def raw_u64(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """Outputs start .. start+n-1 of stream ``key`` as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64_t(i * _s64(GAMMA) + _s64(key))


def normal_f32(key: int, n: int, std: float, device="cpu", start: int = 0) -> torch.Tensor:
    """n approximately N(0, std^2) float32 values (Irwin-Hall of four 16-bit uniforms)."""
    u = raw_u64(key, n, device, start)
    s = (u & 0xFFFF) + (_lsr(u, 16) & 0xFFFF) + (_lsr(u, 32) & 0xFFFF) + _lsr(u, 48)
    del u
    c = (s - 2 * 65535).to(torch.float32)  # |c| <= 131070 < 2^24: exact
    scale = torch.tensor(np.float32(std * math.sqrt(3.0) / 65536.0), dtype=torch.float32, device=device)
    return c * scale


def uniform_f32(key: int, n: int, lo: float, hi: float, device="cpu") -> torch.Tensor:
    """n float32 values in [lo, hi): 24 random bits scaled exactly, then one multiply-add."""
    u = _lsr(raw_u64(key, n, device), 40).to(torch.float32) * np.float32(2.0 ** -24)
    width = torch.tensor(np.float32(hi - lo), dtype=torch.float32, device=device)
    lo_t = torch.tensor(np.float32(lo), dtype=torch.float32, device=device)
    return u * width + lo_t


def normal_f32_chunked(key: int, n: int, std: float, device="cpu", chunk: int = 1 << 25) -> torch.Tensor:
    """normal_f32 produced in slices so the int64 temporaries stay small."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = normal_f32(key, m, std, device, start=s)
    return out
