"""Workload table and seeded input builders for the routed FP8 MoE expert step.

The five shapes follow the workloads the pages describe or imply:

* the Gemma-4-like decode gate (128 experts, top-8, hidden 2816) of the Metal
  ``moe_gate.rs`` page (module doc and ``MoeGateParams``);
* the unaligned grouped shape (E=256, top-8, 2048 tokens, hidden 768, intermediate
  1152) of the DeepGEMM W8A8 Mega MoE pull request ("Testing");
* a tiny case, a DeepSeek-V3-shaped prefill with group-limited sigmoid routing (the
  group knobs of the MindIE-SD ``fused_moe`` parameter table) and a large prefill with
  a Zipf-skewed expert load;
* one expert-parallel shard of that prefill (32 local experts, ~1024 rows each), the
  per-GPU shape of the MATE Mega MoE expert-parallel path on 8 ranks.

Value recipes (all seeded, all synthetic; no dataset is involved):

* hidden states x: N(0,1) float32, rounded to bfloat16 (round-to-nearest-even);
* router logits: N(0,1) float32 plus a per-expert float32 bias where the workload has
  one (N(0,1.5) for the unaligned shape; a Zipf profile for the large prefill);
* expert weights w13 [E,H,2I] and w2 [E,I,H]: N(0,0.02) float32, one stream per
  expert; the caller quantises them to E4M3 with 128x128 UE8M0 block scales;
* gate prelude (decode shape): RMSNorm weight 1+N(0,0.1), router weight N(0,0.02)
  float32 [E,H], per-expert scale U(0.5,1.5);
* optional expert biases: w13_bias N(0,0.25) float32 [E,2I], w2_bias N(0,0.1) [E,H].

Small per-expert vectors (biases, norm weight, router weight, per-expert scale) are
always generated on the CPU and moved, so that nothing here relies on a device's
transcendental functions.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

from . import rng

# stream ids
S_X, S_LOGITS, S_BIAS, S_W13, S_W2, S_WR, S_WNORM, S_PESCALE, S_B13, S_B2 = range(10)

# Zipf(s=1.1) bias profile: bias_e = -1.1 * ZIPF_ALPHA * ln(e + 1).  ZIPF_ALPHA was
# calibrated at seed 0 so that experts 0..7 receive about 40% of the top-8 assignments
# of the large-prefill workload (tests/golden/calibrate_zipf.py recomputes it with the
# oracle's routing; tests/test_workloads.py checks the share).
ZIPF_S = 1.1
ZIPF_ALPHA = 0.543


@dataclass(frozen=True)
class Workload:
    cfg: int            # workload id, part of every stream key
    name: str
    T: int              # tokens
    H: int              # hidden size
    I: int              # expert intermediate size
    E: int              # experts (all local)
    k: int              # top-k
    scoring: str = "softmax"       # "softmax" | "sigmoid"
    renormalize: bool = True
    group_count: int = 1
    k_group: int = 1
    group_select_mode: int = 0     # 0: max score in group, 1: sum of top-2 scores
    routed_scaling_factor: float = 1.0
    prelude: bool = False          # RMSNorm + fp32 router matmul + per-expert scale
    rms_eps: float = 1e-6
    bias: str = "none"             # "none" | "normal1.5" | "zipf"
    seed: int = 0
    shared: int = 0                # 1: one shared expert (weights of expert index E) on every token
    ffn_bias: bool = False         # per-expert gate/up and down biases (w13_bias, w2_bias)

    @property
    def A(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def key(self, stream: int, index: int = 0) -> int:
        return rng.stream_key(self.seed, self.cfg, stream, index)

    def flops(self) -> float:
        """Algorithmic FP8 GEMM flops: gate+up (2*A*H*2I) plus down (2*A*I*H), over the
        routed assignments and the shared expert's T rows."""
        return 6.0 * self.T * (self.k + self.shared) * self.H * self.I


CONFIGS = {
    1: Workload(1, "tiny", T=64, H=256, I=512, E=8, k=2, scoring="softmax", renormalize=True),
    2: Workload(2, "decode_gemma4", T=32, H=2816, I=768, E=128, k=8, scoring="softmax",
                renormalize=True, prelude=True, rms_eps=1e-6),
    3: Workload(3, "unaligned_grouped", T=2048, H=768, I=1152, E=256, k=8, scoring="softmax",
                renormalize=True, bias="normal1.5"),
    4: Workload(4, "prefill_dsv3", T=4096, H=7168, I=2048, E=256, k=8, scoring="sigmoid",
                renormalize=True, group_count=8, k_group=4, group_select_mode=1,
                routed_scaling_factor=2.5),
    5: Workload(5, "prefill_zipf", T=16384, H=4096, I=1536, E=128, k=8, scoring="softmax",
                renormalize=True, bias="zipf"),
    # One expert-parallel shard of the DeepSeek-V3-shaped prefill on 8 GPUs: the GPU holds 32
    # of the 256 experts and receives every assignment routed to them, about 8x the rows per
    # expert of the one-GPU case (32768 assignments over 32 experts, ~1024 rows each).  Routing
    # keeps the group-limited sigmoid knobs on the local experts (8 groups of 4).
    6: Workload(6, "ep8_shard_dsv3", T=4096, H=7168, I=2048, E=32, k=8, scoring="sigmoid",
                renormalize=True, group_count=8, k_group=4, group_select_mode=1,
                routed_scaling_factor=2.5),
}


def hidden_f32(wl: Workload, device="cpu") -> torch.Tensor:
    return rng.normal_f32_chunked(wl.key(S_X), wl.T * wl.H, 1.0, device).view(wl.T, wl.H)


def hidden_bf16(wl: Workload, device="cpu") -> torch.Tensor:
    return hidden_f32(wl, device).to(torch.bfloat16)


def expert_bias(wl: Workload) -> torch.Tensor:
    """Per-expert float32 logit bias (CPU)."""
    if wl.bias == "none":
        return torch.zeros(wl.E, dtype=torch.float32)
    if wl.bias == "normal1.5":
        return rng.normal_f32(wl.key(S_BIAS), wl.E, 1.5)
    if wl.bias == "zipf":
        e = np.arange(wl.E, dtype=np.float64)
        return torch.from_numpy((-ZIPF_S * ZIPF_ALPHA * np.log(e + 1.0)).astype(np.float32))
    raise ValueError(wl.bias)


def router_logits(wl: Workload, device="cpu") -> torch.Tensor:
    noise = rng.normal_f32_chunked(wl.key(S_LOGITS), wl.T * wl.E, 1.0, device).view(wl.T, wl.E)
    return noise + expert_bias(wl).to(device)


def gate_prelude_params(wl: Workload, device="cpu"):
    """(norm_weight [H], router_weight [E,H], per_expert_scale [E]) float32."""
    one = torch.tensor(np.float32(1.0))
    norm_w = rng.normal_f32(wl.key(S_WNORM), wl.H, 0.1) + one
    router_w = rng.normal_f32(wl.key(S_WR), wl.E * wl.H, 0.02).view(wl.E, wl.H)
    pe_scale = rng.uniform_f32(wl.key(S_PESCALE), wl.E, 0.5, 1.5)
    return norm_w.to(device), router_w.to(device), pe_scale.to(device)


def expert_weight_f32(wl: Workload, which: str, e: int, device="cpu") -> torch.Tensor:
    """Float32 weight of expert e: which='w13' -> [H, 2I], which='w2' -> [I, H]."""
    if which == "w13":
        K, N, s = wl.H, 2 * wl.I, S_W13
    elif which == "w2":
        K, N, s = wl.I, wl.H, S_W2
    else:
        raise ValueError(which)
    return rng.normal_f32_chunked(wl.key(s, e), K * N, 0.02, device).view(K, N)


def expert_ffn_biases(wl: Workload, device="cpu"):
    """(w13_bias [E', 2I], w2_bias [E', H]) float32, E' = E + shared: N(0, 0.25) on the
    gate/up sums, N(0, 0.1) on the down output (about the spread of the unbiased sums and
    outputs of the workloads above), generated on the CPU."""
    ne = wl.E + wl.shared
    b13 = rng.normal_f32(wl.key(S_B13), ne * 2 * wl.I, 0.25).view(ne, 2 * wl.I)
    b2 = rng.normal_f32(wl.key(S_B2), ne * wl.H, 0.1).view(ne, wl.H)
    return b13.to(device), b2.to(device)


def make_small_inputs(wl: Workload, device="cpu") -> dict:
    """All inputs of a small workload as tensors (weights still float32)."""
    d = {"x": hidden_bf16(wl, device)}
    if wl.prelude:
        d["norm_w"], d["router_w"], d["pe_scale"] = gate_prelude_params(wl, device)
    else:
        d["logits"] = router_logits(wl, device)
    ne = wl.E + wl.shared   # the shared expert's weights come last (index E)
    d["w13"] = torch.stack([expert_weight_f32(wl, "w13", e, device) for e in range(ne)])
    d["w2"] = torch.stack([expert_weight_f32(wl, "w2", e, device) for e in range(ne)])
    return d


def bf16_to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bfloat16 tensor (CPU numpy)."""
    return x.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def describe(wl: Workload) -> str:
    r = f"{wl.scoring}" + (" renorm" if wl.renormalize else "")
    if wl.group_count > 1:
        r += f" G={wl.group_count} k_group={wl.k_group} mode={wl.group_select_mode}"
    if wl.routed_scaling_factor != 1.0:
        r += f" rsf={wl.routed_scaling_factor}"
    if wl.prelude:
        r += " +RMSNorm/router prelude"
    if wl.shared:
        r += " +shared expert"
    if wl.ffn_bias:
        r += " +ffn biases"
    if wl.bias != "none":
        r += f" bias={wl.bias}"
    return f"T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.k} ({r})"

