#!/usr/bin/env python3
"""Benchmark of the routed FP8 MoE expert step on one MI355X.

    python bench.py [--config 5] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one moe_fused call: gate prelude / routing, dispatch, activation quantisation,
gate+up FP8 GEMM with SwiGLU + requantisation, down FP8 GEMM and the weighted combine,
over one batch of seeded synthetic tokens whose inputs already sit in HBM.  Steps rotate
through LAYERS copies of the expert weights, as consecutive MoE layers of a model would,
so the 256 MB Infinity Cache cannot hand a step the weights the previous step read.

Prints one JSON line: throughput (tokens/s) over exactly K timed steps, FP8 TFLOP/s, a
roofline entry for the dominant kernel (algorithmic bytes or flops per launch divided by
its average duration, measured with HIP events recorded on the launch stream), and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + FP8 TFLOP/s; % of FP8-MFMA or HBM roofline, 1 MI355X"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 matrix, TFLOP/s
LAYERS = 4
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["mixture_experts_fp8_amd/csrc/k_ffn.hip", "mixture_experts_fp8_amd/csrc/k_ffn_rb.hip",
                  "mixture_experts_fp8_amd/csrc/k_mx.hip", "mixture_experts_fp8_amd/csrc/moe_common.h",
                  "mixture_experts_fp8_amd/csrc/work_items.h", "mixture_experts_fp8_amd/csrc/k_w16.hip"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id 1..5 (default 5: the large Zipf-skewed prefill, the largest that fits one GPU "
                         "by tokens and flops; 2: the Gemma-4-like decode); 6: one 8-GPU expert-parallel shard of 4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared", action="store_true",
                    help="add one shared expert (same H, I) run on every token in the same launches")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="0: the workload's own default sample")
    ap.add_argument("--expert-out", default="auto", choices=["auto", "fp32", "bf16"],
                    help="dtype of the per-assignment expert outputs between the down GEMM and the combine; auto: "
                         "bf16 when they would take 16 MB or more as fp32 (the prefill shapes), else fp32")
    ap.add_argument("--expert-out-bf16", action="store_true", help="same as --expert-out bf16")
    ap.add_argument("--quant", default="fp8", choices=["fp8", "mxfp8", "w4a8", "w8a16"],
                    help="fp8: E4M3 with 128-element scales (default); mxfp8: 32-element scales; "
                         "w4a8: E2M1 weights with MXFP8 activations; w8a16: the fp8 weights with bf16 activations")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (a known-size kernel for HBM counter calibration)")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (created eagerly) for the library's stage boundaries; only
    the slots listed in `only` (default: all) get an event, the others stay null."""

    def __init__(self, n: int, only=None):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = (ctypes.c_void_p * n)()
        for i in (range(n) if only is None else only):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.ev[i] = h.value

    def elapsed_s(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(self.ev[i]), self.ct.c_void_p(self.ev[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value * 1e-3

    def destroy(self):
        for h in self.ev:
            if h:
                self.hip.hipEventDestroy(self.ct.c_void_p(h))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# bytes per weight element, bytes per activation element, activation elements per scale byte
# (0: no activation scales) and weight elements per scale byte
SCHEME_BYTES = {"fp8": (1.0, 1, 128, 128 * 128), "mxfp8": (1.0, 1, 32, 32), "w4a8": (0.5, 1, 32, 32),
                "w8a16": (1.0, 2, 0, 128 * 128)}
# peak of the matrix-core type each scheme contracts in (TFLOP/s, dense)
SCHEME_PEAK = {"fp8": 5000.0, "mxfp8": 5000.0, "w4a8": 5000.0, "w8a16": 2500.0}


def act_bytes(n: int, ab: int, ga: int) -> float:
    """Bytes of n activation elements and their scales."""
    return n * ab + (n / ga if ga else 0)


def stage_bytes_flops(wl, counts: np.ndarray, eo_bytes: int, quant: str = "fp8"):
    """Algorithmic HBM bytes and FP8 flops per launch of the two GEMM stages.

    gate+up: every active expert's w13 once (H*2I weight elements at wb bytes each plus
    one scale byte per weight group), each token's activation row once (H elements at ab
    bytes plus H/ga scale bytes), each assignment's h row written once (I elements, I/ga
    scales).  down: every active expert's w2 once, each h row read once, each assignment's
    output row written once (H * eo_bytes).  wb = 1 for E4M3 weights and 0.5 for E2M1; ab = 1
    for E4M3 activations and 2 for bf16 (W8A16, no activation scales); groups of ga = 128 (or
    32) activations and gw = 128 x 128 (or 32) weights per scale byte.
    """
    wb, ab, ga, gw = SCHEME_BYTES[quant]
    H, I, T, A = wl.H, wl.I, wl.T, wl.T * (wl.k + wl.shared)
    n_act = int((counts > 0).sum())
    g1_bytes = n_act * (H * 2 * I * wb + H * 2 * I / gw) + act_bytes(T * H, ab, ga) + act_bytes(A * I, ab, ga)
    g2_bytes = n_act * (I * H * wb + I * H / gw) + act_bytes(A * I, ab, ga) + A * H * eo_bytes
    g1_flops = 4.0 * A * H * I
    g2_flops = 2.0 * A * H * I
    return {"gate_up_gemm": (int(g1_bytes), g1_flops), "down_gemm": (int(g2_bytes), g2_flops)}, n_act


def step_algorithmic_bytes(wl, n_act: int, quant: str = "fp8") -> int:
    """Minimum traffic of a whole step: active experts' weights and scales, x, logits
    (or the prelude tensors), y, ids and weights."""
    wb, _, _, gw = SCHEME_BYTES[quant]
    H, I, T, E, k = wl.H, wl.I, wl.T, wl.E, wl.k
    b = int(n_act * (3 * H * I * wb + 3 * H * I / gw))
    b += 2 * T * H + 2 * T * H + 8 * T * (k + wl.shared)
    b += 4 * E * H + 4 * H + 4 * E if wl.prelude else 4 * T * E
    return b


def roofline_entry(name, dur_s, nbytes, flops, traffic, peak_tflops=PEAK_FP8_TFLOPS):
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (peak_tflops * 1e12)
    if t_hbm >= t_mfma:
        ach = nbytes / dur_s / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "algorithmic_bytes": int(nbytes),
                "avg_us": round(dur_s * 1e6, 2)}
    ach = flops / dur_s / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": peak_tflops, "unit": "TFLOP/s",
            "frac": round(ach / peak_tflops, 4), "traffic": traffic, "algorithmic_flops": flops,
            "avg_us": round(dur_s * 1e6, 2)}


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source; otherwise None."""
    p = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, sample_tokens: int, quant: str = "fp8", min_seconds: float = 10.0):
    """The oracle as it stands, timed on the host on a bounded sample of the workload's
    tokens (weights quantised by the oracle beforehand, untimed)."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from gen import workloads as W
    from oracle import moe as omoe
    from oracle import mx as omx
    from oracle import routing as orouting
    from oracle import w8a16 as ow16

    x = W.hidden_bf16(wl)
    xf = W.bf16_to_f64(x)
    p = orouting.RouteParams(wl.E, wl.k, wl.scoring, wl.renormalize, wl.group_count, wl.k_group,
                             wl.group_select_mode, wl.routed_scaling_factor)
    if wl.prelude:
        nw, rw, pe = W.gate_prelude_params(wl)
        pre = (nw.numpy(), rw.numpy(), pe.numpy(), wl.rms_eps)
        inputs = {"x": xf}
    else:
        pre = None
        inputs = {"logits": W.router_logits(wl).numpy()}
    n = min(sample_tokens, wl.T)
    tokens = np.linspace(0, wl.T - 1, n).astype(np.int64)
    ids, _, _ = omoe.route_workload(inputs, p, pre)
    experts = sorted(set(int(e) for e in ids[tokens].reshape(-1)) | ({wl.E} if wl.shared else set()))

    def src(e):
        return (W.expert_weight_f32(wl, "w13", e).numpy(), W.expert_weight_f32(wl, "w2", e).numpy())

    if quant in ("fp8", "w8a16"):
        ex = omoe.QuantizedExperts(src, cache=len(experts))
        fwd = omoe.forward if quant == "fp8" else ow16.forward
    else:
        fmt = omx.FMT_E2M1 if quant == "w4a8" else omx.FMT_E4M3
        ex, fwd = omx.QuantizedExpertsMX(src, fmt, cache=len(experts)), omx.forward
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:   # input preparation, untimed
        ex.preload(dict(zip(experts, pool.map(ex.quantize, experts))))
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:   # whole passes over the sample until at least min_seconds have gone by
            ids, w, _ = omoe.route_workload(inputs, p, pre)    # routing of the whole batch
            if wl.shared:   # the shared expert as slot k with weight 1 (oracle.moe.forward_shared)
                ids = np.concatenate([ids, np.full((len(ids), 1), wl.E, dtype=ids.dtype)], axis=1)
                w = np.concatenate([np.asarray(w, dtype=np.float64), np.ones((len(w), 1))], axis=1)
            out = fwd(xf, ids, w, ex, tokens=tokens)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    assert out["y"].shape == (n, wl.H)
    return {"value": round(n * reps / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {wl.T} tokens (evenly spaced), all of their {len(experts)} experts; routing "
                      f"of the full batch included; {reps} passes, {dt:.1f} s on one host thread"}


def expert_out_dtype(wl, choice):
    """dtype of the per-assignment expert outputs: the choice, or for "auto" bf16 once they would
    take 16 MB or more as float32 (the prefill shapes, where writing and re-reading them is a
    visible share of the step's traffic) and float32 below (the decode shapes, where it is free)."""
    if choice != "auto":
        return choice
    return "bf16" if wl.T * (wl.k + wl.shared) * wl.H * 4 >= (16 << 20) else "fp32"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the expert step runs on one GPU with every expert local; --gpus {args.gpus} is "
              f"not supported (there is no expert-parallel exchange across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_fp8_amd as M
    from gen import workloads as W
    from mixture_experts_fp8_amd import binding as B

    wl = W.CONFIGS[args.config]
    if args.shared:
        wl = wl.replace(shared=1)
    if args.expert_out_bf16:
        args.expert_out = "bf16"
    args.expert_out_bf16 = expert_out_dtype(wl, args.expert_out) == "bf16"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: {W.describe(wl)}", file=sys.stderr, flush=True)

    # ---- inputs, resident in HBM before timing
    x = W.hidden_bf16(wl, dev)
    logits, pre = None, None
    if wl.prelude:
        nw, rw, pe = W.gate_prelude_params(wl, dev)
        pre = M.Prelude(nw, rw, pe, wl.rms_eps)
    else:
        logits = W.router_logits(wl, dev)
    H, I, E = wl.H, wl.I, wl.E + wl.shared   # the shared expert's weights come last
    quant = M.QUANT_SCHEMES[args.quant]
    if quant in (M.MOE_QUANT_FP8_BLOCK128, M.MOE_QUANT_W8A16):   # W8A16 reads the same packed weights
        w13p = torch.empty(E * H * 2 * I, dtype=torch.uint8, device=dev)
        w2p = torch.empty(E * I * H, dtype=torch.uint8, device=dev)
        w13s = torch.empty(E, H // 128, 2 * I // 128, dtype=torch.uint8, device=dev)
        w2s = torch.empty(E, I // 128, H // 128, dtype=torch.uint8, device=dev)
        for e in range(E):
            q, s = M.moe_quant_weight_blocks(W.expert_weight_f32(wl, "w13", e, dev)[None])
            w13s[e] = s[0]
            w13p[e * H * 2 * I:(e + 1) * H * 2 * I] = M.moe_prepack_weights(q)
            q, s = M.moe_quant_weight_blocks(W.expert_weight_f32(wl, "w2", e, dev)[None])
            w2s[e] = s[0]
            w2p[e * I * H:(e + 1) * I * H] = M.moe_prepack_weights(q)
    else:
        wfmt = M.MOE_WFMT_E2M1 if quant == M.MOE_QUANT_W4A8 else M.MOE_WFMT_E4M3
        n13, n2 = H * 2 * I // (2 if wfmt else 1), I * H // (2 if wfmt else 1)
        w13p = torch.empty(E * n13, dtype=torch.uint8, device=dev)
        w2p = torch.empty(E * n2, dtype=torch.uint8, device=dev)
        w13s = torch.empty(E * H * 2 * I // 32, dtype=torch.uint8, device=dev)
        w2s = torch.empty(E * I * H // 32, dtype=torch.uint8, device=dev)
        for e in range(E):
            q, s = M.moe_quant_weight_mx(W.expert_weight_f32(wl, "w13", e, dev)[None], wfmt)
            pq, ps = M.moe_prepack_weights_mx(q, s, wfmt)
            w13p[e * n13:(e + 1) * n13], w13s[e * ps.numel():(e + 1) * ps.numel()] = pq, ps
            q, s = M.moe_quant_weight_mx(W.expert_weight_f32(wl, "w2", e, dev)[None], wfmt)
            pq, ps = M.moe_prepack_weights_mx(q, s, wfmt)
            w2p[e * n2:(e + 1) * n2], w2s[e * ps.numel():(e + 1) * ps.numel()] = pq, ps
    layers = [M.PackedWeights(E, H, I, w13p, w13s, w2p, w2s, quant)]
    for _ in range(LAYERS - 1):
        layers.append(M.PackedWeights(E, H, I, w13p.clone(), w13s.clone(), w2p.clone(), w2s.clone(), quant))
    params = M.route_params(wl.E, wl.k, wl.scoring, wl.renormalize, wl.group_count, wl.k_group,
                            wl.group_select_mode, wl.routed_scaling_factor)
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    y = torch.empty(wl.T, H, dtype=torch.bfloat16, device=dev)
    calls = [M.MoeFused(params, wl.T, lw, x, logits, pre, args.expert_out_bf16, y=y, expert_counts=counts,
                        shared_expert=bool(wl.shared)) for lw in layers]
    torch.cuda.synchronize()

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- warmup, then exactly K timed steps
    for i in range(args.warmup):
        calls[i % LAYERS]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        calls[i % LAYERS]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = wl.T * args.steps / elapsed

    # ---- per-stage durations from HIP events recorded on the launch stream
    nst = B.MOE_STAGES
    evs = [HipEvents(nst + 1) for _ in range(args.steps)]
    for i in range(args.steps):
        calls[i % LAYERS](stage_events=evs[i].ev)
    torch.cuda.synchronize()
    stage_s = np.zeros(nst)
    for i in range(args.steps):
        for s in range(nst):
            stage_s[s] += evs[i].elapsed_s(s, s + 1)
        evs[i].destroy()
    stage_s /= args.steps
    # the activation quantisation runs inside the routing kernel: its own stage is empty
    names = dict(zip(B.STAGE_NAMES, B.STAGE_NAMES))
    names["route"] = "route_and_quant_act"
    stages = {names[B.STAGE_NAMES[s]]: round(stage_s[s] * 1e6, 2) for s in range(nst) if B.STAGE_NAMES[s] != "quant_act"}

    cnt = counts.cpu().numpy()
    eo_bytes = 2 if args.expert_out_bf16 else 4
    per_stage, n_act = stage_bytes_flops(wl, cnt, eo_bytes, args.quant)
    dom = max(per_stage, key=lambda n: stage_s[B.STAGE_NAMES.index(n)])
    other = [n for n in per_stage if n != dom][0]

    def kernel_time(name):
        """Average duration of one stage's kernel, from only the two events around it."""
        i = B.STAGE_NAMES.index(name)
        ev2 = [HipEvents(nst + 1, only=(i, i + 1)) for _ in range(args.steps)]
        for k in range(args.steps):
            calls[k % LAYERS](stage_events=ev2[k].ev)
        torch.cuda.synchronize()
        t = sum(e.elapsed_s(i, i + 1) for e in ev2) / args.steps
        for e in ev2:
            e.destroy()
        return t

    tname = (wl.name + ("_shared" if wl.shared else "")) + ("" if args.quant == "fp8" else f"_{args.quant}")
    peak = SCHEME_PEAK[args.quant]
    roof = roofline_entry(dom, kernel_time(dom), *per_stage[dom], load_traffic(tname, dom), peak)
    roof_other = roofline_entry(other, kernel_time(other), *per_stage[other], load_traffic(tname, other), peak)

    step_bytes = step_algorithmic_bytes(wl, n_act, args.quant)
    total_flops = wl.flops()
    step_s = elapsed / args.steps
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3 (fp32 accumulate)", "mxfp8": "mxfp8_e4m3 (fp32 accumulate)",
                  "w4a8": "fp4_e2m1 weights x fp8_e4m3 activations (fp32 accumulate)",
                  "w8a16": "fp8_e4m3 weights decoded to bf16 x bf16 activations (fp32 accumulate)"}[args.quant],
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {W.describe(wl)}", "tokens_per_step": wl.T,
                   "weight_copies_rotated": LAYERS, "expert_out": "bf16" if args.expert_out_bf16 else "fp32",
                   "quant": {"fp8": "E4M3, UE8M0 per (row,128) / 128x128 block", "mxfp8": "E4M3, UE8M0 per 32",
                             "w4a8": "E2M1 weights + E4M3 activations, UE8M0 per 32",
                             "w8a16": "E4M3 weights, UE8M0 per 128x128 block; bf16 activations"}[args.quant],
                   "active_experts": n_act},
        "fp8_tflops": round(total_flops / step_s / 1e12, 3),
        "step_hbm_frac": round(step_bytes / step_s / 1e9 / PEAK_HBM_GBS, 4),
        "step_mfma_frac": round(total_flops / step_s / 1e12 / SCHEME_PEAK[args.quant], 4),
        "step_algorithmic_bytes": int(step_bytes),
        "stages_us": stages,
        "roofline": roof,
        "roofline_other_gemm": roof_other,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        n = args.cpu_sample_tokens or {1: 64, 2: 32, 3: 64, 4: 2, 5: 8, 6: 2}[args.config]
        out["cpu_baseline"] = cpu_baseline(wl, n, args.quant)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
