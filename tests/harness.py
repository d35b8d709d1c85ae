"""Shared plumbing of the parity tests: build a workload's inputs on both sides, run the
oracle for some tokens, run the HIP path, compare.

The two sides meet only through gen (seeded inputs): the oracle quantises its own copy
of the float32 weights; the GPU path quantises with moe_quant_weight_blocks.
"""
from __future__ import annotations

import atexit
import collections
import concurrent.futures as cf
import multiprocessing
import os

import numpy as np
import torch

from gen import workloads as W
from oracle import codec, moe as omoe, routing as orouting

import mixture_experts_fp8_amd as M


def oracle_params(wl: W.Workload) -> orouting.RouteParams:
    return orouting.RouteParams(wl.E, wl.k, wl.scoring, wl.renormalize, wl.group_count, wl.k_group,
                                wl.group_select_mode, wl.routed_scaling_factor)


def device_params(wl: W.Workload):
    return M.route_params(wl.E, wl.k, wl.scoring, wl.renormalize, wl.group_count, wl.k_group,
                          wl.group_select_mode, wl.routed_scaling_factor)


# ---- the oracle over many experts.  Worker processes (spawned: fresh interpreters that never
# touch the GPU) quantise each expert's regenerated float32 weights with the oracle's codec
# and run the oracle's expert FFN on its rows; the quantised weights come back and are kept
# here for later calls that use the same weights (least recently used sets dropped first once
# the kept bytes pass ORACLE_QCACHE_GIB, default 64).  Quantising the weights is most of the
# oracle's time on the full-size prefill shapes, which several tests check under one scheme.
_POOL = None
_QCACHE: "collections.OrderedDict" = collections.OrderedDict()   # weights key -> {expert: quantised}
_QBYTES: dict = {}


def _weights_key(wl: W.Workload, scheme: str):
    """What an expert's quantised weights depend on: the stream keys of gen.workloads
    (seed, workload id, expert index), the shape (H, I) and the quantisation (W8A16 reads
    the FP8 weights)."""
    return (wl.seed, wl.cfg, wl.H, wl.I, "fp8" if scheme == "w8a16" else scheme)


def _qcache_budget() -> int:
    return int(float(os.environ.get("ORACLE_QCACHE_GIB", "64")) * 2**30)


def oracle_workers() -> int:
    return int(os.environ.get("ORACLE_WORKERS", str(max(1, min(16, len(os.sched_getaffinity(0)))))))


def _worker_init():
    # one thread per worker process: the parallelism is across experts
    torch.set_num_threads(1)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ProcessPoolExecutor(oracle_workers(), mp_context=multiprocessing.get_context("spawn"),
                                       initializer=_worker_init)
        atexit.register(_POOL.shutdown, wait=False, cancel_futures=True)
    return _POOL


def _mx_fmt(scheme: str) -> str:
    from oracle import mx as omx
    return omx.FMT_E2M1 if scheme == "w4a8" else omx.FMT_E4M3


def _quantize(wl: W.Workload, scheme: str, e: int):
    """Expert e's weights quantised by the oracle for `scheme` (W8A16 reads the FP8 ones)."""
    from oracle import mx as omx
    w13 = W.expert_weight_f32(wl, "w13", e).numpy()
    w2 = W.expert_weight_f32(wl, "w2", e).numpy()
    if scheme in ("fp8", "w8a16"):
        return omoe.QuantizedExperts(lambda _: (w13, w2)).quantize(e)
    return omx.QuantizedExpertsMX(lambda _: (w13, w2), _mx_fmt(scheme)).quantize(e)


def _expert_job(args):
    """Worker side: one expert's FFN in the oracle (quantising its weights first if needed)."""
    from oracle import mx as omx
    from oracle import w8a16 as ow16
    wl, scheme, e, q, xr, sr, b13, b2, acc_err = args
    fresh = q is None
    if fresh:
        q = _quantize(wl, scheme, e)
    if scheme == "fp8":
        r = omoe.expert_ffn(xr, sr, *q, acc_err, b13, b2)
    elif scheme == "w8a16":
        r = ow16.expert_ffn(xr, *q, b13, b2)
    else:
        r = omx.expert_ffn(xr, sr, *q, _mx_fmt(scheme), acc_err, b13, b2)
    return (q if fresh else None), r


def oracle_ffn_map(wl: W.Workload, scheme: str = "fp8"):
    """An ``ffn_map`` for the oracle's forward functions that runs the per-expert FFNs of
    workload `wl` under quantisation scheme `scheme` ("fp8", "mxfp8", "w4a8", "w8a16") in the
    worker processes."""
    key = _weights_key(wl, scheme)
    if key not in _QCACHE:   # new, or dropped earlier: its bytes start from zero
        _QBYTES[key] = 0
    cache = _QCACHE.setdefault(key, {})
    _QCACHE.move_to_end(key)

    def ffn_map(jobs, acc_err):
        args = [(wl, scheme, e, cache.get(e), xr, sr, b13, b2, acc_err) for e, xr, sr, b13, b2 in jobs]
        out = []
        for (e, *_), (q, r) in zip(jobs, _pool().map(_expert_job, args)):
            if q is not None:
                cache[e] = q
                _QBYTES[key] = _QBYTES.get(key, 0) + sum(int(np.asarray(a).nbytes) for a in q)
            out.append(r)
        _QCACHE.move_to_end(key)
        while sum(_QBYTES.get(k, 0) for k in _QCACHE) > _qcache_budget() and len(_QCACHE) > 1:
            old, _ = _QCACHE.popitem(last=False)
            _QBYTES.pop(old, None)
        return out
    return ffn_map


def item_sample_tokens(ids: np.ndarray, E: int, every: int = 64, tile: int = 128) -> np.ndarray:
    """Tokens whose rows cover every work item of the grouped GEMMs: in the oracle's stable
    permutation of `ids` [T, k] over E experts, the middle row of each `tile`-row tile of each
    expert (every 128-row tile, so both tiles of a 256-row item), plus every `every`-th token."""
    T, k = ids.shape
    counts, offsets, sorted_assign, _ = orouting.permute(ids, E)
    rows = [offsets[e] + m + min(tile // 2, (counts[e] - m) // 2)
            for e in range(E) for m in range(0, int(counts[e]), tile)]
    tok = set((sorted_assign[np.asarray(rows, dtype=np.int64)] // k).tolist()) if rows else set()
    tok |= set(range(0, T, every))
    return np.array(sorted(tok), dtype=np.int64)


def oracle_experts(wl: W.Workload, cache: int = 8) -> omoe.QuantizedExperts:
    def src(e):
        return (W.expert_weight_f32(wl, "w13", e).numpy(), W.expert_weight_f32(wl, "w2", e).numpy())
    return omoe.QuantizedExperts(src, cache=cache)


def oracle_experts_for(wl: W.Workload, experts, workers: int = 8) -> omoe.QuantizedExperts:
    """Oracle experts with the listed ones quantised up front, in a thread pool."""
    import concurrent.futures as cf
    ex = oracle_experts(wl, cache=max(8, len(experts)))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        qs = dict(zip(experts, pool.map(ex.quantize, experts)))
    ex.preload(qs)
    return ex


def device_weights(wl: W.Workload, device="cuda") -> M.PackedWeights:
    """Generate each expert's float32 weights on the GPU, quantise and pack them there."""
    H, I, E = wl.H, wl.I, wl.E + wl.shared   # the shared expert's weights come last
    w13p = torch.empty(E * H * 2 * I, dtype=torch.uint8, device=device)
    w2p = torch.empty(E * I * H, dtype=torch.uint8, device=device)
    w13s = torch.empty(E, H // 128, 2 * I // 128, dtype=torch.uint8, device=device)
    w2s = torch.empty(E, I // 128, H // 128, dtype=torch.uint8, device=device)
    for e in range(E):
        q, s = M.moe_quant_weight_blocks(W.expert_weight_f32(wl, "w13", e, device)[None])
        w13s[e] = s[0]
        w13p[e * H * 2 * I:(e + 1) * H * 2 * I] = M.moe_prepack_weights(q)
        q, s = M.moe_quant_weight_blocks(W.expert_weight_f32(wl, "w2", e, device)[None])
        w2s[e] = s[0]
        w2p[e * I * H:(e + 1) * I * H] = M.moe_prepack_weights(q)
    return _with_biases(wl, M.PackedWeights(E, H, I, w13p, w13s, w2p, w2s), device)


def _with_biases(wl: W.Workload, w: M.PackedWeights, device) -> M.PackedWeights:
    return w.with_biases(*W.expert_ffn_biases(wl, device)) if wl.ffn_bias else w


def oracle_biases(wl: W.Workload):
    """The workload's expert biases as float64 arrays for the oracle, or None."""
    if not wl.ffn_bias:
        return None
    b13, b2 = W.expert_ffn_biases(wl)
    return b13.numpy().astype(np.float64), b2.numpy().astype(np.float64)


def device_weights_mx(wl: W.Workload, quant: int, device="cuda") -> M.PackedWeights:
    """Generate, MX-quantise and pack each expert's weights on the GPU (scheme `quant`)."""
    H, I, E = wl.H, wl.I, wl.E + wl.shared
    wfmt = M.MOE_WFMT_E2M1 if quant == M.MOE_QUANT_W4A8 else M.MOE_WFMT_E4M3
    div = 2 if wfmt == M.MOE_WFMT_E2M1 else 1
    n13, n2 = H * 2 * I // div, I * H // div
    w13p = torch.empty(E * n13, dtype=torch.uint8, device=device)
    w2p = torch.empty(E * n2, dtype=torch.uint8, device=device)
    w13s = torch.empty(E * H * 2 * I // 32, dtype=torch.uint8, device=device)
    w2s = torch.empty(E * I * H // 32, dtype=torch.uint8, device=device)
    for e in range(E):
        q, s = M.moe_quant_weight_mx(W.expert_weight_f32(wl, "w13", e, device)[None], wfmt)
        pq, ps = M.moe_prepack_weights_mx(q, s, wfmt)
        w13p[e * n13:(e + 1) * n13] = pq
        w13s[e * ps.numel():(e + 1) * ps.numel()] = ps
        q, s = M.moe_quant_weight_mx(W.expert_weight_f32(wl, "w2", e, device)[None], wfmt)
        pq, ps = M.moe_prepack_weights_mx(q, s, wfmt)
        w2p[e * n2:(e + 1) * n2] = pq
        w2s[e * ps.numel():(e + 1) * ps.numel()] = ps
    return _with_biases(wl, M.PackedWeights(E, H, I, w13p, w13s, w2p, w2s, quant), device)


def oracle_experts_mx_for(wl: W.Workload, fmt: str, experts, workers: int = 8):
    """MX oracle experts (weights in `fmt`) with the listed ones quantised up front."""
    import concurrent.futures as cf
    from oracle import mx as omx

    def src(e):
        return (W.expert_weight_f32(wl, "w13", e).numpy(), W.expert_weight_f32(wl, "w2", e).numpy())
    ex = omx.QuantizedExpertsMX(src, fmt, cache=max(8, len(experts)))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        qs = dict(zip(experts, pool.map(ex.quantize, experts)))
    ex.preload(qs)
    return ex


def oracle_route(wl: W.Workload, x_f64=None, logits=None):
    """(ids, weights, margin) of the oracle for all tokens."""
    p = oracle_params(wl)
    if wl.prelude:
        nw, rw, pe = W.gate_prelude_params(wl)
        return omoe.route_workload({"x": x_f64}, p, (nw.numpy(), rw.numpy(), pe.numpy(), wl.rms_eps))
    return omoe.route_workload({"logits": logits.numpy() if torch.is_tensor(logits) else logits}, p)


def device_inputs(wl: W.Workload, device="cuda"):
    """x bf16, logits or prelude tensors on the GPU (same bits as the CPU copies)."""
    x = W.hidden_bf16(wl, device)
    if wl.prelude:
        nw, rw, pe = W.gate_prelude_params(wl, device)
        return x, None, M.Prelude(nw, rw, pe, wl.rms_eps)
    return x, W.router_logits(wl, device), None


def rel_errors(y_dev: np.ndarray, y_ref: np.ndarray):
    d = y_dev.astype(np.float64) - y_ref
    fro = np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-300)
    mx = np.abs(d).max() / max(np.abs(y_ref).max(), 1e-300)
    return fro, mx


def assert_output_close(y_dev: np.ndarray, y_ref: np.ndarray, what: str = "", bound=None):
    """The output bar: relative Frobenius error <= 5e-3 and max |err| <= 2e-2 * max |y|,
    against the oracle's unrounded float64 y.

    `bound` (the oracle's "y_bound" / "o_bound", same shape as y) is the near-tie allowance:
    for each output element, the largest change that the re-quantisation decisions lying
    within the oracle's tie tolerance of a rounding midpoint or scale boundary could make if
    the device's float32 h took them the other way (each decision's exact effect, added in
    absolute value).  The max-error bar then applies to the error beyond that allowance,
    element by element; the Frobenius bar always applies to the raw error.  The number of rows
    whose raw error needed the allowance is printed."""
    y_dev = np.asarray(y_dev, dtype=np.float64)
    fro, mx = rel_errors(y_dev, y_ref)
    if bound is None or mx <= 2e-2:
        assert fro <= 5e-3 and mx <= 2e-2, f"{what}: rel fro {fro:.3e}, rel max {mx:.3e}"
        return fro, mx
    scale = np.abs(y_ref).max()
    d = np.abs(y_dev - y_ref)
    excess = np.maximum(d - np.asarray(bound), 0.0)
    mx_ex = excess.max() / scale
    rows = int((d.max(axis=1) / scale > 2e-2).sum())
    print(f"  {what}: {rows} of {len(d)} rows beyond rel max 2e-2 before the near-tie allowance "
          f"(raw rel max {mx:.3e}); beyond the allowance rel max {mx_ex:.3e}", flush=True)
    assert fro <= 5e-3, f"{what}: rel fro {fro:.3e}"
    assert mx_ex <= 2e-2, f"{what}: rel max {mx_ex:.3e} beyond the near-tie allowance"
    return fro, mx_ex


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact values of a bf16 tensor (bf16 -> fp32 is exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def quant_reference(x_bf16_cpu: torch.Tensor):
    return codec.quant_rows_128(W.bf16_to_f64(x_bf16_cpu))
