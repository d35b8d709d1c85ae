"""Thin ctypes binding of libmoe_fp8.so (the C ABI declared in include/moe_fp8.h).

Each function takes torch tensors that already live on the GPU, checks dtypes and
shapes only as far as needed to marshal pointers, and calls the C entry point of the
same name on the current HIP stream.  No step of the MoE computation runs here: if the
library is missing the call fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import dataclasses
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe_fp8.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_SCORING_SOFTMAX, MOE_SCORING_SIGMOID = 0, 1
MOE_ROUTE_IDS_GIVEN = 1
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_FUSED_EXPERT_OUT_BF16 = 1
MOE_FUSED_SHARED_EXPERT = 2
MOE_QUANT_FP8_BLOCK128, MOE_QUANT_MXFP8, MOE_QUANT_W4A8, MOE_QUANT_W8A16 = 0, 1, 2, 3
MOE_WFMT_E4M3, MOE_WFMT_E2M1 = 0, 1
QUANT_SCHEMES = {"fp8": MOE_QUANT_FP8_BLOCK128, "mxfp8": MOE_QUANT_MXFP8, "w4a8": MOE_QUANT_W4A8,
                 "w8a16": MOE_QUANT_W8A16}

EXPORTED = ["moe_route", "moe_route_workspace_size", "moe_quant_act", "moe_quant_weight_blocks",
            "moe_prepack_weights", "moe_grouped_ffn", "moe_ffn_workspace_size", "moe_combine",
            "moe_fused", "moe_workspace_size", "moe_last_error", "moe_quant_act_mx", "moe_quant_weight_mx",
            "moe_prepack_weights_mx", "moe_fused_static"]
MOE_STATIC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class RouteParams(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("group_count", ctypes.c_int32), ("k_group", ctypes.c_int32),
                ("group_select_mode", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float)]


class GatePrelude(ctypes.Structure):
    _fields_ = [("norm_weight", ctypes.c_void_p), ("router_weight", ctypes.c_void_p),
                ("per_expert_scale", ctypes.c_void_p), ("rms_eps", ctypes.c_float)]


class FfnArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("k", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("xq", ctypes.c_void_p), ("xs", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_assign", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("expert_out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p), ("quant", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("debug_h", ctypes.c_void_p), ("debug_hq", ctypes.c_void_p),
                ("debug_hs", ctypes.c_void_p), ("w13_bias", ctypes.c_void_p), ("w2_bias", ctypes.c_void_p)]


class FusedArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("route", RouteParams),
                ("hidden_states", ctypes.c_void_p), ("router_logits", ctypes.c_void_p),
                ("prelude", ctypes.POINTER(GatePrelude)), ("w13", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("flags", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)), ("quant", ctypes.c_int32),
                ("act_q", ctypes.c_void_p), ("act_scales", ctypes.c_void_p), ("w13_bias", ctypes.c_void_p),
                ("w2_bias", ctypes.c_void_p)]


MOE_STAGES = 6
STAGE_NAMES = ["quant_act", "route", "dispatch", "gate_up_gemm", "down_gemm", "combine"]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_fp8.so (built by python -m mixture_experts_fp8_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_fp8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(RouteParams), i32, vp, vp, i32, ctypes.POINTER(GatePrelude), i32,
                                vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route_workspace_size.restype = sz
        L.moe_route_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.moe_quant_act.restype = ctypes.c_int
        L.moe_quant_act.argtypes = [vp, i32, i32, i64, vp, vp, vp]
        L.moe_quant_weight_blocks.restype = ctypes.c_int
        L.moe_quant_weight_blocks.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_prepack_weights.restype = ctypes.c_int
        L.moe_prepack_weights.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_grouped_ffn.restype = ctypes.c_int
        L.moe_grouped_ffn.argtypes = [ctypes.POINTER(FfnArgs)]
        L.moe_ffn_workspace_size.restype = sz
        L.moe_ffn_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp]
        L.moe_fused.restype = ctypes.c_int
        L.moe_fused.argtypes = [ctypes.POINTER(FusedArgs)]
        L.moe_fused_static.restype = ctypes.c_int
        L.moe_fused_static.argtypes = [ctypes.POINTER(FusedArgs)]
        L.moe_workspace_size.restype = sz
        L.moe_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
        L.moe_quant_act_mx.restype = ctypes.c_int
        L.moe_quant_act_mx.argtypes = [vp, i32, i32, i64, vp, vp, vp]
        L.moe_quant_weight_mx.restype = ctypes.c_int
        L.moe_quant_weight_mx.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_prepack_weights_mx.restype = ctypes.c_int
        L.moe_prepack_weights_mx.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
        _lib = L
    return _lib


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, moe_last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A uint8 device buffer whose data pointer is 256-byte aligned."""
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def route_params(num_experts: int, top_k: int, scoring: str = "softmax", renormalize: bool = False,
                 group_count: int = 1, k_group: int = 1, group_select_mode: int = 0,
                 routed_scaling_factor: float = 1.0) -> RouteParams:
    sc = {"softmax": MOE_SCORING_SOFTMAX, "sigmoid": MOE_SCORING_SIGMOID}[scoring]
    return RouteParams(num_experts, top_k, sc, int(bool(renormalize)), group_count, k_group,
                       group_select_mode, routed_scaling_factor)


@dataclass
class Prelude:
    norm_weight: torch.Tensor        # [H] f32
    router_weight: torch.Tensor      # [E, H] f32
    per_expert_scale: Optional[torch.Tensor]   # [E] f32
    rms_eps: float = 1e-6

    def c(self) -> GatePrelude:
        return GatePrelude(_ptr(self.norm_weight), _ptr(self.router_weight), _ptr(self.per_expert_scale),
                           self.rms_eps)


# ---- entry points ---------------------------------------------------------------------

def moe_quant_act(x: torch.Tensor):
    """x bf16 [rows, cols] -> (xq uint8 [rows, cols] E4M3, xs uint8 [rows, cols/128] UE8M0)."""
    _need(x, "x", torch.bfloat16)
    rows, cols = x.shape
    xq = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    xs = torch.empty(rows, max(cols // 128, 1), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quant_act(_ptr(x), rows, cols, cols, _ptr(xq), _ptr(xs), _stream()))
    return xq, xs


def moe_quant_weight_blocks(w: torch.Tensor):
    """w f32 [E, K, N] -> (q uint8 [E, K, N] E4M3, scale uint8 [E, K/128, N/128])."""
    _need(w, "w", torch.float32)
    E, K, N = w.shape
    q = torch.empty(E, K, N, dtype=torch.uint8, device=w.device)
    s = torch.empty(E, max(K // 128, 1), max(N // 128, 1), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quant_weight_blocks(_ptr(w), E, K, N, _ptr(q), _ptr(s), _stream()))
    return q, s


def moe_prepack_weights(w: torch.Tensor) -> torch.Tensor:
    """Logical E4M3 [E, K, N] -> packed layout (same number of bytes, flat)."""
    _need(w, "w", torch.uint8)
    E, K, N = w.shape
    out = torch.empty(E * K * N, dtype=torch.uint8, device=w.device)
    _check(lib().moe_prepack_weights(_ptr(w), E, K, N, _ptr(out), _stream()))
    return out


def moe_quant_act_mx(x: torch.Tensor):
    """x bf16 [rows, cols] -> (xq uint8 [rows, cols] E4M3, xs uint8 [rows, cols/32] UE8M0)."""
    _need(x, "x", torch.bfloat16)
    rows, cols = x.shape
    xq = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    xs = torch.empty(rows, max(cols // 32, 1), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quant_act_mx(_ptr(x), rows, cols, cols, _ptr(xq), _ptr(xs), _stream()))
    return xq, xs


def moe_quant_weight_mx(w: torch.Tensor, wfmt: int):
    """w f32 [E, K, N] -> (codes uint8 [E, K, N] (E4M3) or [E, K, N/2] (E2M1), scale uint8 [E, K/32, N])."""
    _need(w, "w", torch.float32)
    E, K, N = w.shape
    q = torch.empty(E, K, N // 2 if wfmt == MOE_WFMT_E2M1 else N, dtype=torch.uint8, device=w.device)
    s = torch.empty(E, max(K // 32, 1), N, dtype=torch.uint8, device=w.device)
    _check(lib().moe_quant_weight_mx(_ptr(w), E, K, N, wfmt, _ptr(q), _ptr(s), _stream()))
    return q, s


def moe_prepack_weights_mx(q: torch.Tensor, s: torch.Tensor, wfmt: int):
    """Logical MX weights (moe_quant_weight_mx) -> (packed codes, packed scales), flat."""
    _need(q, "q", torch.uint8)
    _need(s, "scale", torch.uint8)
    E, K, N = s.shape[0], q.shape[1], s.shape[2]
    pq = torch.empty(q.numel(), dtype=torch.uint8, device=q.device)
    ps = torch.empty(s.numel(), dtype=torch.uint8, device=q.device)
    _check(lib().moe_prepack_weights_mx(_ptr(q), _ptr(s), E, K, N, wfmt, _ptr(pq), _ptr(ps), _stream()))
    return pq, ps


def moe_route(params: RouteParams, T: int, router_logits: Optional[torch.Tensor] = None,
              hidden_states: Optional[torch.Tensor] = None, prelude: Optional[Prelude] = None,
              topk_ids: Optional[torch.Tensor] = None, topk_weights: Optional[torch.Tensor] = None,
              device=None):
    """Routing + dispatch.  With topk_ids/topk_weights given, only the dispatch runs.

    Returns dict(topk_ids, topk_weights, expert_counts, expert_offsets, sorted_assign, assign_pos)."""
    E, k = params.num_experts, params.top_k
    dev = device or (router_logits.device if router_logits is not None else hidden_states.device)
    flags = 0
    if topk_ids is not None:
        flags = MOE_ROUTE_IDS_GIVEN
        _need(topk_ids, "topk_ids", torch.int32, (T, k))
        _need(topk_weights, "topk_weights", torch.float32, (T, k))
    else:
        topk_ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        topk_weights = torch.empty(T, k, dtype=torch.float32, device=dev)
        if router_logits is not None:
            _need(router_logits, "router_logits", torch.float32, (T, E))
    H = 0
    if hidden_states is not None:
        _need(hidden_states, "hidden_states", torch.bfloat16)
        H = hidden_states.shape[1]
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_assign = torch.empty(T * k, dtype=torch.int32, device=dev)
    assign_pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    with_pre = int(prelude is not None and flags == 0)
    nbytes = lib().moe_route_workspace_size(T, E, k, H, with_pre)
    ws = workspace(max(nbytes, 256), dev)
    pre = ctypes.byref(prelude.c()) if prelude is not None else None
    _check(lib().moe_route(ctypes.byref(params), T, _ptr(router_logits), _ptr(hidden_states), H, pre, flags,
                           _ptr(topk_ids), _ptr(topk_weights), _ptr(counts), _ptr(offsets), _ptr(sorted_assign),
                           _ptr(assign_pos), _ptr(ws), ws.numel(), _stream()))
    return {"topk_ids": topk_ids, "topk_weights": topk_weights, "expert_counts": counts,
            "expert_offsets": offsets, "sorted_assign": sorted_assign, "assign_pos": assign_pos}


@dataclass
class PackedWeights:
    """Expert weights in the packed layout plus their logical UE8M0 block scales."""
    E: int
    H: int
    I: int
    w13: torch.Tensor       # packed [E*H*2I]
    w13_scale: torch.Tensor  # [E, H/128, 2I/128]
    w2: torch.Tensor        # packed [E*I*H]
    w2_scale: torch.Tensor  # [E, I/128, H/128]
    quant: int = MOE_QUANT_FP8_BLOCK128   # MX schemes: packed MX weights and packed scales
    w13_bias: Optional[torch.Tensor] = None   # optional float32 [E, 2I]: gate/up sums, before SwiGLU
    w2_bias: Optional[torch.Tensor] = None    # optional float32 [E, H]: each expert's output

    @staticmethod
    def from_logical(w13q: torch.Tensor, w13s: torch.Tensor, w2q: torch.Tensor, w2s: torch.Tensor) -> "PackedWeights":
        E, H, I2 = w13q.shape
        return PackedWeights(E, H, I2 // 2, moe_prepack_weights(w13q), w13s.contiguous(),
                             moe_prepack_weights(w2q), w2s.contiguous())

    def with_quant(self, quant: int) -> "PackedWeights":
        """The same packed E4M3 weights and 128 x 128 scales under another scheme that reads
        them (MOE_QUANT_W8A16)."""
        if self.quant != MOE_QUANT_FP8_BLOCK128 or quant not in (MOE_QUANT_FP8_BLOCK128, MOE_QUANT_W8A16):
            raise ValueError("only the 128-block E4M3 weights serve both MOE_QUANT_FP8_BLOCK128 and MOE_QUANT_W8A16")
        return dataclasses.replace(self, quant=quant)

    def with_biases(self, w13_bias: Optional[torch.Tensor], w2_bias: Optional[torch.Tensor]) -> "PackedWeights":
        """The same weights with per-expert biases (either may be None)."""
        if w13_bias is not None:
            _need(w13_bias, "w13_bias", torch.float32, (self.E, 2 * self.I))
        if w2_bias is not None:
            _need(w2_bias, "w2_bias", torch.float32, (self.E, self.H))
        return dataclasses.replace(self, w13_bias=w13_bias, w2_bias=w2_bias)


def pack_weights_mx(w13: torch.Tensor, w2: torch.Tensor, quant: int) -> PackedWeights:
    """float32 w13 [E, H, 2I] and w2 [E, I, H] -> packed weights of an MX scheme."""
    wfmt = MOE_WFMT_E2M1 if quant == MOE_QUANT_W4A8 else MOE_WFMT_E4M3
    E, H, I2 = w13.shape
    q13, s13 = moe_quant_weight_mx(w13, wfmt)
    q2, s2 = moe_quant_weight_mx(w2, wfmt)
    p13, ps13 = moe_prepack_weights_mx(q13, s13, wfmt)
    p2, ps2 = moe_prepack_weights_mx(q2, s2, wfmt)
    return PackedWeights(E, H, I2 // 2, p13, ps13, p2, ps2, quant)


def moe_grouped_ffn(xq: Optional[torch.Tensor], xs: Optional[torch.Tensor], routing: dict, w: PackedWeights, k: int,
                    out_dtype=torch.float32, x: Optional[torch.Tensor] = None, debug: bool = False):
    """Both expert GEMMs; returns expert_out [T*k, H] in expert-sorted slot order.
    MOE_QUANT_W8A16 weights take the bf16 hidden states x [T, H] instead of xq / xs.
    debug: also return (expert_out, h, hq, hs), the test outputs of moe_ffn_args: float32 h
    [T*k, I] before re-quantisation, the re-quantised hq [T*k, I] (uint8 E4M3, or bfloat16 for
    W8A16) and hs [T*k, I/128] ([T*k, I/32] for the MX schemes; None for W8A16), sorted order."""
    if w.quant == MOE_QUANT_W8A16:
        if x is None:
            raise ValueError("MOE_QUANT_W8A16 takes the bf16 hidden states x")
        T, H = x.shape
        _need(x, "x", torch.bfloat16, (T, H))
        dev = x.device
    else:
        T, H = xq.shape
        dev = xq.device
    dt = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}[out_dtype]
    out = torch.empty(T * k, H, dtype=out_dtype, device=dev)
    nbytes = lib().moe_ffn_workspace_size(T, H, w.I, w.E, k)
    ws = workspace(max(nbytes, 256), dev)
    dh = dhq = dhs = None
    if debug:
        A = T * k
        dh = torch.empty(A, w.I, dtype=torch.float32, device=dev)
        if w.quant == MOE_QUANT_W8A16:
            dhq = torch.empty(A, w.I, dtype=torch.bfloat16, device=dev)
        else:
            dhq = torch.empty(A, w.I, dtype=torch.uint8, device=dev)
            dhs = torch.empty(A, w.I // (128 if w.quant == MOE_QUANT_FP8_BLOCK128 else 32), dtype=torch.uint8,
                              device=dev)
    a = FfnArgs(T, k, H, w.I, w.E, _ptr(xq), _ptr(xs), _ptr(routing["expert_counts"]),
                _ptr(routing["expert_offsets"]), _ptr(routing["sorted_assign"]), _ptr(w.w13), _ptr(w.w13_scale),
                _ptr(w.w2), _ptr(w.w2_scale), _ptr(out), dt, _ptr(ws), ws.numel(), _stream(), w.quant, _ptr(x),
                _ptr(dh), _ptr(dhq), _ptr(dhs), _ptr(w.w13_bias), _ptr(w.w2_bias))
    _check(lib().moe_grouped_ffn(ctypes.byref(a)))
    return (out, dh, dhq, dhs) if debug else out


def moe_combine(expert_out: torch.Tensor, assign_pos: torch.Tensor, topk_weights: torch.Tensor) -> torch.Tensor:
    """y [T, H] bf16 = sum_j w[t, j] * expert_out[assign_pos[t*k + j]]."""
    T, k = topk_weights.shape
    H = expert_out.shape[1]
    dt = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}[expert_out.dtype]
    y = torch.empty(T, H, dtype=torch.bfloat16, device=expert_out.device)
    _check(lib().moe_combine(_ptr(expert_out), dt, _ptr(assign_pos), _ptr(topk_weights), T, k, H, _ptr(y),
                             _stream()))
    return y


def moe_workspace_size(T: int, H: int, I: int, E: int, k: int, flags: int = 0) -> int:
    return lib().moe_workspace_size(T, H, I, E, k, flags)


class MoeFused:
    """Holds the argument struct and workspace of one fused configuration so that repeated
    calls (benchmark loops, graph capture) only re-issue the C call."""

    def __init__(self, params: RouteParams, T: int, w: PackedWeights, hidden_states: torch.Tensor,
                 router_logits: Optional[torch.Tensor] = None, prelude: Optional[Prelude] = None,
                 expert_out_bf16: bool = False, y: Optional[torch.Tensor] = None,
                 topk_ids: Optional[torch.Tensor] = None, topk_weights: Optional[torch.Tensor] = None,
                 expert_counts: Optional[torch.Tensor] = None, shared_expert: bool = False,
                 act_q: Optional[torch.Tensor] = None, act_scales: Optional[torch.Tensor] = None,
                 static_scratch: bool = False):
        """static_scratch: call moe_fused_static (the library's own scratch array, no
        workspace) instead of moe_fused."""
        H = hidden_states.shape[1]
        _need(hidden_states, "hidden_states", torch.bfloat16, (T, H))
        if router_logits is not None:
            _need(router_logits, "router_logits", torch.float32, (T, params.num_experts))
        if w.E != params.num_experts + int(shared_expert):
            raise ValueError(f"weights hold {w.E} experts; need num_experts + {int(shared_expert)} "
                             f"= {params.num_experts + int(shared_expert)}")
        self.flags = ((MOE_FUSED_EXPERT_OUT_BF16 if expert_out_bf16 else 0) |
                      (MOE_FUSED_SHARED_EXPERT if shared_expert else 0))
        self.y = y if y is not None else torch.empty(T, H, dtype=torch.bfloat16, device=hidden_states.device)
        self.static = static_scratch
        if static_scratch:
            self.ws = None
        else:
            nbytes = lib().moe_workspace_size(T, H, w.I, params.num_experts, params.top_k, self.flags)
            self.ws = workspace(max(nbytes, 256), hidden_states.device)
        if act_q is not None:
            _need(act_q, "act_q", torch.uint8, (T, H))
        if act_scales is not None:
            _need(act_scales, "act_scales", torch.uint8, (T, H // (128 if w.quant == MOE_QUANT_FP8_BLOCK128 else 32)))
        self._keep = (hidden_states, router_logits, prelude, w, topk_ids, topk_weights, expert_counts, act_q,
                      act_scales)
        self._pre = prelude.c() if prelude is not None else None
        self.args = FusedArgs(T, H, w.I, params, _ptr(hidden_states), _ptr(router_logits),
                              ctypes.pointer(self._pre) if self._pre is not None else None,
                              _ptr(w.w13), _ptr(w.w13_scale), _ptr(w.w2), _ptr(w.w2_scale), _ptr(self.y),
                              _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts), self.flags, _ptr(self.ws),
                              0 if self.ws is None else self.ws.numel(), None, None, w.quant, _ptr(act_q),
                              _ptr(act_scales), _ptr(w.w13_bias), _ptr(w.w2_bias))

    def __call__(self, stream: Optional[int] = None, stage_events=None) -> torch.Tensor:
        """stage_events: None or a ctypes array of MOE_STAGES + 1 hipEvent_t handles that the
        library records on the stream at the stage boundaries (null entries are skipped)."""
        self.args.stream = _stream() if stream is None else stream
        if stage_events is None:
            self.args.stage_events = None
        else:
            if len(stage_events) != MOE_STAGES + 1:
                raise ValueError(f"stage_events: need {MOE_STAGES + 1} hipEvent_t slots")
            self._ev_arr = stage_events
            self.args.stage_events = ctypes.cast(stage_events, ctypes.POINTER(ctypes.c_void_p))
        fn = lib().moe_fused_static if self.static else lib().moe_fused
        _check(fn(ctypes.byref(self.args)))
        return self.y


def moe_fused(params: RouteParams, hidden_states: torch.Tensor, w: PackedWeights,
              router_logits: Optional[torch.Tensor] = None, prelude: Optional[Prelude] = None,
              expert_out_bf16: bool = False, return_routing: bool = False, shared_expert: bool = False,
              act_q: Optional[torch.Tensor] = None, act_scales: Optional[torch.Tensor] = None,
              static_scratch: bool = False):
    """The whole step in one C call.  Returns y bf16 [T, H] (and ids, weights, counts).
    shared_expert: w holds num_experts + 1 experts, the last one run on every token and added
    with weight 1 (ids / weights then have top_k + 1 columns, counts num_experts + 1 entries).
    act_q, act_scales: optional uint8 tensors ([T, H] and [T, H/128], or [T, H/32] for the
    micro-scaled schemes) that receive the step's quantised activations.
    static_scratch: run through moe_fused_static (no workspace; the library's scratch array)."""
    T = hidden_states.shape[0]
    dev = hidden_states.device
    ids = weights = counts = None
    sh = int(shared_expert)
    if return_routing:
        ids = torch.empty(T, params.top_k + sh, dtype=torch.int32, device=dev)
        weights = torch.empty(T, params.top_k + sh, dtype=torch.float32, device=dev)
        counts = torch.empty(params.num_experts + sh, dtype=torch.int32, device=dev)
    f = MoeFused(params, T, w, hidden_states, router_logits, prelude, expert_out_bf16, None, ids, weights, counts,
                 shared_expert, act_q, act_scales, static_scratch)
    y = f()
    return (y, ids, weights, counts) if return_routing else y


def moe_fused_static(params: RouteParams, hidden_states: torch.Tensor, w: PackedWeights,
                     router_logits: Optional[torch.Tensor] = None, prelude: Optional[Prelude] = None,
                     expert_out_bf16: bool = False, return_routing: bool = False, shared_expert: bool = False,
                     act_q: Optional[torch.Tensor] = None, act_scales: Optional[torch.Tensor] = None):
    """moe_fused through the C entry point moe_fused_static: no workspace, the library's own
    scratch array (MOE_STATIC_SCRATCH_BYTES per GPU).  Same arguments and results as
    moe_fused; steps that need more scratch raise MoeError (MOE_ERR_UNSUPPORTED)."""
    return moe_fused(params, hidden_states, w, router_logits, prelude, expert_out_bf16, return_routing,
                     shared_expert, act_q, act_scales, static_scratch=True)
