"""Guard bands around every buffer the library writes.

Each output buffer (and the workspace) sits inside one device arena between bands of canary
bytes; after the call every byte outside the buffers must still hold the canary, and the
buffers must hold exactly what the same call writes into ordinary allocations.  This catches
a kernel that writes past a tile, a row or the workspace size it reported, which the parity
tests (reading only the valid part of each output) would not see.  Shapes cover every kernel
family: 16-row decode tiles with the gate prelude, 128-row tiles (persistent gate/up and
down), 256-row pairs, the MX schemes on 16-, 128- and 256-row tiles, W8A16, the shared
expert, biases and both expert-output dtypes.
"""
import ctypes

import numpy as np
import pytest
import torch

from gen import workloads as W

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
B = M.binding
DEV = "cuda"
CANARY = 0xA5
BAND = 4096


class Arena:
    """Buffers of the given byte sizes, 256-byte aligned, each between canary bands."""

    def __init__(self, sizes):
        self.offs, o = [], BAND
        for n in sizes:
            self.offs.append(o)
            o = (o + n + BAND + 255) // 256 * 256
        self.sizes = list(sizes)
        raw = torch.full((o + 256,), CANARY, dtype=torch.uint8, device=DEV)
        shift = (-raw.data_ptr()) % 256
        self.buf = raw[shift:shift + o]
        self._raw = raw

    def ptr(self, i):
        return self.buf.data_ptr() + self.offs[i]

    def view(self, i, dtype, shape):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        assert n <= self.sizes[i]
        return self.buf[self.offs[i]:self.offs[i] + n].view(dtype).view(*shape)

    def assert_guards(self, what):
        torch.cuda.synchronize()
        host = self.buf.cpu().numpy()
        mask = np.ones(len(host), dtype=bool)
        for o, n in zip(self.offs, self.sizes):
            mask[o:o + n] = False
        bad = np.nonzero((host != CANARY) & mask)[0]
        assert len(bad) == 0, f"{what}: {len(bad)} guard bytes overwritten, first at arena offset {bad[:8]}"


def _weights(wl, scheme):
    if scheme == "fp8":
        return HN.device_weights(wl)
    if scheme == "w8a16":
        return HN.device_weights(wl).with_quant(M.MOE_QUANT_W8A16)
    return HN.device_weights_mx(wl, M.QUANT_SCHEMES[scheme])


CASES = {
    "decode_prelude": (W.Workload(180, "g_dec", T=24, H=512, I=256, E=16, k=4, prelude=True), "fp8", False),
    "tiles128": (W.Workload(181, "g_t128", T=600, H=256, I=384, E=32, k=2, bias="normal1.5"), "fp8", False),
    "pairs_bf16": (W.Workload(182, "g_p2", T=1500, H=512, I=256, E=8, k=4), "fp8", True),
    "plain_H384": (W.Workload(183, "g_h384", T=600, H=384, I=256, E=8, k=3), "fp8", False),
    "mx_tiles128": (W.Workload(184, "g_mxt", T=300, H=512, I=384, E=16, k=4), "mxfp8", False),
    "w4a8_pairs": (W.Workload(185, "g_w4p", T=600, H=512, I=384, E=8, k=3), "w4a8", True),
    "mx_decode": (W.Workload(186, "g_mxd", T=30, H=384, I=256, E=16, k=2), "w4a8", False),
    "w8a16": (W.Workload(187, "g_w16", T=40, H=256, I=384, E=8, k=3), "w8a16", False),
    "shared_bias": (W.Workload(188, "g_shb", T=200, H=256, I=256, E=8, k=2, shared=1, ffn_bias=True), "fp8", True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_writes_only_its_outputs(name):
    wl, scheme, eo_bf16 = CASES[name]
    print("guards fused", name, scheme, W.describe(wl), flush=True)
    x, logits, pre = HN.device_inputs(wl)
    w = _weights(wl, scheme)
    p = HN.device_params(wl)
    T, H, sh = wl.T, wl.H, wl.shared
    kk, EE = wl.k + sh, wl.E + sh
    quant_act = scheme != "w8a16"
    gs = H // (128 if scheme == "fp8" else 32)
    flags = (M.MOE_FUSED_EXPERT_OUT_BF16 if eo_bf16 else 0) | (M.MOE_FUSED_SHARED_EXPERT if sh else 0)
    ws_bytes = M.moe_workspace_size(T, H, wl.I, wl.E, wl.k, flags)
    sizes = [T * H * 2, T * kk * 4, T * kk * 4, EE * 4, ws_bytes]
    if quant_act:
        sizes += [T * H, T * gs]
    ar = Arena(sizes)
    y = ar.view(0, torch.bfloat16, (T, H))
    ids = ar.view(1, torch.int32, (T, kk))
    wts = ar.view(2, torch.float32, (T, kk))
    cnt = ar.view(3, torch.int32, (EE,))
    aq = ar.view(5, torch.uint8, (T, H)) if quant_act else None
    asc = ar.view(6, torch.uint8, (T, gs)) if quant_act else None
    f = B.MoeFused(p, T, w, x, logits, pre, eo_bf16, y, ids, wts, cnt, bool(sh), aq, asc)
    f.args.workspace = ar.ptr(4)
    f.args.workspace_bytes = ws_bytes
    f()
    ar.assert_guards(f"moe_fused {name}")
    # the same call into ordinary buffers
    ref = B.moe_fused(p, x, w, router_logits=logits, prelude=pre, expert_out_bf16=eo_bf16, return_routing=True,
                      shared_expert=bool(sh))
    torch.cuda.synchronize()
    assert torch.equal(y, ref[0]) and torch.equal(ids, ref[1]) and torch.equal(wts, ref[2])
    assert torch.equal(cnt, ref[3])


@pytest.mark.parametrize("name", ["tiles128", "pairs_bf16", "mx_tiles128", "w8a16", "decode_prelude"])
def test_route_ffn_combine_write_only_their_outputs(name):
    wl, scheme, eo_bf16 = CASES[name]
    print("guards separate", name, scheme, W.describe(wl), flush=True)
    x, logits, pre = HN.device_inputs(wl)
    w = _weights(wl, scheme)
    p = HN.device_params(wl)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    A = T * k
    L = M.lib()
    # routing (with the prelude where the workload has one)
    rws = L.moe_route_workspace_size(T, E, k, H if pre else 0, 1 if pre else 0)
    ar = Arena([A * 4, A * 4, E * 4, (E + 1) * 4, A * 4, A * 4, rws])
    outs = [ar.ptr(i) for i in range(6)]
    pre_c = ctypes.byref(pre.c()) if pre else None
    B._check(L.moe_route(ctypes.byref(p), T, B._ptr(logits), B._ptr(x) if pre else None, H if pre else 0, pre_c, 0,
                         *outs, ar.ptr(6), rws, B._stream()))
    ar.assert_guards(f"moe_route {name}")
    r = {"topk_ids": ar.view(0, torch.int32, (T, k)), "topk_weights": ar.view(1, torch.float32, (T, k)),
         "expert_counts": ar.view(2, torch.int32, (E,)), "expert_offsets": ar.view(3, torch.int32, (E + 1,)),
         "sorted_assign": ar.view(4, torch.int32, (A,)), "assign_pos": ar.view(5, torch.int32, (A,))}
    ref_r = M.moe_route(p, T, router_logits=logits, hidden_states=x if pre else None, prelude=pre)
    for key in r:
        assert torch.equal(r[key], ref_r[key]), key
    # activation quantisation
    xq = xs = None
    if scheme != "w8a16":
        gs = H // (128 if scheme == "fp8" else 32)
        aq = Arena([T * H, T * gs])
        fn = L.moe_quant_act if scheme == "fp8" else L.moe_quant_act_mx
        B._check(fn(B._ptr(x), T, H, H, aq.ptr(0), aq.ptr(1), B._stream()))
        aq.assert_guards(f"quant_act {name}")
        xq, xs = aq.view(0, torch.uint8, (T, H)), aq.view(1, torch.uint8, (T, gs))
    # grouped FFN with its test outputs
    fws = L.moe_ffn_workspace_size(T, H, I, E, k)
    eo_el = 2 if eo_bf16 else 4
    hq_el = 2 if scheme == "w8a16" else 1
    nhs = 0 if scheme == "w8a16" else A * (I // (128 if scheme == "fp8" else 32))
    af = Arena([A * H * eo_el, fws, A * I * 4, A * I * hq_el, max(nhs, 1)])
    args = B.FfnArgs(T, k, H, I, E, B._ptr(xq), B._ptr(xs), B._ptr(r["expert_counts"]), B._ptr(r["expert_offsets"]),
                     B._ptr(r["sorted_assign"]), B._ptr(w.w13), B._ptr(w.w13_scale), B._ptr(w.w2), B._ptr(w.w2_scale),
                     af.ptr(0), B.MOE_DTYPE_BF16 if eo_bf16 else B.MOE_DTYPE_F32, af.ptr(1), fws, B._stream(), w.quant,
                     B._ptr(x) if scheme == "w8a16" else None, af.ptr(2), af.ptr(3), af.ptr(4) if nhs else None,
                     B._ptr(w.w13_bias), B._ptr(w.w2_bias))
    B._check(L.moe_grouped_ffn(ctypes.byref(args)))
    af.assert_guards(f"moe_grouped_ffn {name}")
    eo_dt = torch.bfloat16 if eo_bf16 else torch.float32
    eo = af.view(0, eo_dt, (A, H))
    ref_eo = M.moe_grouped_ffn(xq, xs, ref_r, w, k, out_dtype=eo_dt, x=x if scheme == "w8a16" else None)
    torch.cuda.synchronize()
    assert torch.equal(eo, ref_eo)
    # combine
    ac = Arena([T * H * 2])
    B._check(L.moe_combine(B._ptr(eo), B.MOE_DTYPE_BF16 if eo_bf16 else B.MOE_DTYPE_F32, B._ptr(r["assign_pos"]),
                           B._ptr(r["topk_weights"]), T, k, H, ac.ptr(0), B._stream()))
    ac.assert_guards(f"moe_combine {name}")
    assert torch.equal(ac.view(0, torch.bfloat16, (T, H)), M.moe_combine(eo, r["assign_pos"], r["topk_weights"]))
