"""moe_fused_static, the entry point that allocates nothing (its temporaries live in the
library's own scratch array): through the C ABI it gives the bits of moe_fused, call after
call on one GPU, also when a smaller step follows a larger one in the same array."""
import ctypes

import numpy as np
import pytest
import torch

from gen import workloads as W

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
from mixture_experts_fp8_amd import binding as B  # noqa: E402


def _pair(wl, **kw):
    x, logits, pre = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    p = HN.device_params(wl)
    y_ref, ids_ref, wts_ref, cnt_ref = M.moe_fused(p, x, w, router_logits=logits, prelude=pre, return_routing=True,
                                                   **kw)
    y, ids, wts, cnt = M.moe_fused_static(p, x, w, router_logits=logits, prelude=pre, return_routing=True, **kw)
    torch.cuda.synchronize()
    return (y, ids, wts, cnt), (y_ref, ids_ref, wts_ref, cnt_ref)


def test_static_scratch_matches_moe_fused_twice_second_smaller():
    # a decode step (prelude, 16-row tiles), then a smaller step (fewer tokens, 128-row tiles
    # with pairs) in the same array: each equals moe_fused bit for bit
    first = W.CONFIGS[2]                                                          # T = 32
    second = W.Workload(180, "static_small", T=20, H=256, I=256, E=2, k=2)        # smaller workspace
    assert B.lib().moe_workspace_size(second.T, second.H, second.I, second.E, second.k, 0) < \
        B.lib().moe_workspace_size(first.T, first.H, first.I, first.E, first.k, 0)
    for wl in (first, second):
        got, ref = _pair(wl)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), wl.name
    # and a third call repeating the first: nothing left in the array changes the result
    got, ref = _pair(first)
    assert torch.equal(got[0], ref[0])
    # the shared expert and bf16 expert outputs through the same array
    got, ref = _pair(W.Workload(181, "static_sh", T=40, H=256, I=256, E=6, k=2, shared=1), shared_expert=True,
                     expert_out_bf16=True)
    assert torch.equal(got[0], ref[0])


def test_static_scratch_rejects_large_steps_and_a_workspace():
    wl = W.CONFIGS[3]      # the unaligned shape needs more scratch than the library holds
    need = B.lib().moe_workspace_size(wl.T, wl.H, wl.I, wl.E, wl.k, 0)
    assert need > B.MOE_STATIC_SCRATCH_BYTES
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights(wl)
    with pytest.raises(B.MoeError) as ei:
        M.moe_fused_static(HN.device_params(wl), x, w, router_logits=logits)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED and "scratch" in str(ei.value)
    # a workspace given to the static entry point is an error, not silently ignored
    small = W.Workload(182, "static_ws", T=8, H=128, I=128, E=2, k=1)
    xs, ls, _ = HN.device_inputs(small)
    ww = HN.device_weights(small)
    y = torch.empty(small.T, small.H, dtype=torch.bfloat16, device=xs.device)
    ws = B.workspace(1 << 20, xs.device)
    a = B.FusedArgs(small.T, small.H, small.I, HN.device_params(small), xs.data_ptr(), ls.data_ptr(), None,
                    ww.w13.data_ptr(), ww.w13_scale.data_ptr(), ww.w2.data_ptr(), ww.w2_scale.data_ptr(), y.data_ptr(),
                    None, None, None, 0, ws.data_ptr(), ws.numel(), None, None, 0, None, None)
    assert B.lib().moe_fused_static(ctypes.byref(a)) == B.MOE_ERR_INVALID
    assert "workspace must be NULL" in M.moe_last_error()
