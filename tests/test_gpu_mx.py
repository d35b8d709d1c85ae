"""GPU parity of the micro-scaled schemes (MXFP8, W4A8) against the oracle (oracle.mx).

Quantisers and the pre-pack are compared bit for bit; the expert step end to end with the
output bar of the 128-group path (relative Frobenius <= 5e-3, max |err| <= 2e-2 max |y|).
"""

import numpy as np
import pytest
import torch

from gen import rng, workloads as W
from oracle import mx as omx

import harness as HN

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_experts_fp8_amd")
DEV = "cuda"
SCHEMES = {"mxfp8": (1, omx.FMT_E4M3), "w4a8": (2, omx.FMT_E2M1)}


def test_quant_act_mx_bit_exact():
    r = np.random.default_rng(11)
    R, C = 97, 416
    x = r.standard_normal((R, C)) * np.exp2(r.integers(-30, 30, size=(R, 1)))
    x[3] = 0.0                                  # all-zero groups
    x[5, 32:64] = 0.0
    x[7, :32] = 1.0625 * 2.0 ** -3              # E4M3 midpoints after scaling
    x[7, 0] = 448 * 2.0 ** -3
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    xq, xs = M.moe_quant_act_mx(xb.to(DEV))
    q, s = omx.quant_rows_32(W.bf16_to_f64(xb))
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy(), s)


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_quant_weight_mx_bit_exact(scheme):
    _, fmt = SCHEMES[scheme]
    wfmt = M.MOE_WFMT_E2M1 if fmt == omx.FMT_E2M1 else M.MOE_WFMT_E4M3
    E, K, N = 3, 256, 96
    w = rng.normal_f32(rng.stream_key(0, 201, 0), E * K * N, 0.02).view(E, K, N)
    w[1, :32, 5] = 0.0                                               # an all-zero group
    w[2, 32:64, 7] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * 2.0 ** -9   # E2M1 ties
    q, s = M.moe_quant_weight_mx(w.to(DEV), wfmt)
    for e in range(E):
        qr, sr = omx.quant_weight_k32(w[e].double().numpy(), fmt)
        if fmt == omx.FMT_E2M1:
            qr = (qr[:, 0::2] & 15) | ((qr[:, 1::2] & 15) << 4)
        assert np.array_equal(q[e].cpu().numpy(), qr), e
        assert np.array_equal(s[e].cpu().numpy(), sr), e


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_prepack_mx_layout(scheme):
    _, fmt = SCHEMES[scheme]
    wfmt = M.MOE_WFMT_E2M1 if fmt == omx.FMT_E2M1 else M.MOE_WFMT_E4M3
    E, K, N = 2, 256, 48
    g = torch.Generator().manual_seed(12)
    q = torch.randint(0, 256, (E, K, N // 2 if wfmt else N), generator=g, dtype=torch.uint8)
    s = torch.randint(0, 256, (E, K // 32, N), generator=g, dtype=torch.uint8)
    pq, ps = M.moe_prepack_weights_mx(q.to(DEV), s.to(DEV), wfmt)
    pq, ps, qn, sn = pq.cpu().numpy(), ps.cpu().numpy(), q.numpy(), s.numpy()
    for e in range(E):
        for n16 in range(N // 16):
            for kb in range(K // 128):
                blk = (e * (N // 16) + n16) * (K // 128) + kb
                for lane in (0, 5, 16, 31, 47, 63):
                    n, k0 = n16 * 16 + lane % 16, kb * 128 + (lane // 16) * 32
                    assert ps[blk * 64 + lane] == sn[e, k0 // 32, n]
                    for b in (0, 7, 15):
                        if wfmt:
                            lo = (qn[e, k0 + 2 * b, n // 2] >> (4 * (n % 2))) & 15
                            hi = (qn[e, k0 + 2 * b + 1, n // 2] >> (4 * (n % 2))) & 15
                            assert pq[blk * 1024 + lane * 16 + b] == lo | (hi << 4)
                        else:
                            for h in (0, 1):
                                k = kb * 128 + h * 64 + (lane // 16) * 16 + b
                                assert pq[blk * 2048 + h * 1024 + lane * 16 + b] == qn[e, k, n]


def _run(wl, quant, w=None):
    x, logits, pre = HN.device_inputs(wl)
    w = w or HN.device_weights_mx(wl, quant)
    y, ids, wts, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, prelude=pre,
                                      return_routing=True)
    torch.cuda.synchronize()
    return y, ids.cpu().numpy(), counts.cpu().numpy()


def _oracle(wl, scheme, tokens=None):
    x = W.hidden_bf16(wl)
    xf = W.bf16_to_f64(x)
    logits = None if wl.prelude else W.router_logits(wl)
    ids, w, margin = HN.oracle_route(wl, x_f64=xf, logits=logits)
    tok = np.arange(wl.T) if tokens is None else (tokens(ids) if callable(tokens) else np.asarray(tokens))
    return omx.forward(xf, ids, w, None, tokens=tok, ffn_map=HN.oracle_ffn_map(wl, scheme)), ids, margin


SMALL = {
    "cfg1": W.CONFIGS[1],
    "ragged": W.Workload(131, "mx_ragged", T=37, H=256, I=384, E=5, k=3),
    "T1": W.Workload(132, "mx_one", T=1, H=128, I=128, E=1, k=1),
    "prelude": W.Workload(133, "mx_pre", T=9, H=512, I=256, E=16, k=4, prelude=True),
}


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", list(SMALL))
def test_mx_fused_small(scheme, name):
    quant, fmt = SCHEMES[scheme]
    wl = SMALL[name]
    print("mx fused", scheme, name, W.describe(wl), flush=True)
    y, ids, counts = _run(wl, quant)
    ref, ids_ref, margin = _oracle(wl, scheme)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    fro, mxe = HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], f"{scheme} {name}", ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mxe:.2e}", flush=True)


# prefill-sized shapes on the larger MX tiles (H % 256 == 0): 128-row tiles where experts
# average 25..127 rows, 256-row items from 128 on; several K blocks, one K block in the down
# GEMM (I = 128), ragged and skewed tiles, single-tile items; and the 16-row kernels at prefill
# size where H % 256 != 0
PREFILL = {
    "tiles128": W.Workload(139, "mx_t128", T=300, H=512, I=384, E=16, k=4),
    "tiles128_down_kb1": W.Workload(140, "mx_t128kb1", T=200, H=256, I=128, E=8, k=3),
    "pairs": W.Workload(134, "mx_pairs", T=600, H=512, I=384, E=8, k=3),
    "pairs_down_kb1": W.Workload(135, "mx_kb1", T=400, H=256, I=128, E=4, k=2),
    "pairs_skewed_ragged": W.Workload(136, "mx_skew", T=777, H=768, I=640, E=16, k=4, bias="normal1.5"),
    "H384_16row": W.Workload(137, "mx_h384", T=500, H=384, I=256, E=4, k=2),
}


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", list(PREFILL))
def test_mx_fused_prefill_tiles(scheme, name):
    quant, fmt = SCHEMES[scheme]
    wl = PREFILL[name]
    print("mx fused prefill", scheme, name, W.describe(wl), flush=True)
    y, ids, counts = _run(wl, quant)
    ref, ids_ref, margin = _oracle(wl, scheme)
    ok = margin >= 1e-5
    assert np.array_equal(ids[ok], ids_ref[ok])
    fro, mxe = HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], f"{scheme} {name}", ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mxe:.2e}", flush=True)


# configs 2 in full; 3, 4 and 5 on the tokens whose rows cover every 128 rows of every expert
# (every 16-row tile group of these kernels' tile list holds a checked row at most 128 rows
# away) plus every 64th token
@pytest.mark.timeout(900)
@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_mx_fused_workloads(scheme, cfg):
    quant, fmt = SCHEMES[scheme]
    wl = W.CONFIGS[cfg]
    print("mx fused workload", scheme, cfg, W.describe(wl), flush=True)
    y, ids, counts = _run(wl, quant)
    sample = None if cfg == 2 else (lambda ids_ref: HN.item_sample_tokens(ids_ref, wl.E))
    ref, ids_ref, margin = _oracle(wl, scheme, sample)
    tok = ref["tokens"]
    print(f"  {len(tok)} of {wl.T} tokens", flush=True)
    ok = margin[tok] >= 1e-5
    assert np.array_equal(ids[tok][ok], ids_ref[tok][ok])
    assert counts.sum() == wl.T * wl.k
    fro, mxe = HN.assert_output_close(HN.bf16_to_f64(y)[tok][ok], ref["y"][ok], f"{scheme} cfg{cfg}",
                                      ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mxe:.2e}", flush=True)


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_mx_grouped_ffn_unit_and_bf16_out(scheme):
    quant, fmt = SCHEMES[scheme]
    wl = W.CONFIGS[1]
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights_mx(wl, quant)
    r = M.moe_route(HN.device_params(wl), wl.T, router_logits=logits)
    xq, xs = M.moe_quant_act_mx(x)
    ref, ids_ref, _ = _oracle(wl, scheme)
    assert np.array_equal(xq.cpu().numpy(), ref["xq"]) and np.array_equal(xs.cpu().numpy(), ref["xs"])
    pos = r["assign_pos"].cpu().numpy().astype(np.int64)
    for dt in (torch.float32, torch.bfloat16):
        eo = M.moe_grouped_ffn(xq, xs, r, w, wl.k, out_dtype=dt)
        HN.assert_output_close(eo.float().cpu().numpy().astype(np.float64)[pos], ref["o"], f"{scheme} o {dt}",
                               ref["o_bound"])


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_mx_fused_shared_expert(scheme):
    quant, fmt = SCHEMES[scheme]
    wl = W.Workload(146, "mx_shared", T=40, H=256, I=256, E=6, k=2, shared=1)
    print("mx fused shared", scheme, W.describe(wl), flush=True)
    x, logits, _ = HN.device_inputs(wl)
    w = HN.device_weights_mx(wl, quant)
    y, ids, wts, counts = M.moe_fused(HN.device_params(wl), x, w, router_logits=logits, return_routing=True,
                                      shared_expert=True)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    xf = W.bf16_to_f64(W.hidden_bf16(wl))
    ids_ref, w_ref, margin = HN.oracle_route(wl, x_f64=xf, logits=W.router_logits(wl))
    ok = margin >= 1e-5
    assert (ids[:, wl.k] == wl.E).all() and np.array_equal(ids[ok, :wl.k], ids_ref[ok])
    assert counts.cpu().numpy()[wl.E] == wl.T
    # the shared expert as slot k with weight 1, as the FP8 oracle's forward_shared defines it
    ids_all = np.concatenate([ids_ref, np.full((wl.T, 1), wl.E, dtype=ids_ref.dtype)], axis=1)
    w_all = np.concatenate([np.asarray(w_ref, dtype=np.float64), np.ones((wl.T, 1))], axis=1)
    ref = omx.forward(xf, ids_all, w_all, None, ffn_map=HN.oracle_ffn_map(wl, scheme))
    fro, mxe = HN.assert_output_close(HN.bf16_to_f64(y)[ok], ref["y"][ok], f"{scheme} shared", ref["y_bound"][ok])
    print(f"  rel fro {fro:.2e} rel max {mxe:.2e}", flush=True)


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("wl", [W.CONFIGS[2], W.Workload(147, "mx_h7168", T=64, H=7168, I=256, E=4, k=2)],
                         ids=["decode_gemma4", "H7168_two_pass_rows"])
def test_mx_fused_activation_quant_bit_exact(scheme, wl):
    # the fused call's 32-group activation quantisation, taken in caller buffers: the
    # oracle's E4M3 codes and UE8M0 scales exactly, and y unchanged by taking them; H = 7168
    # takes the routing kernel's two-pass row quantisation (rows longer than 4096)
    quant, _ = SCHEMES[scheme]
    print("mx fused act quant", scheme, W.describe(wl), flush=True)
    x, logits, pre = HN.device_inputs(wl)
    w = HN.device_weights_mx(wl, quant)
    p = HN.device_params(wl)
    xq = torch.empty(wl.T, wl.H, dtype=torch.uint8, device=DEV)
    xs = torch.empty(wl.T, wl.H // 32, dtype=torch.uint8, device=DEV)
    y = M.moe_fused(p, x, w, router_logits=logits, prelude=pre, act_q=xq, act_scales=xs)
    y0 = M.moe_fused(p, x, w, router_logits=logits, prelude=pre)
    torch.cuda.synchronize()
    q, s = omx.quant_rows_32(W.bf16_to_f64(W.hidden_bf16(wl)))
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy(), s)
    assert torch.equal(y, y0)
