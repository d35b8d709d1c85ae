"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte and flop
accounting of the two GEMM stages and of the step, and the roofline entry's choice of bound.
The expected values are worked out by hand below from the definitions (weights of every
active expert read once, activation rows read once, h written once and read once, outputs
written once)."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _wl(**kw):
    d = dict(T=4, H=256, I=128, E=3, k=2, shared=0, prelude=False)
    d.update(kw)
    return SimpleNamespace(**d)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stage_bytes_fp8_by_hand():
    # T=4 tokens, k=2 -> A=8 assignments; experts 0 and 2 active (counts 3 and 5).
    # gate+up: 2 experts x (256 x 256 weight bytes + 256*256/16384 = 4 scale bytes) = 131080,
    #   x rows 4 x 256 = 1024 (+ 1024/128 = 8 scale bytes), h 8 x 128 = 1024 (+ 8) -> 133144
    # down: 2 x (128 x 256 + 2) = 65540, h read 1024 + 8, fp32 out 8 x 256 x 4 = 8192 -> 74764
    wl = _wl()
    b, n_act = bench.stage_bytes_flops(wl, np.array([3, 0, 5]), eo_bytes=4)
    assert n_act == 2
    assert b["gate_up_gemm"] == (133144, 4.0 * 8 * 256 * 128)
    assert b["down_gemm"] == (74764, 2.0 * 8 * 256 * 128)


def test_stage_bytes_w4a8_and_w8a16_by_hand():
    wl = _wl()
    # W4A8: half a byte per weight, one scale byte per 32 weights and per 32 activations.
    # gate+up: 2 x (65536 x 0.5 + 65536/32) = 69632; x 1024 + 32; h 1024 + 32 -> 71744
    b, _ = bench.stage_bytes_flops(wl, np.array([3, 0, 5]), eo_bytes=2, quant="w4a8")
    assert b["gate_up_gemm"][0] == 71744
    # down: 2 x (32768 x 0.5 + 1024) = 34816; h 1024 + 32; bf16 out 8 x 256 x 2 = 4096 -> 39968
    assert b["down_gemm"][0] == 39968
    # W8A16: E4M3 weights with 128x128 scales, activations 2 bytes and no scales.
    # gate+up: 131080 + x 2048 + h 2048 = 135176; down: 65540 + 2048 + 8192 = 75780
    b, _ = bench.stage_bytes_flops(wl, np.array([3, 0, 5]), eo_bytes=4, quant="w8a16")
    assert b["gate_up_gemm"][0] == 135176
    assert b["down_gemm"][0] == 75780


def test_step_bytes_by_hand():
    # 2 active experts x 3 x 256 x 128 weight bytes (+ 2 x 6 scale bytes) = 196620; x read and
    # y written 2 x 4 x 256 x 2 = 4096; ids + weights 8 x 8 = 64; logits 4 x 3 x 4 = 48
    assert bench.step_algorithmic_bytes(_wl(), 2) == 196620 + 4096 + 64 + 48
    # with the prelude: router weights 3 x 256 x 4, norm 256 x 4, per-expert scale 3 x 4
    assert bench.step_algorithmic_bytes(_wl(prelude=True), 2) == 196620 + 4096 + 64 + 3072 + 1024 + 12


def test_roofline_entry_picks_the_binding_roof():
    # 8 GB in 2 ms: the HBM time (1 ms) exceeds the FP8 time of 1 TFLOP (0.2 ms)
    r = bench.roofline_entry("k", 2e-3, 8e9, 1e12, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    # 8 MB and 10 TFLOP in 4 ms: the FP8 time (2 ms) exceeds the HBM time (1 us)
    r = bench.roofline_entry("k", 4e-3, 8e6, 1e13, 12345)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2500.0) and r["frac"] == pytest.approx(0.5)
    assert r["traffic"] == 12345
    # a bf16 contraction is priced against the bf16 peak
    r = bench.roofline_entry("k", 4e-3, 8e6, 1e13, None, peak_tflops=bench.SCHEME_PEAK["w8a16"])
    assert r["peak"] == 2500.0 and r["frac"] == pytest.approx(1.0)


def test_traffic_is_dropped_once_the_kernels_change(tmp_path, monkeypatch):
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 777}
    (tmp_path / "traffic_gate_up_gemm_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "gate_up_gemm") == 777
    rec["source_hash"] = "0" * 16
    (tmp_path / "traffic_gate_up_gemm_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "gate_up_gemm") is None
    assert bench.load_traffic("absent", "gate_up_gemm") is None


def test_expert_out_auto_is_bf16_for_the_prefill_shapes_only():
    from gen import workloads as W
    auto = {c: bench.expert_out_dtype(W.CONFIGS[c], "auto") for c in W.CONFIGS}
    assert auto == {1: "fp32", 2: "fp32", 3: "bf16", 4: "bf16", 5: "bf16", 6: "bf16"}
    assert bench.expert_out_dtype(W.CONFIGS[2].replace(shared=1), "auto") == "fp32"
    assert bench.expert_out_dtype(W.CONFIGS[5], "fp32") == "fp32"
    assert bench.expert_out_dtype(W.CONFIGS[1], "bf16") == "bf16"
