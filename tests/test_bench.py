"""Host-side pieces of bench.py: the algorithmic counts, the recorded-traffic
lookup and the one-GPU contract (no GPU needed)."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_decode_counts_match_the_byte_rule():
    """Algorithmic bytes: every active expert once + router + x in + out."""
    wl = synth.WORKLOADS["decode_bf16"]
    D = 76
    c = bench.layer_counts(wl, 16, D)
    H, I, E = wl.hidden, wl.inter, wl.experts
    assert c["bytes"] == D * 3 * I * H * 2 + E * H * 2 + 2 * 16 * H * 2
    assert c["gateup"]["bytes"] >= D * 2 * I * H * 2
    assert c["flops"] == 2 * 16 * E * H + 2 * 16 * 8 * 3 * H * I


def test_mxfp4_counts_take_half_a_byte_per_weight_and_a_scale_byte_per_32():
    wl = synth.WORKLOADS["decode_mxfp4"]
    D = 76
    c = bench.layer_counts(wl, 16, D)
    H, I, E = wl.hidden, wl.inter, wl.experts
    w13 = D * (2 * I * H // 2 + 2 * I * H // 32)
    w2 = D * (H * I // 2 + H * I // 32)
    assert c["bytes"] == w13 + w2 + E * H * 2 + 2 * 16 * H * 2
    assert c["gateup"]["bytes"] == w13 + 16 * H * 2 + 16 * 8 * I * 2   # x in, bf16 h out
    assert bench.MFMA_PEAK_TFLOPS["mxfp4"] == bench.MFMA_PEAK_TFLOPS["bf16"]
    assert bench.COMPUTE_DTYPE["mxfp4"] == "bf16"


def test_fp8_layer_products_take_the_bf16_peak():
    assert bench.MFMA_PEAK_TFLOPS["fp8"] == bench.MFMA_PEAK_TFLOPS["bf16"]
    assert bench.COMPUTE_DTYPE["fp8"] == "bf16"


def test_every_config_entry_names_a_workload_with_a_cpu_sample():
    for name, m, launch in bench.CONFIG_RUNS:
        assert name in synth.WORKLOADS and launch in ("eager", "graph")
        assert m <= synth.WORKLOADS[name].m
        assert name in bench.CPU_SAMPLE
    assert "large_fp8" in bench.CPU_SAMPLE


def test_recorded_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The counters stand only while the kernel's sources are the ones counted."""
    files = bench.KERNEL_SOURCES["small_m"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixture_experts_ffn_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"decode_bf16|m=16|gateup": {"read_bytes": 100.0, "write_bytes": 5.0,
                                        "source_sha256": h.hexdigest()}}
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    real_csrc = os.path.join(ROOT, "mixture_experts_ffn_06_amd")
    (tmp_path / "mixture_experts_ffn_06_amd").symlink_to(real_csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("decode_bf16", 16, "gateup", "small_m") == 105.0
    assert bench.recorded_traffic("decode_bf16", 16, "down", "small_m") is None
    assert bench.recorded_traffic("decode_bf16", 16, "gateup", "simple") is None
    rec["decode_bf16|m=16|gateup"]["source_sha256"] = "0" * 64
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("decode_bf16", 16, "gateup", "small_m") is None
