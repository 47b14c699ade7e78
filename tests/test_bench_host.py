"""Host-side checks of bench.py (no GPU): the one-GPU contract, the gating of
the measured HBM traffic on the GEMM source, and the step's work accounting
against the sizes of the decode-step workload (36 layers of a Qwen3-8B-shaped
stack, 128 x (16 + 16) rows, 8K cache, vocabulary 151,936)."""

import hashlib
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    # a copy of the tree's summary and source under a temporary root
    (tmp_path / "profiles").mkdir()
    src_dir = tmp_path / "diffusion_augmented_decoding_amd" / "csrc"
    src_dir.mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "profiles", "uno_gemm_bf16_full_step_traffic.txt"), tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "diffusion_augmented_decoding_amd", "csrc", "gated_lora.hip"), src_dir)
    text = (tmp_path / "profiles" / "uno_gemm_bf16_full_step_traffic.txt").read_text()
    recorded = [ln.split()[1] for ln in text.splitlines() if ln.startswith("source_sha256")][0]
    current = hashlib.sha256((src_dir / "gated_lora.hip").read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.measured_traffic("uno_gemm_bf16_full_step_traffic.txt", "gated_lora.hip")
    if recorded == current:
        assert got is not None and got > 1e8
    else:
        assert got is None
    # any change to the source disables the figure
    with open(src_dir / "gated_lora.hip", "a") as f:
        f.write("\n// edited\n")
    assert bench.measured_traffic("uno_gemm_bf16_full_step_traffic.txt", "gated_lora.hip") is None
    # a missing summary gives no figure either
    assert bench.measured_traffic("no_such_summary.txt", "gated_lora.hip") is None


def test_step_work_accounting():
    f = bench.FULL
    assert (f["n_layers"], f["batch"], f["block"], f["ctx"], f["hidden"], f["inter"], f["vocab"]) == \
        (36, 128, 16, 8192, 4096, 12288, 151936)
    rows = 4096
    main_head, down = bench.full_step_flops(m_on=2048)
    head = 2.0 * rows * 151936 * 4096
    # base projections per layer: q 4096x4096, k and v 1024x4096, o 4096x4096,
    # gate and up 12288x4096, down 4096x12288 (N x K), 2 M N K flops each
    base_per_layer = 2.0 * rows * (4096 * 4096 * 2 + 1024 * 4096 * 2 + 12288 * 4096 * 3)
    lora_up = 2.0 * 2048 * 128 * (4096 * 2 + 1024 * 2 + 12288 * 2 + 4096) * 36
    assert main_head == pytest.approx(base_per_layer * 36 + lora_up + head, rel=1e-12)
    assert base_per_layer * 36 / 1e12 == pytest.approx(56.9, rel=2e-3)     # 56.9 TFLOP of base GEMMs
    assert head / 1e12 == pytest.approx(5.10, rel=2e-3)                    # LM head 5.10 TFLOP
    # LoRA-down on the gated rows: x A^T for every projection's input width
    assert down == pytest.approx(2.0 * 2048 * 128 * (4096 * 6 + 12288) * 36, rel=1e-12)
    # KV cache read per step: 36 layers x K and V of 128 sequences x 8192 x 8 heads x 128, bf16
    kv_step = 36 * 2.0 * 128 * 8192 * 8 * 128 * 2
    assert kv_step / 1e9 == pytest.approx(154.6, rel=2e-3)
    assert bench.full_step_attention_bytes() * 36 > kv_step
