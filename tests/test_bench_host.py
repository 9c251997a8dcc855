"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the recorded HBM traffic
lookup that is valid only for the kernel source it was measured on, the algorithmic work."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    v = bench.recorded_traffic("mixtral-token-choice-bf16")
    assert v is None or v > 1e9
    # a copy of the tree whose GEMM source differs: the record no longer applies
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "hbm_traffic_gemm.md"), tmp_path / "profiles")
    csrc = tmp_path / "mixture_experts_layer_42_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = open(os.path.join(ROOT, "mixture_experts_layer_42_amd", "csrc", "gemm.hip")).read()
    (csrc / "gemm.hip").write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("mixtral-token-choice-bf16") == v
    (csrc / "gemm.hip").write_text(src + "\n// changed\n")
    assert bench.recorded_traffic("mixtral-token-choice-bf16") is None
    assert bench.recorded_traffic("no-such-workload") is None


@pytest.mark.parametrize("name", ["mixtral-token-choice-bf16", "fine-grained-shared-bf16"])
def test_algorithmic_flops(name):
    cfg = mi.workload(name)
    w = bench.algorithmic(cfg, 1000)
    d, f, fs, T = cfg.d_model, cfg.d_ff, cfg.d_ff_shared, cfg.T
    assert w["gate_up"] == 4.0 * d * f * 1000 + 4.0 * d * fs * T
    assert w["down"] == 2.0 * d * f * 1000 + 2.0 * d * fs * T
