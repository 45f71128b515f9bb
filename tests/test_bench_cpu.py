"""Host logic of bench.py, on the CPU: the one-GPU contract, the hash gate on the
committed counter summary, and the algorithmic byte counts behind roofline.achieved."""
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_while_the_profiled_sources_are_unchanged(monkeypatch):
    traffic, src = bench.profile_traffic("balanced")
    if traffic is not None:                      # the committed summary matches these sources
        assert src.startswith("profiles" + os.sep)
        assert 5e8 < traffic < 5e9
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: "0000000000000000")
    assert bench.profile_traffic("balanced") == (None, None)
    assert bench.profile_traffic("no such workload") == (None, None)


def test_kernel_source_hash_follows_the_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "grouped_gemm_expert_offsets_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.BF16_KERNEL_SOURCES:
        (csrc / name).write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "kgw_bf16.hip").write_text("y")
    assert bench.kernel_source_hash() != h0


def _wl(name):
    spec = workloads.config_spec(name, 1)
    return SimpleNamespace(hidden=spec["hidden"], n=spec["n"], tokens_sum=sum(spec["counts"]), counts=spec["counts"],
                           num_experts=len(spec["counts"]), kind=spec["kind"], out_dtype=spec["out_dtype"],
                           accumulate=spec["accumulate"])


@pytest.mark.parametrize("name", ["tiny", "balanced", "skewed", "fp8", "many_small"])
def test_algorithmic_bytes_closed_form(name):
    w = _wl(name)
    H, N, T, E = w.hidden, w.n, w.tokens_sum, w.num_experts
    if w.kind == "fp8":
        inputs = H * T + T * N + (T // 128) * (H + N)          # e4m3 bytes + one scale byte per 128 tokens
    else:
        inputs = 2 * (H * T + T * N)                            # bf16
    # accumulate leaves experts without tokens untouched; overwrite zero-fills them
    touched = sum(1 for c in w.counts if c > 0) if w.accumulate else E
    out = touched * H * N * (4 if w.out_dtype == torch.float32 else 2)
    assert bench.algorithmic_bytes(w) == inputs + out * (2 if w.accumulate else 1)


def test_skewed_accumulate_skips_empty_experts():
    w = _wl("skewed")
    assert w.accumulate and sum(1 for c in w.counts if c == 0) == 4
    full = 2 * (w.hidden * w.tokens_sum + w.tokens_sum * w.n) + 32 * w.hidden * w.n * 4 * 2
    assert bench.algorithmic_bytes(w) == full - 4 * w.hidden * w.n * 4 * 2


def test_headline_workload_bytes_and_flops():
    # balanced: E=8, hidden 4096, N 2048, tokens_sum 35584, bf16 output
    w = _wl("balanced")
    assert (w.num_experts, w.hidden, w.n, w.tokens_sum) == (8, 4096, 2048, 35584)
    assert bench.algorithmic_bytes(w) == 571473920.0
    assert 2 * w.hidden * w.n * w.tokens_sum == 597000454144
