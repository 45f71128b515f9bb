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
    for workload, kind in (("balanced", "bf16"), ("fp8", "fp8")):
        traffic, src = bench.profile_traffic(workload, kind)
        if traffic is not None:                  # the committed summary matches these sources
            assert src.startswith("profiles" + os.sep)
            assert 5e8 < traffic < 5e10
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: "0000000000000000")
    assert bench.profile_traffic("balanced", "bf16") == (None, None)
    assert bench.profile_traffic("fp8", "fp8") == (None, None)
    assert bench.profile_traffic("no such workload", "bf16") == (None, None)


@pytest.mark.parametrize("kind,main", [("bf16", "kgw_bf16.hip"), ("fp8", "kgw_fp8_exact.hip")])
def test_kernel_source_hash_follows_the_sources(tmp_path, monkeypatch, kind, main):
    csrc = tmp_path / "grouped_gemm_expert_offsets_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES[kind]:
        (csrc / name).write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash(bench.KERNEL_SOURCES[kind])
    (csrc / main).write_text("y")
    assert bench.kernel_source_hash(bench.KERNEL_SOURCES[kind]) != h0


def test_headline_is_the_largest_configuration():
    # the headline runs the configuration with the most useful work, through the entry point
    # that meets the accuracy bound
    flops = {n: 2 * s["hidden"] * s["n"] * sum(s["counts"])
             for n, s in ((n, workloads.config_spec(n, 1)) for n in workloads.CONFIG_NAMES)}
    assert bench.HEADLINE == max(flops, key=flops.get) == "fp8"


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
    # fp8: E=32, hidden 7168, N 4096, tokens_sum 264320, e4m3 operands, bf16 output
    w = _wl("fp8")
    assert (w.num_experts, w.hidden, w.n, w.tokens_sum) == (32, 7168, 4096, 264320)
    T = 264320
    assert bench.algorithmic_bytes(w) == 7168 * T + T * 4096 + (T // 128) * (7168 + 4096) + 32 * 7168 * 4096 * 2
    assert 2 * w.hidden * w.n * w.tokens_sum == 2 * 7168 * 4096 * 264320


def test_single_line_option_names_every_secondary_kind():
    # `--line` runs one secondary measurement alone (what the committed profiles of those
    # kernels were taken with); unknown names are refused before anything runs
    assert set(bench.LINES) == {"fp4", "mgrouped_nt", "mgrouped_nn", "mgrouped_fp8_nt", "mgrouped_fp8_nn",
                                "quantize_fp8_A", "quantize_fp8_B", "quantize_fp4_A", "quantize_fp4_B"}
    assert all(callable(f) for f in bench.LINES.values())
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--line", "no_such_line"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "invalid choice" in r.stderr
