#!/usr/bin/env python3
"""Throughput of the K-grouped MoE weight-gradient GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S]

One step = one kgw_wgrad_* call over one batch of seeded synthetic input
already resident in HBM: offsets decode, tile scheduling, zero-fill, operand
staging, the MFMA K loop and the epilogue all run inside that one launch.
The headline workload is the largest of the five configurations: the fp8
e4m3 weight gradient with one UE8M0 scale per 128 tokens (E=32, hidden 7168,
N 4096, n_e = roundup128(8192*U(0.7,1.3)), seed 1, bf16 output, overwrite),
through kgw_wgrad_fp8, the entry point that meets the accuracy bound.  Useful
work = 2 * hidden * N * tokens_sum FLOP, priced against the dense fp8 MFMA
peak (the exact kernel multiplies on the bf16 MFMA, whose rate is half that).

Prints ONE JSON line.  `roofline.achieved` divides the useful FLOP of one
launch by the launch's average duration, timed with HIP events recorded on
the launch stream around every timed launch.  `roofline.traffic` comes from
the rocprofv3 counter summary committed under profiles/ for this workload,
and is null when the kernel sources changed after those counters were taken.
`cpu_baseline` times the CPU oracle on a bounded sample of each of the five
configurations (the headline's is the top-level value).  `secondary` reports
the other workloads (balanced, skewed-accumulate, many-small and tiny bf16,
the native fp8 path, 32-token (MX-style) scales, FP4 operands, the m-grouped
forward and dgrad of the fp8 workload's layer, and the on-device fp8 and FP4
quantisers) with the same timing.

Warm-up: from idle the GPU needs about 100 ms of continuous load before its
clocks settle, so every timed workload first runs for at least
`--warmup-seconds` (headline, default 1 s) or `--secondary-warm-seconds`
(default 0.2 s), and at least W launches.  The numbers are steady-state
throughput, as in a training loop.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of MFMA peak, K-grouped MoE wgrad (bf16 and fp8), 1 GPU"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10066.3     # MI355X dense fp4 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
HEADLINE = "fp8"


# Sources each timed kernel is built from (the bf16 kernel for the bf16 workloads, the exact
# fp8 kernel for the headline).
KERNEL_SOURCES = {
    "bf16": ("kgw_bf16.hip", "kgw_device.h", "kgw_internal.h", "kgw_tile_io.h", "kgw_host.hip"),
    "fp8": ("kgw_fp8_exact.hip", "kgw_device.h", "kgw_internal.h", "kgw_tile_io.h", "kgw_host.hip"),
}


def kernel_source_hash(files=KERNEL_SOURCES["fp8"]) -> str:
    """Short sha256 over the named csrc files; a profile summary records it so that its
    counter readings are used only while the kernel they were taken on is unchanged."""
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(ROOT, "grouped_gemm_expert_offsets_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_traffic(workload: str, kind: str):
    """HBM bytes per launch from profiles/<...>.md, if taken on the current kernel sources."""
    cur = kernel_source_hash(KERNEL_SOURCES[kind])
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        if f"workload: {workload}" not in text:
            continue
        m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
        m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
        if m_hash and m_bytes and m_hash.group(1) == cur:
            return float(m_bytes.group(1)), os.path.relpath(path, ROOT)
    return None, None


def algorithmic_bytes(wl) -> float:
    """Read A and B once, write the output once (read it too when accumulating), plus scales.
    In accumulate mode an expert without tokens is left untouched, so its output counts zero."""
    import torch
    H, N, T = wl.hidden, wl.n, wl.tokens_sum
    el_in = 1 if wl.kind == "fp8" else 2
    el_out = 4 if wl.out_dtype == torch.float32 else 2
    touched = sum(1 for c in wl.counts if c > 0) if wl.accumulate else len(wl.counts)
    b = (H * T + T * N) * el_in + touched * H * N * el_out * (2 if wl.accumulate else 1)
    if wl.kind == "fp8":
        b += (T // 128) * (H + N)
    return float(b)


def make_call(wl, out, native=False, layout=("k", "n")):
    import grouped_gemm_expert_offsets_amd as kgw
    if layout != ("k", "n"):
        # fp8 operands stored in another layout (exact path, byte scales): A (T, hidden) for
        # a_major "m", B (n, T) for b_major "k"
        a = wl.A.t().contiguous() if layout[0] == "m" else wl.A
        b = wl.B.t().contiguous() if layout[1] == "k" else wl.B
        return lambda: kgw.kgw_wgrad_fp8_ex(a, wl.sfa, b, wl.sfb, wl.offsets, a_major=layout[0], b_major=layout[1],
                                            out=out, accumulate=wl.accumulate)
    if wl.kind == "bf16":
        return lambda: kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out, accumulate=wl.accumulate)
    if wl.scale_block == 32:
        import workloads
        sfa, sfb = workloads.pack_scale_words(wl.sfa), workloads.pack_scale_words(wl.sfb)
        return lambda: kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED_32,
                                            native=native, out=out, accumulate=wl.accumulate)
    fn = kgw.kgw_wgrad_fp8_native if native else kgw.kgw_wgrad_fp8
    return lambda: fn(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out, accumulate=wl.accumulate)


def time_call(call, steps: int, warmup: int, min_warm_s: float = 0.0, stats: dict = None):
    """Wall time of `steps` back-to-back calls plus HIP-event time of each launch, after
    `warmup` untimed calls (continued until `min_warm_s` seconds have passed, if given).
    The warm-up actually run is recorded in `stats` (launches, seconds)."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    for _ in range(warmup):
        call()
        done += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t_warm < min_warm_s:
        for _ in range(4):
            call()
        done += 4
        torch.cuda.synchronize()
    if stats is not None:
        stats["warmup_launches"] = done
        stats["warmup_seconds"] = time.perf_counter() - t_warm
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        call()
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall_ms / steps, launch_ms


def run_flushed(name: str, steps: int, warmup: int):
    """The workload with a 512 MiB device write before every launch (untimed), so each timed
    launch starts with the operands out of the Infinity Cache (256 MB): HIP events around
    each launch on the launch stream, mean over `steps` after `warmup` launches."""
    import torch
    import workloads
    wl = workloads.make_workload(name, seed=1, device="cuda")
    out = wl.C0 if wl.accumulate else torch.empty((wl.num_experts, wl.hidden, wl.n), dtype=wl.out_dtype,
                                                  device="cuda")
    call = make_call(wl, out)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        call()
    times = []
    for _ in range(steps):
        scratch.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        call()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    mean = sum(times) / len(times)
    res = {"workload": name + "_mall_flushed", "launch_ms_mean": mean, "launch_ms_min": min(times),
           "launch_ms_max": max(times), "tflops": wl.flops / (mean * 1e-3) / 1e12}
    res["frac_of_mfma_peak"] = res["tflops"] / PEAK_BF16_TFLOPS
    del wl, out, scratch
    torch.cuda.empty_cache()
    return res


def run_workload(name: str, steps: int, warmup: int, native=False, seed: int = 1, min_warm_s: float = 0.0,
                 scale_block: int = 128, layout=("k", "n")):
    import torch
    import workloads
    if scale_block == 128:
        wl = workloads.make_workload(name, seed=seed, device="cuda")
    else:
        spec = workloads.config_spec(name, seed)
        std = spec.pop("std")
        wl = workloads.make_operands(seed=seed, device="cuda", std=std, name=name, scale_block=scale_block, **spec)
    out = wl.C0 if wl.accumulate else torch.empty((wl.num_experts, wl.hidden, wl.n), dtype=wl.out_dtype,
                                                  device="cuda")
    warm = {}
    ms_step, launch_ms = time_call(make_call(wl, out, native, layout), steps, warmup, min_warm_s, warm)
    launch_ms.sort()
    mean_launch = sum(launch_ms) / len(launch_ms)
    res = {
        "workload": (name + ("_mx32" if scale_block == 32 else "") + ("_native" if native else "") +
                     ("" if layout == ("k", "n") else f"_a_{layout[0]}_major_b_{layout[1]}_major")),
        "ms_per_step": ms_step,
        "launch_ms_mean": mean_launch,
        "launch_ms_median": launch_ms[len(launch_ms) // 2],
        "launch_ms_min": launch_ms[0],
        "launch_ms_max": launch_ms[-1],
        "tflops": wl.flops / (mean_launch * 1e-3) / 1e12,
        "flops_per_launch": wl.flops,
        "algorithmic_bytes": algorithmic_bytes(wl),
        "warmup_launches": warm["warmup_launches"],
        "warmup_seconds": warm["warmup_seconds"],
    }
    peak = PEAK_FP8_TFLOPS if wl.kind == "fp8" else PEAK_BF16_TFLOPS
    res["frac_of_mfma_peak"] = res["tflops"] / peak
    res["hbm_gbps_algorithmic"] = res["algorithmic_bytes"] / (mean_launch * 1e-3) / 1e9
    res["frac_of_hbm_peak"] = res["hbm_gbps_algorithmic"] / PEAK_HBM_GBPS
    del wl, out
    torch.cuda.empty_cache()
    return res


def run_quantize(token_axis: int, steps: int, warmup: int, min_warm_s: float = 0.0, fp4: bool = False):
    """kgw_quantize_fp8 (or kgw_quantize_fp4, 32-token scales packed as the FP4 product takes
    them) on the bf16 operand shape of the product it feeds (A: (hidden, tokens_sum),
    token_axis 1; B: (tokens_sum, n), token_axis 0): the fp8 workload's, or for fp4 the FP4
    line's (the same counts rounded up to 256 tokens, as the FP4 product requires).
    HBM-bound: per element 2 bytes read and 1 (fp8) or 0.5 (fp4) written, plus one scale byte
    per 128 (fp8) or 32 (fp4) tokens."""
    import torch
    import grouped_gemm_expert_offsets_amd as kgw
    import workloads
    spec = workloads.config_spec("fp8", 1)
    counts = workloads.counts_uniform(32, 8192, 256, 1) if fp4 else spec["counts"]
    T, H, N = sum(counts), spec["hidden"], spec["n"]
    shape = (H, T) if token_axis else (T, N)
    g = torch.Generator(device="cuda").manual_seed(1)
    x = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    fn = kgw.kgw_quantize_fp4 if fp4 else kgw.kgw_quantize_fp8
    ms_step, launch_ms = time_call(lambda: fn(x, token_axis), steps, warmup, min_warm_s)
    mean_launch = sum(launch_ms) / len(launch_ms)
    nbytes = (2.5 * x.numel() + x.numel() / 32) if fp4 else (3.0 * x.numel() + x.numel() / 128)
    kind = "fp4" if fp4 else "fp8"
    res = {
        "workload": f"quantize_{kind}_{'A' if token_axis else 'B'} {shape[0]}x{shape[1]} bf16 "
                    f"({'fp4' if fp4 else 'fp8'} workload operand)",
        "ms_per_step": ms_step,
        "launch_ms_mean": mean_launch,
        "algorithmic_bytes": nbytes,
        "hbm_gbps_algorithmic": nbytes / (mean_launch * 1e-3) / 1e9,
    }
    res["frac_of_hbm_peak"] = res["hbm_gbps_algorithmic"] / PEAK_HBM_GBPS
    del x
    torch.cuda.empty_cache()
    return res


def run_mgrouped(layout: str, steps: int, warmup: int, min_warm_s: float = 0.0):
    """kgw_mgrouped_bf16 on the fp8 workload's layer: 32 groups of roundup128(8192*U(0.7,1.3))
    rows; forward ("nt") X (T, 7168) @ W^T with W (32, 4096, 7168); dgrad ("nn") dY (T, 4096) @ W
    with W (32, 4096, 7168) read as (K=4096, N=7168); bf16 output."""
    import torch
    import grouped_gemm_expert_offsets_amd as kgw
    import workloads
    counts = workloads.counts_uniform(32, 8192, 128, 1)
    K, N = (7168, 4096) if layout == "nt" else (4096, 7168)
    wl = workloads.make_mgrouped(counts, K, N, layout, seed=1, device="cuda")
    out = torch.empty((wl.M, N), dtype=torch.bfloat16, device="cuda")
    ms_step, launch_ms = time_call(lambda: kgw.kgw_mgrouped_bf16(wl.A, wl.W, offsets=wl.offsets, layout=layout,
                                                                 out=out), steps, warmup, min_warm_s)
    mean_launch = sum(launch_ms) / len(launch_ms)
    res = {
        "workload": f"mgrouped_{layout} {'forward' if layout == 'nt' else 'dgrad'} M={wl.M} K={K} N={N} E=32 bf16",
        "ms_per_step": ms_step,
        "launch_ms_mean": mean_launch,
        "tflops": wl.flops / (mean_launch * 1e-3) / 1e12,
        "flops_per_launch": wl.flops,
    }
    res["frac_of_mfma_peak"] = res["tflops"] / PEAK_BF16_TFLOPS
    del wl, out
    torch.cuda.empty_cache()
    return res


def run_mgrouped_fp8(layout: str, steps: int, warmup: int, min_warm_s: float = 0.0):
    """kgw_mgrouped_fp8 on the fp8 workload's layer: 32 groups of roundup128(8192*U(0.7,1.3))
    rows, e4m3 operands with 1x128 UE8M0 scales along K (block-quantised Gaussian draws), bf16
    output; forward ("nt") X (T, 7168) @ W^T with W (32, 4096, 7168); dgrad ("nn") dY (T, 4096)
    @ W with the weight stored (32, K=4096, N=7168)."""
    import torch
    import grouped_gemm_expert_offsets_amd as kgw
    import workloads
    counts = workloads.counts_uniform(32, 8192, 128, 1)
    K, N = (7168, 4096) if layout == "nt" else (4096, 7168)
    wl = workloads.make_mgrouped_fp8(counts, K, N, seed=1, device="cuda")
    W = wl.W if layout == "nt" else wl.W.transpose(1, 2).contiguous()
    out = torch.empty((wl.M, N), dtype=torch.bfloat16, device="cuda")
    ms_step, launch_ms = time_call(lambda: kgw.kgw_mgrouped_fp8(wl.A, wl.sa, W, wl.sw, offsets=wl.offsets,
                                                                layout=layout, out=out), steps, warmup, min_warm_s)
    mean_launch = sum(launch_ms) / len(launch_ms)
    res = {
        "workload": (f"mgrouped_fp8_{layout} {'forward' if layout == 'nt' else 'dgrad'} M={wl.M} K={K} N={N} E=32 "
                     "e4m3 1x128 UE8M0, bf16 out"),
        "ms_per_step": ms_step,
        "launch_ms_mean": mean_launch,
        "tflops": wl.flops / (mean_launch * 1e-3) / 1e12,
        "flops_per_launch": wl.flops,
    }
    res["frac_of_mfma_peak"] = res["tflops"] / PEAK_FP8_TFLOPS
    res["frac_of_bf16_mfma_peak"] = res["tflops"] / PEAK_BF16_TFLOPS
    del wl, W, out
    torch.cuda.empty_cache()
    return res


def run_fp4(steps: int, warmup: int, min_warm_s: float = 0.0):
    """kgw_wgrad_fp4 on the fp8 workload's shape (E=32, hidden 7168, n 4096, counts
    roundup256(8192*U(0.7,1.3))), e2m1 operands with uniformly random codes and 32-token scales
    drawn on the device, bf16 output."""
    import torch
    import grouped_gemm_expert_offsets_amd as kgw
    import workloads
    counts = workloads.counts_uniform(32, 8192, 256, 1)
    wl = workloads.make_fp4_operands(counts, 7168, 4096, seed=1, device="cuda", random_codes=True)
    sa, sb = workloads.pack_scale_words(wl["sfa"]), workloads.pack_scale_words(wl["sfb"])
    out = torch.empty((32, 7168, 4096), dtype=torch.bfloat16, device="cuda")
    ms_step, launch_ms = time_call(lambda: kgw.kgw_wgrad_fp4(wl["A"], sa, wl["B"], sb, wl["offsets"], out=out),
                                   steps, warmup, min_warm_s)
    mean_launch = sum(launch_ms) / len(launch_ms)
    flops = 2.0 * 7168 * 4096 * sum(counts)
    res = {
        "workload": f"fp4 e2m1 32-token UE8M0 E=32 H=7168 N=4096 tokens_sum={sum(counts)}, bf16 out",
        "ms_per_step": ms_step,
        "launch_ms_mean": mean_launch,
        "tflops": flops / (mean_launch * 1e-3) / 1e12,
        "flops_per_launch": flops,
    }
    res["frac_of_mfma_peak"] = res["tflops"] / PEAK_FP4_TFLOPS
    del wl, out, sa, sb
    torch.cuda.empty_cache()
    return res


def _oracle_sample(name: str, target_seconds: float):
    """Time the CPU oracle on a bounded sample of workload `name` (seed 1): whole rows of its
    first non-empty expert (the tokens of that expert, all N columns), as many as fit in about
    `target_seconds`, from the very tensors the GPU line consumes (generated on the device and
    copied out).  The tiny workload is small enough to run whole."""
    import numpy as np
    import torch
    import oracle
    import workloads
    wl = workloads.make_workload(name, seed=1, device="cuda")
    threads = oracle.num_threads()
    if name == "tiny":
        A, B, off = wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu()
        t0 = time.perf_counter()
        oracle.wgrad_bf16(A, B, off)
        dt = time.perf_counter() - t0
        return {"value": wl.flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"the whole {name} workload: {wl.flops:.3e} FLOP in {dt:.3f} s", "seconds": dt}
    e = next(i for i, c in enumerate(wl.counts) if c > 0)
    begin = int(sum(wl.counts[:e]))
    n_e = wl.counts[e]
    rows = min(wl.hidden, max(threads, 1))
    # one expert's tokens only, re-based so the oracle sees a one-expert problem
    def take(r):
        A = wl.A[:r, begin:begin + n_e].contiguous().cpu()
        B = wl.B[begin:begin + n_e].contiguous().cpu()
        off = torch.tensor([n_e], dtype=torch.int32)
        if wl.kind == "bf16":
            return lambda: oracle.wgrad_rows_bf16(A, B, off, 0, np.arange(r))
        sa = wl.sfa[begin // 128:(begin + n_e) // 128, :r].contiguous().cpu()
        sb = wl.sfb[begin // 128:(begin + n_e) // 128].contiguous().cpu()
        return lambda: oracle.wgrad_rows_fp8(A, sa, B, sb, off, 0, np.arange(r))
    t0 = time.perf_counter()
    take(rows)()                                            # calibration: one row per thread
    per_row = (time.perf_counter() - t0) / rows
    rows = int(min(wl.hidden, max(rows, target_seconds / max(per_row, 1e-9))))
    call = take(rows)
    del wl
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    call()
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * workloads.config_spec(name, 1)["n"] * n_e
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"expert {e} ({n_e} tokens) rows 0..{rows - 1}, all N columns of the {name} workload: "
                      f"{flops:.3e} FLOP in {dt:.1f} s (fp64 C oracle, OpenMP over rows)",
            "seconds": dt}


def run_mfma_ceiling(iters: int = 20000):
    """What this board's MFMAs sustain on the workloads' own operand values (kgw_mfma_ceiling):
    bf16 MFMA on N(0,1)*0.02 bf16 values (the balanced workload's distribution), bf16 MFMA on
    e4m3 codes converted to bf16 (the exact fp8 path's operands), the scaled fp8 MFMA on the
    same codes (the native path) and the scaled MFMA's FP4 mode on uniformly random e2m1 codes
    (the FP4 line's operands), each from the seeded generators of those workloads.  MFMA power
    depends on the data and the chip lowers its clock past its power limit, so these rates,
    with the clock they ran at, bound what any kernel can reach on such operands."""
    import torch
    import grouped_gemm_expert_offsets_amd as kgw
    import workloads
    g = torch.Generator(device="cuda").manual_seed(1)
    bf = workloads.randn_bf16((1024, 8192), 0.02, g, "cuda")
    x = workloads.randn_bf16((1024, 8192), 1.0, g, "cuda")
    codes, _ = workloads.quantize_token_blocks(x, token_axis=1)
    fp4 = torch.randint(0, 256, (1024, 8192), generator=g, device="cuda", dtype=torch.uint8)
    out = {}
    for name, src, kind, peak in (("bf16 MFMA, N(0,1)*0.02 bf16 operands", bf, 0, PEAK_BF16_TFLOPS),
                                  ("bf16 MFMA, e4m3 codes as bf16 (exact fp8 path)", codes, 1, PEAK_BF16_TFLOPS),
                                  ("scaled fp8 MFMA, e4m3 codes (native fp8 path)", codes, 2, PEAK_FP8_TFLOPS),
                                  ("scaled FP4 MFMA, uniformly random e2m1 codes (FP4 path)", fp4, 3,
                                   PEAK_FP4_TFLOPS)):
        for _ in range(3):
            kgw.kgw_mfma_ceiling(src, kind, iters=iters // 4)
        tflops, ghz = kgw.kgw_mfma_ceiling(src, kind, iters=iters)
        out[name] = {"tflops": round(tflops, 1), "clock_ghz": round(ghz, 3), "frac_of_peak": round(tflops / peak, 4)}
    del bf, x, codes, fp4
    torch.cuda.empty_cache()
    return out


# The secondary measurements that `--line` runs alone: (steps, warmup, min_warm_s) -> result.
LINES = {
    "fp4": lambda k, w, t: run_fp4(k, w, t),
    "mgrouped_nt": lambda k, w, t: run_mgrouped("nt", k, w, t),
    "mgrouped_nn": lambda k, w, t: run_mgrouped("nn", k, w, t),
    "mgrouped_fp8_nt": lambda k, w, t: run_mgrouped_fp8("nt", k, w, t),
    "mgrouped_fp8_nn": lambda k, w, t: run_mgrouped_fp8("nn", k, w, t),
    "quantize_fp8_A": lambda k, w, t: run_quantize(1, k, w, t),
    "quantize_fp8_B": lambda k, w, t: run_quantize(0, k, w, t),
    "quantize_fp4_A": lambda k, w, t: run_quantize(1, k, w, t, fp4=True),
    "quantize_fp4_B": lambda k, w, t: run_quantize(0, k, w, t, fp4=True),
}


def cpu_baseline(target_seconds: float):
    """The CPU oracle on a bounded sample of every configuration (about `target_seconds` in
    all), plus a one-thread sample of the balanced workload; the headline's is the top level."""
    import oracle
    per = {}
    names = ["tiny", "balanced", "skewed", "fp8", "many_small"]
    for name in names:
        per[name] = _oracle_sample(name, target_seconds / (len(names) - 1))
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        one = _oracle_sample("balanced", max(1.0, target_seconds / 20))
    finally:
        oracle.set_num_threads(threads)
    head = dict(per[HEADLINE])
    head["per_config"] = {k: {kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                          for k, v in per.items()}
    head["single_thread"] = {k: v for k, v in one.items() if k != "kind"}
    return head


def copy_calibration(gib: float = 1.0):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = int(gib * (1 << 30)) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 2, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="the headline's warm-up runs at least this long (clock settling)")
    ap.add_argument("--secondary-warm-seconds", type=float, default=0.2)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--native-fp8", action="store_true", help="time kgw_wgrad_fp8_native for fp8 workloads")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--line", choices=sorted(LINES),
                    help="run only this secondary measurement and print its result (for profiling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the K-grouped wgrad kernel runs on one device and this build has "
              "no multi-GPU path (expert parallelism would run the same kernel per GPU on its local experts).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import grouped_gemm_expert_offsets_amd as kgw
    kgw.load_library()
    torch.cuda.set_device(0)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.line:
        print(json.dumps(LINES[args.line](args.steps, args.warmup, args.warmup_seconds)), flush=True)
        return

    head = run_workload(args.workload, args.steps, args.warmup, native=args.native_fp8,
                        min_warm_s=args.warmup_seconds)
    import workloads
    spec = workloads.config_spec(args.workload, 1)
    kind = spec["kind"]
    traffic, traffic_src = profile_traffic(head["workload"], kind)
    peak = PEAK_FP8_TFLOPS if kind == "fp8" else PEAK_BF16_TFLOPS
    value = head["flops_per_launch"] / (head["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": head["warmup_launches"],
        "warmup_seconds": round(head["warmup_seconds"], 3),
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if kind == "fp8" else "bf16",
        "data": "synthetic (seeded; shapes and count distributions of the pages' MoE workloads)",
        "config": {
            "workload": workloads.DESCRIPTIONS[args.workload],
            "entry_point": ("kgw_wgrad_bf16" if kind == "bf16" else
                            "kgw_wgrad_fp8_native" if args.native_fp8 else "kgw_wgrad_fp8"),
            "num_experts": len(spec["counts"]),
            "hidden": spec["hidden"],
            "n": spec["n"],
            "tokens_sum": int(sum(spec["counts"])),
            "counts": spec["counts"] if len(spec["counts"]) <= 32 else "see workloads.config_spec",
            "seed": 1,
            "out_dtype": str(spec["out_dtype"]).replace("torch.", ""),
            "accumulate": spec["accumulate"],
            "parallelism": "single GPU",
        },
        "frac_of_mfma_peak": value / peak,
        "roofline": {
            "bound": "mfma",
            "achieved": head["tflops"],
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": head["tflops"] / peak,
            "traffic": traffic,
            "traffic_source": traffic_src,
            "algorithmic_bytes": head["algorithmic_bytes"],
            "kernel": ("wgrad_bf16_kernel" if kind == "bf16" else
                       "wgrad_fp8_native_kernel" if args.native_fp8 else "wgrad_fp8_kernel"),
            "launch_ms_mean": head["launch_ms_mean"],
            "launch_ms_min": head["launch_ms_min"],
            "launch_ms_max": head["launch_ms_max"],
        },
        "kernel_source_hash": kernel_source_hash(KERNEL_SOURCES[kind]),
    }
    if kind == "fp8" and not args.native_fp8:
        # the exact kernel multiplies on the bf16 MFMA: its own rate ceiling is the bf16 peak
        line["roofline"]["frac_of_bf16_mfma_peak"] = head["tflops"] / PEAK_BF16_TFLOPS
    if not args.no_secondary:
        sec = []
        sec_steps, sec_warm = max(5, args.steps // 5), 2

        def add(r):
            sec.append({k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})

        for name, native, block in (("balanced", False, 128), ("skewed", False, 128), ("fp8", True, 128),
                                    ("fp8", False, 32), ("fp8", True, 32), ("many_small", False, 128),
                                    ("tiny", False, 128)):
            if name == args.workload and native == args.native_fp8 and block == 128:
                continue
            steps = sec_steps * 10 if name in ("balanced", "tiny") else sec_steps
            add(run_workload(name, steps, sec_warm, native=native, min_warm_s=args.secondary_warm_seconds,
                             scale_block=block))
        for layout in (("k", "k"), ("m", "n"), ("m", "k")):
            add(run_workload("fp8", sec_steps, sec_warm, min_warm_s=args.secondary_warm_seconds, layout=layout))
        add(run_flushed("balanced", 30, 50))
        add(run_fp4(sec_steps, sec_warm, args.secondary_warm_seconds))
        for layout in ("nt", "nn"):
            add(run_mgrouped(layout, sec_steps, sec_warm, args.secondary_warm_seconds))
        for layout in ("nt", "nn"):
            add(run_mgrouped_fp8(layout, sec_steps, sec_warm, args.secondary_warm_seconds))
        for fp4 in (False, True):
            for axis in (1, 0):
                add(run_quantize(axis, sec_steps, sec_warm, args.secondary_warm_seconds, fp4=fp4))
        line["secondary"] = sec
        line["mfma_ceiling"] = run_mfma_ceiling()
        if kind == "fp8" and not args.native_fp8:
            ceil = line["mfma_ceiling"]["bf16 MFMA, e4m3 codes as bf16 (exact fp8 path)"]["tflops"]
            line["roofline"]["frac_of_measured_mfma_ceiling"] = head["tflops"] / ceil
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
