"""GPU parity of the m-grouped GEMM (forward "nt" / dgrad "nn") against the CPU oracle.

Groups are 128-row aligned, so some 256-row output tiles hold two groups (the kernel's two-pass
path) and some rows belong to no group (left untouched).  Integer-valued operands make every
fp32 partial sum exact: those cases are compared bit for bit; Gaussian cases use the fp32 /
bf16 tolerances of the other parity tests.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, assert_fp32_close, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
# group boundaries at 128, 512, 512, 768: tiles 0 (groups 0|1), 2 (3|4) straddle; 128 pad rows
COUNTS = [128, 384, 0, 256, 640]
PAD = 128


def run(wl, grouping, out, accumulate=False):
    kw = {"offsets": wl.offsets} if grouping == "offsets" else {"m_indices": wl.m_indices}
    kgw.kgw_mgrouped_bf16(wl.A, wl.W, layout=wl.layout, out=out, accumulate=accumulate, **kw)
    torch.cuda.synchronize()
    return out


def reference(wl):
    return oracle.mgrouped_bf16(wl.A.cpu(), wl.W.cpu(), m_indices=wl.m_indices.cpu(), layout=wl.layout)


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("grouping", ["offsets", "m_indices"])
@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_integer_bit_exact(layout, grouping, accumulate):
    wl = workloads.make_mgrouped(COUNTS, 192, 264, layout, seed=101, device=DEV, pad_rows=PAD, integer_range=4)
    M = wl.M
    if accumulate:
        g = torch.Generator(device=DEV).manual_seed(102)
        c0 = torch.randint(-8, 9, (M, 264), generator=g, device=DEV, dtype=torch.int32).float()
    else:
        c0 = torch.full((M, 264), float("nan"), device=DEV)
    out = run(wl, grouping, c0.clone(), accumulate)
    ref = reference(wl)
    valid = ~np.isnan(ref[:, 0])
    exp = ref + to_f64(c0) if accumulate else ref
    got = to_f64(out)
    assert np.array_equal(got[valid], exp[valid])
    # rows of no group are left as they were (NaN or the initial values)
    assert torch.equal(out[~torch.from_numpy(valid).to(DEV)].isnan(), c0[~torch.from_numpy(valid).to(DEV)].isnan())
    if accumulate:
        assert np.array_equal(got[~valid], to_f64(c0)[~valid])


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_random_against_oracle(layout, out_dtype):
    wl = workloads.make_mgrouped(COUNTS, 448, 392, layout, seed=103, device=DEV, pad_rows=PAD)
    out = torch.full((wl.M, 392), float("nan"), device=DEV, dtype=out_dtype)
    run(wl, "offsets", out)
    ref = reference(wl)
    valid = ~np.isnan(ref[:, 0])
    got = to_f64(out)
    assert np.all(np.isnan(got[~valid]))
    if out_dtype == torch.float32:
        assert_fp32_close(got[valid][None], ref[valid][None], f"mgrouped {layout} fp32")
    else:
        assert_bf16_close(got[valid][None], ref[valid][None], f"mgrouped {layout} bf16")


def test_two_group_tile_matches_single_group_runs():
    # a tile whose halves belong to groups 0 and 1 equals the two halves computed alone
    wl = workloads.make_mgrouped([128, 128], 256, 256, "nt", seed=104, device=DEV)
    both = run(wl, "offsets", torch.empty((256, 256), device=DEV))
    for h in (0, 1):
        sub = workloads.MGroupedWorkload(counts=[128], K=256, N=256, layout="nt",
                                         A=wl.A[128 * h:128 * (h + 1)].contiguous(), W=wl.W[h:h + 1].contiguous(),
                                         offsets=torch.tensor([128], dtype=torch.int32, device=DEV))
        one = run(sub, "offsets", torch.empty((128, 256), device=DEV))
        assert torch.equal(both[128 * h:128 * (h + 1)], one)


def test_k_zero_and_unknown_group_ids():
    wl = workloads.make_mgrouped([128, 256], 64, 64, "nn", seed=105, device=DEV, pad_rows=128)
    idx = wl.m_indices.clone()
    idx[128:256] = 7                     # ids outside [0, E): no group
    out = torch.full((wl.M, 64), float("nan"), device=DEV)
    kgw.kgw_mgrouped_bf16(wl.A, wl.W, m_indices=idx, layout="nn", out=out)
    torch.cuda.synchronize()
    ref = oracle.mgrouped_bf16(wl.A.cpu(), wl.W.cpu(), m_indices=idx.cpu(), layout="nn")
    valid = ~np.isnan(ref[:, 0])
    assert valid.sum() == 256 and np.all(np.isnan(to_f64(out)[~valid]))
    assert_fp32_close(to_f64(out)[valid][None], ref[valid][None], "unknown ids")
    # K == 0: rows of a group become +0.0, others untouched
    A0 = torch.empty((wl.M, 0), dtype=torch.bfloat16, device=DEV)
    W0 = torch.empty((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    out0 = torch.full((wl.M, 64), float("nan"), device=DEV)
    kgw.kgw_mgrouped_bf16(A0, W0, offsets=wl.offsets, layout="nn", out=out0)
    torch.cuda.synchronize()
    assert torch.all(out0[:384] == 0) and not torch.signbit(out0[:384]).any() and torch.all(out0[384:].isnan())


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_full_layer_sampled_rows(layout):
    # the fp8 workload's layer (32 local experts, n_e = roundup128(8192 * U(0.7, 1.3))):
    # forward X (T, 7168) @ W^T with W (32, 4096, 7168); dgrad dY (T, 4096) @ W (32, 4096, 7168)
    counts = workloads.counts_uniform(32, 8192, 128, 1)
    K, N = (7168, 4096) if layout == "nt" else (4096, 7168)
    wl = workloads.make_mgrouped(counts, K, N, layout, seed=1, device=DEV)
    out = run(wl, "offsets", torch.empty((wl.M, N), dtype=torch.bfloat16, device=DEV))
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 127, 128, wl.M - 1], rng.integers(0, wl.M, 12)]))
    groups = oracle.row_groups_from_offsets(wl.offsets.cpu(), wl.M)[rows]
    ref = oracle.mgrouped_bf16(wl.A.cpu()[torch.from_numpy(rows)], wl.W.cpu(), m_indices=groups, layout=layout)
    got = to_f64(out[torch.from_numpy(rows).to(DEV)])
    assert_bf16_close(got[None], ref[None], f"full {layout}", rms=np.array([np.sqrt(np.mean(ref * ref))]))
