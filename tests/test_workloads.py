"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import workloads


def test_tiny_counts():
    assert workloads.counts_tiny() == [256, 0, 512, 256]
    assert workloads.offsets_from_counts([256, 0, 512, 256]).tolist() == [256, 256, 768, 1024]


def test_balanced_counts_are_aligned_and_in_range():
    for seed in (1, 2, 101):
        c = workloads.counts_uniform(8, 4096, 256, seed)
        assert len(c) == 8 and all(x % 256 == 0 for x in c)
        assert all(int(np.ceil(4096 * 0.7)) <= x <= 4096 * 1.3 + 255 for x in c)
    assert workloads.counts_uniform(8, 4096, 256, 1) == [4352, 5376, 3328, 5376, 3840, 4096, 5120, 4096]


def test_skewed_counts():
    for seed in (1, 101, 202):
        c = workloads.counts_skewed(seed)
        assert len(c) == 32 and all(x % 256 == 0 for x in c)
        assert sum(c) <= 262144 and c.count(0) >= 4
    c = workloads.counts_skewed(1)
    assert sum(c) == 158976 and max(c) == 34048


def test_fp8_counts():
    c = workloads.counts_uniform(32, 8192, 128, 1)
    assert all(x % 128 == 0 for x in c) and sum(c) == 264320


def test_many_small_counts():
    for seed in (1, 5, 101):
        c = workloads.counts_many_small(seed)
        assert len(c) == 256 and sum(c) == 65536 and all(x % 256 == 0 for x in c)
        assert c.count(0) == 102
    assert max(workloads.counts_many_small(1)) == 6656


def test_seeds_reproduce():
    a = workloads.make_workload("tiny", seed=4)
    b = workloads.make_workload("tiny", seed=4)
    assert torch.equal(a.A, b.A) and torch.equal(a.B, b.B)
    c = workloads.make_workload("tiny", seed=5)
    assert not torch.equal(a.A, c.A)


def test_fp8_quantiser_properties():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(16, 512, generator=g).to(torch.bfloat16)
    x[2, 128:256] = 0
    q, s = workloads.quantize_token_blocks(x, token_axis=1)
    assert q.shape == (16, 512) and q.dtype == torch.uint8 and s.shape == (4, 16)
    vals = q.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(vals).all() and vals.abs().max() <= 448
    assert s[1, 2].item() == 127  # all-zero block
    # dequantised value is within half an e4m3 step (relative 2^-4) of the bf16 input
    sc = torch.exp2(s.float() - 127).t().repeat_interleave(128, dim=1)
    deq = vals * sc
    err = (deq - x.float()).abs()
    assert torch.all(err <= x.float().abs() * 2.0 ** -4 + sc * 2.0 ** -9)
    # the block maximum uses the top binade: 224 <= amax/scale <= 448
    blk = (x.float().abs() / sc).reshape(16, 4, 128).amax(-1)
    nz = blk > 0
    assert torch.all(blk[nz] <= 448) and torch.all(blk[nz] > 224)


def test_integer_operands_exact():
    wl = workloads.make_operands([256, 256], 8, 16, "bf16", torch.float32, True, seed=1, integer_range=4)
    assert torch.equal(wl.A.float(), wl.A.float().round()) and wl.A.float().abs().max() <= 4
    assert wl.C0.shape == (2, 8, 16)


def test_mgrouped_inputs():
    wl = workloads.make_mgrouped([256, 0, 128], 64, 32, "nt", seed=2, pad_rows=128)
    assert wl.A.shape == (512, 64) and wl.W.shape == (3, 32, 64) and wl.A.dtype == torch.bfloat16
    assert wl.offsets.tolist() == [256, 256, 384]
    idx = wl.m_indices.tolist()
    assert idx[:256] == [0] * 256 and idx[256:384] == [2] * 128 and idx[384:] == [-1] * 128
    nn = workloads.make_mgrouped([128], 16, 8, "nn", seed=2)
    assert nn.W.shape == (1, 16, 8)
    again = workloads.make_mgrouped([256, 0, 128], 64, 32, "nt", seed=2, pad_rows=128)
    assert torch.equal(again.A, wl.A) and torch.equal(again.W, wl.W)


def test_fp4_random_codes_shapes():
    wl = workloads.make_fp4_operands([256, 0, 512], 24, 40, seed=3, random_codes=True)
    assert wl["A"].shape == (24, 384) and wl["B"].shape == (40, 384)
    assert wl["sfa"].shape == (24, 24) and wl["sfb"].shape == (24, 40)
    assert int(wl["sfa"].min()) >= 122 and int(wl["sfa"].max()) <= 132
    again = workloads.make_fp4_operands([256, 0, 512], 24, 40, seed=3, random_codes=True)
    assert torch.equal(again["A"], wl["A"]) and torch.equal(again["sfb"], wl["sfb"])
