"""GPU parity of the FP4 (e2m1, 32-token UE8M0 scales) weight gradient against the CPU oracle.

Operands come from the seeded generator (packed e2m1 bytes, byte scales); the scales go to the
kernel in the packed 32-token word layout.  The native instruction's block sums are exact for
e2m1 operands, so integer-valued cases compare bit for bit and random cases use the fp32 / bf16
tolerances of the other parity tests.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, assert_fp32_close, sample_rows, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"


def to_dev(wl):
    return (wl["A"].to(DEV), workloads.pack_scale_words(wl["sfa"]).to(DEV), wl["B"].to(DEV),
            workloads.pack_scale_words(wl["sfb"]).to(DEV), wl["offsets"].to(DEV))


def fp4_oracle(wl):
    return oracle.wgrad_fp4(wl["A"], wl["sfa"], wl["B"], wl["sfb"], wl["offsets"])


def misaligned_copy(t):
    # the same words at an address 4 bytes past a 16-byte boundary
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


# the scale words move by 16-byte loads when hidden and n are multiples of 4 and both scale
# arrays are 16-byte aligned, else by dword loads: both paths, bit for bit
@pytest.mark.parametrize("scale_path", ["16B", "dword_hidden", "dword_pointer"])
@pytest.mark.parametrize("accumulate", [False, True])
def test_integer_bit_exact_with_block_scales(accumulate, scale_path):
    # integers of e2m1 with random per-32-token scales 2^-1..2^2: exact in fp32
    counts = [256, 0, 512, 768, 256]
    H = 270 if scale_path == "dword_hidden" else 264
    wl = workloads.make_fp4_operands(counts, H, 392, seed=121, integer_range=6)
    g = torch.Generator().manual_seed(122)
    wl["sfa"] = torch.randint(126, 130, wl["sfa"].shape, generator=g, dtype=torch.int32).to(torch.uint8)
    wl["sfb"] = torch.randint(126, 130, wl["sfb"].shape, generator=g, dtype=torch.int32).to(torch.uint8)
    A, sa, B, sb, off = to_dev(wl)
    if scale_path == "dword_pointer":
        sa, sb = misaligned_copy(sa), misaligned_copy(sb)
        assert sa.data_ptr() % 16 == 4
    if accumulate:
        c0 = torch.randint(-8, 9, (5, H, 392), generator=g, dtype=torch.int32).float().to(DEV)
    else:
        c0 = torch.full((5, H, 392), float("nan"), device=DEV)
    out = c0.clone()
    kgw.kgw_wgrad_fp4(A, sa, B, sb, off, out=out, accumulate=accumulate)
    torch.cuda.synchronize()
    ref = oracle.apply_output_mode(fp4_oracle(wl), accumulate, to_f64(c0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_random_against_oracle(out_dtype):
    counts = [512, 256, 0, 1280, 256]
    wl = workloads.make_fp4_operands(counts, 328, 400, seed=123)
    A, sa, B, sb, off = to_dev(wl)
    out = torch.full((5, 328, 400), float("nan"), device=DEV, dtype=out_dtype)
    kgw.kgw_wgrad_fp4(A, sa, B, sb, off, out=out)
    torch.cuda.synchronize()
    ref = fp4_oracle(wl)
    got = to_f64(out)
    assert np.all(got[2] == 0.0)
    if out_dtype == torch.float32:
        assert_fp32_close(got, ref, "fp4 fp32")
    else:
        assert_bf16_close(got, ref, "fp4 bf16")


def test_split_k_and_discrete_outputs():
    counts = [4096, 0, 8192, 256]
    wl = workloads.make_fp4_operands(counts, 320, 384, seed=124, integer_range=4)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts), fp8=True) > 0
    A, sa, B, sb, off = to_dev(wl)
    split = kgw.kgw_wgrad_fp4(A, sa, B, sb, off, out_dtype=torch.float32)
    one = kgw.kgw_wgrad_fp4(A, sa, B, sb, off, out_dtype=torch.float32, split_k=False)
    outs = [torch.full((320, 384), float("nan"), device=DEV) for _ in range(4)]
    outs[2] = None
    kgw.kgw_wgrad_fp4(A, sa, B, sb, off, outs=outs)
    torch.cuda.synchronize()
    W = fp4_oracle(wl)
    assert np.array_equal(to_f64(split), W) and torch.equal(split, one)
    for e in (0, 1, 3):
        assert torch.equal(outs[e], one[e])


def test_full_fp8_workload_shape_sampled_rows():
    # the fp8 workload's shape (E=32, hidden 7168, n 4096) with FP4 operands (uniformly random
    # codes and scales drawn on the device); counts rounded to 256
    counts = workloads.counts_uniform(32, 8192, 256, 1)
    wl = workloads.make_fp4_operands(counts, 7168, 4096, seed=1, device=DEV, random_codes=True)
    A, sa, B, sb, off = to_dev(wl)
    out = kgw.kgw_wgrad_fp4(A, sa, B, sb, off)
    torch.cuda.synchronize()
    host = {k: wl[k].cpu() for k in ("A", "sfa", "B", "sfb", "offsets")}
    for e in (0, 17, 31):
        rows = sample_rows(7168, 4, e)
        ref = oracle.wgrad_rows_fp4(host["A"], host["sfa"], host["B"], host["sfb"], host["offsets"], e, rows)
        got = to_f64(out[e][torch.from_numpy(rows).to(DEV)])
        assert_bf16_close(got[None], ref[None], f"fp4 full expert {e}", rms=np.array([np.sqrt(np.mean(ref * ref))]))
