"""kgw_wgrad_bf16_noalloc (the entry point that allocates nothing) against kgw_wgrad_bf16.

Two calls in a row through the C-ABI, the second on a smaller input: both split K (their
fp32 partials go to the library's fixed per-device scratch, the first call's leftovers
still in it when the second runs) and must equal kgw_wgrad_bf16 given a workspace, bit for
bit (same split plan, same kernels).  A shape that does not split runs in one pass, and
the largest split the plan makes on 256 CUs fills the scratch exactly.
Neither the binding nor the library may allocate through torch's allocator.
"""
import ctypes

import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
SCRATCH_BYTES = 64 << 20


def _noalloc_abi(wl, out, accumulate):
    lib = kgw.load_library()
    code = {torch.float32: kgw.KGW_OUT_FP32, torch.bfloat16: kgw.KGW_OUT_BF16, torch.float16: kgw.KGW_OUT_FP16}
    hidden, T = wl.A.shape
    st = lib.kgw_wgrad_bf16_noalloc(wl.A.data_ptr(), wl.B.data_ptr(), wl.offsets.data_ptr(), wl.num_experts, hidden,
                                    wl.n, T, out.data_ptr(), code[out.dtype], int(accumulate),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kgw.KGW_SUCCESS, kgw.kgw_status_string(st)


def _case(counts, hidden, n, out_dtype, accumulate, seed):
    return workloads.make_operands(counts, hidden, n, "bf16", out_dtype, accumulate, seed=seed, device=DEV)


def _compare(wl, out_dtype, accumulate, split_k=True):
    shape = (wl.num_experts, wl.hidden, wl.n)
    ref = wl.C0.clone() if accumulate else torch.full(shape, float("nan"), dtype=out_dtype, device=DEV)
    kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, ref, accumulate=accumulate, split_k=split_k)
    got = wl.C0.clone() if accumulate else torch.full(shape, float("nan"), dtype=out_dtype, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    _noalloc_abi(wl, got, accumulate)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(got.view(bits), ref.view(bits))
    return got


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_the_workspace_entry_point_two_calls(out_dtype, accumulate):
    big = _case([4096, 0, 8192, 256], 320, 384, out_dtype, accumulate, seed=91)
    small = _case([2048, 4096], 256, 256, out_dtype, accumulate, seed=92)
    for wl in (big, small):
        ws = kgw.kgw_workspace_bytes(wl.num_experts, wl.hidden, wl.n, wl.tokens_sum)
        assert 0 < ws <= SCRATCH_BYTES, "both calls must split K and fit the scratch"
    _compare(big, out_dtype, accumulate)
    got = _compare(small, out_dtype, accumulate)
    # and the second call's values against the oracle
    W = oracle.wgrad_bf16(small.A.cpu(), small.B.cpu(), small.offsets.cpu())
    ref = oracle.apply_output_mode(W, accumulate, small.C0.cpu().double().numpy() if accumulate else None)
    g = got.cpu().double().numpy()
    if out_dtype == torch.float32:
        err = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        assert err <= 1e-5, err
    else:
        assert np.all(np.abs(g - ref) <= 2 * oracle.bf16_ulp(np.maximum(np.abs(ref), 2.0 ** -8 *
                                                                        np.sqrt(np.mean(W * W)))))


def test_noalloc_one_pass_shape_and_scratch_bound():
    # a shape with enough tiles runs in one pass, as kgw_wgrad_bf16 does
    wl = _case([256, 0, 512, 256], 256, 512, torch.float32, False, seed=93)
    assert kgw.kgw_workspace_bytes(4, 256, 512, 1024) == 0
    _compare(wl, torch.float32, False)
    # split * tiles <= compute units, so on 256 CUs the partials of any split fit 64 MiB
    for E, H, N, T in ((1, 2048, 4096, 65536), (2, 2048, 2048, 32768), (1, 256, 256, 1 << 20),
                       (4, 1024, 1024, 65536), (16, 256, 256, 65536)):
        assert kgw.kgw_workspace_bytes(E, H, N, T) <= SCRATCH_BYTES
    big = _case([16384, 16384], 2048, 2048, torch.float32, False, seed=94)
    assert kgw.kgw_workspace_bytes(2, 2048, 2048, 32768) == SCRATCH_BYTES
    _compare(big, torch.float32, False)


def test_noalloc_dynamic_schedule_shape():
    # a shape on the dynamic schedule: its claim counters live in the scratch too
    rng = np.random.default_rng(95)
    counts = (256 * rng.integers(3, 8, size=32)).tolist()
    assert kgw.kgw_workspace_bytes(32, 2048, 2048, sum(counts)) == 256
    wl = _case(counts, 2048, 2048, torch.bfloat16, False, seed=96)
    _compare(wl, torch.bfloat16, False)
    small = _case([2048, 4096], 256, 256, torch.float32, True, seed=97)      # then a split-K call
    _compare(small, torch.float32, True)
