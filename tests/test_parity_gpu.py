"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Inputs are seeded and synthetic (workloads/); the oracle runs on host copies
of exactly the tensors the GPU consumed.  Small and mid sizes are compared
element by element, including mid-size cases with more work items than CUs on
both branches of the persistent schedule.  At full size every overwrite-mode
output starts as NaN and must come back without one; the balanced workload is
then compared element by element, the larger ones on sampled rows that the
oracle computes one by one, plus whole-tensor properties (zero-filled and
untouched experts) checked on every element.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, assert_fp16_close, assert_fp32_close, rel_frob, sample_rows, to_f64, FP32_REL_FROB

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"


def run_bf16(wl, out=None, out_dtype=None, accumulate=None):
    acc = wl.accumulate if accumulate is None else accumulate
    od = out_dtype or wl.out_dtype
    if out is None and acc:
        out = wl.C0.clone()
    res = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out, out_dtype=od, accumulate=acc)
    torch.cuda.synchronize()
    return res


# Accuracy bound of the native scaled fp8 MFMA entry point: the hardware keeps about 13 bits
# below the largest product of each K group, measured 1.5e-5 relative Frobenius on
# block-quantised Gaussian operands; the bound leaves a factor of ~6.
NATIVE_FP8_REL_FROB = 1e-4


def run_fp8(wl, out=None, out_dtype=None, accumulate=None, native=False):
    acc = wl.accumulate if accumulate is None else accumulate
    od = out_dtype or wl.out_dtype
    if out is None and acc:
        out = wl.C0.clone()
    fn = kgw.kgw_wgrad_fp8_native if native else kgw.kgw_wgrad_fp8
    res = fn(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out, out_dtype=od, accumulate=acc)
    torch.cuda.synchronize()
    return res


def oracle_dense(wl):
    off = wl.offsets.cpu()
    if wl.kind == "bf16":
        return oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), off)
    return oracle.wgrad_fp8(wl.A.cpu(), wl.sfa.cpu(), wl.B.cpu(), wl.sfb.cpu(), off)


def nan_filled(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


# ----------------------------------------------------------------------------
# small and mid sizes: every element
# ----------------------------------------------------------------------------
def test_tiny_config_every_element():
    wl = workloads.make_workload("tiny", seed=1, device=DEV)
    out = nan_filled((4, 256, 512), torch.float32)
    run_bf16(wl, out=out)
    ref = oracle_dense(wl)
    assert_fp32_close(to_f64(out), ref, "tiny")
    assert not torch.signbit(out[1]).any()  # empty expert written with +0.0


EXACT_CASES = [
    # (counts, hidden, n)
    ([256, 0, 512, 256], 256, 512),
    ([256, 0, 768, 512, 0, 256], 320, 392),      # ragged M and N tails, empties in the middle
    ([512, 256], 40, 24),                          # one partial tile
    ([0, 0, 256], 512, 520),
    ([1280], 264, 776),                            # single expert = plain GEMM, 20 K steps
]


@pytest.mark.parametrize("counts,hidden,n", EXACT_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("accumulate", [False, True])
def test_bf16_integer_inputs_bit_exact(counts, hidden, n, out_dtype, accumulate):
    wl = workloads.make_operands(counts, hidden, n, "bf16", out_dtype, accumulate, seed=11, device=DEV,
                                 integer_range=4)
    out = wl.C0.clone() if accumulate else nan_filled((len(counts), hidden, n), out_dtype)
    run_bf16(wl, out=out, accumulate=accumulate)
    W = oracle_dense(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    if out_dtype == torch.bfloat16:
        ref = oracle.round_to_bf16(ref)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("accumulate", [False, True])
def test_bf16_random_mid_size(out_dtype, accumulate):
    counts = [256, 0, 1280, 512, 768, 0, 256]
    wl = workloads.make_operands(counts, 576, 792, "bf16", out_dtype, accumulate, seed=21, device=DEV)
    out = wl.C0.clone() if accumulate else nan_filled((7, 576, 792), out_dtype)
    run_bf16(wl, out=out, accumulate=accumulate)
    W = oracle_dense(wl)
    C0 = to_f64(wl.C0) if accumulate else None
    ref = oracle.apply_output_mode(W, accumulate, C0)
    got = to_f64(out)
    if accumulate:
        for e in (1, 5):  # empty experts: untouched, bit for bit
            assert torch.equal(out[e].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                               wl.C0[e].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    if out_dtype == torch.float32:
        assert_fp32_close(got, ref, "mid fp32")
    else:
        rms = np.sqrt(np.mean(W * W, axis=(1, 2)))
        assert_bf16_close(got, ref, "mid bf16", rms=np.where(rms > 0, rms, np.sqrt(np.mean(ref * ref, axis=(1, 2)))))


def test_no_tokens_at_all():
    wl = workloads.make_operands([0, 0, 0], 64, 64, "bf16", torch.float32, True, seed=3, device=DEV)
    out = nan_filled((3, 64, 64), torch.float32)
    kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out, accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out)) and not torch.signbit(out).any()
    c0 = wl.C0.clone()
    kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, c0, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int32), wl.C0.view(torch.int32))


def test_deterministic_and_stream_ordered():
    wl = workloads.make_operands([512, 256, 0, 1024], 512, 512, "bf16", torch.float32, False, seed=5, device=DEV)
    a = run_bf16(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=torch.float32)
    s.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_validate_offsets_on_device():
    good = torch.tensor([256, 256, 768], dtype=torch.int32, device=DEV)
    kgw.kgw_validate_offsets(good, 768, 256)
    with pytest.raises(ValueError, match="first bad expert 1"):
        kgw.kgw_validate_offsets(torch.tensor([256, 128, 768], dtype=torch.int32, device=DEV), 768, 256)
    with pytest.raises(ValueError):
        kgw.kgw_validate_offsets(good, 1024, 256)


def test_check_offsets_flag_on_device():
    # the asynchronous device check flags the same first bad expert as the host check
    cases = [([256, 256, 768], 768, 256), ([256, 128, 768], 768, 256), ([256, 512], 768, 256),
             ([-256, 0], 0, 256), ([128, 384], 384, 128), ([128, 384], 384, 256), ([0, 0, 0], 0, 256)]
    rng = np.random.default_rng(3)
    big = np.cumsum(256 * rng.integers(0, 4, size=3000)).astype(np.int32)
    cases.append((big.tolist(), int(big[-1]), 256))
    broken = big.copy()
    broken[2500:] += 128                                           # expert 2500 loses alignment
    cases.append((broken.tolist(), int(broken[-1]), 256))
    for offs, T, align in cases:
        want = kgw.kgw_validate_offsets_host(offs, T, align)[1]
        flag = kgw.kgw_check_offsets(torch.tensor(offs, dtype=torch.int32, device=DEV), T, align)
        torch.cuda.synchronize()
        assert int(flag.item()) == want, (offs[:4], T, align)


def test_wgrad_wrapper_rejects_malformed_offsets():
    wl = workloads.make_operands([256, 256, 256], 64, 64, "bf16", torch.float32, False, seed=4, device=DEV)
    bad = torch.tensor([256, 128, 768], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="first bad expert 1"):
        kgw.wgrad(wl.A, wl.B, bad)
    out = kgw.wgrad(wl.A, wl.B, wl.offsets)
    torch.cuda.synchronize()
    assert_fp32_close(to_f64(out), oracle_dense(wl), "wgrad wrapper")


def test_malformed_offsets_stay_in_bounds():
    # decreasing / beyond tokens_sum offsets: wrong values allowed, but the call completes and
    # the experts whose ranges are well formed are still exact.
    wl = workloads.make_operands([256, 256, 256], 64, 64, "bf16", torch.float32, False, seed=4, device=DEV,
                                 integer_range=3)
    bad = torch.tensor([256, 4096, 100], dtype=torch.int32, device=DEV)
    out = kgw.kgw_wgrad_bf16(wl.A, wl.B, bad, out_dtype=torch.float32)
    torch.cuda.synchronize()
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), np.array([256, 512, 768], dtype=np.int32))
    assert np.array_equal(to_f64(out[0]), W[0])


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_more_experts_than_4096(kind):
    # 5000 experts, four with tokens (two past index 4096): the item list spans all of them,
    # the non-empty ones are bit-exact on integer inputs and every empty one is +0.0.
    E, hidden, n = 5000, 256, 64
    counts = [0] * E
    for e, c in ((0, 256), (1234, 512), (4097, 256), (4999, 768)):
        counts[e] = c
    wl = workloads.make_operands(counts, hidden, n, kind, torch.float32, False, seed=51, device=DEV,
                                 integer_range=4)
    out = nan_filled((E, hidden, n), torch.float32)
    if kind == "bf16":
        run_bf16(wl, out=out)
    else:
        run_fp8(wl, out=out)
    ne = [e for e, c in enumerate(counts) if c]
    mask = torch.ones(E, dtype=torch.bool, device=DEV)
    mask[torch.tensor(ne, device=DEV)] = False
    z = out[mask]
    assert torch.count_nonzero(z).item() == 0 and not torch.signbit(z).any().item()
    del z
    rows = np.arange(hidden)
    off = wl.offsets.cpu()
    for e in ne:
        if kind == "bf16":
            ref = oracle.wgrad_rows_bf16(wl.A.cpu(), wl.B.cpu(), off, e, rows)
        else:
            ref = oracle.wgrad_rows_fp8(wl.A.cpu(), wl.sfa.cpu(), wl.B.cpu(), wl.sfb.cpu(), off, e, rows)
        assert np.array_equal(to_f64(out[e]), ref), f"expert {e}"


# ----------------------------------------------------------------------------
# fp16 output (the cuDNN contract's third output type)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fp16_output_integer_bit_exact(kind, accumulate):
    counts = [256, 0, 512, 256]
    wl = workloads.make_operands(counts, 320, 272, kind, torch.float16, accumulate, seed=81, device=DEV,
                                 integer_range=4)
    out = wl.C0.clone() if accumulate else nan_filled((4, 320, 272), torch.float16)
    if kind == "bf16":
        run_bf16(wl, out=out)
    else:
        run_fp8(wl, out=out)
    W = oracle_dense(wl)
    ref = oracle.round_to_fp16(oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None))
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}"
    if accumulate:
        assert torch.equal(out[1].view(torch.int16), wl.C0[1].view(torch.int16))


@pytest.mark.parametrize("split_k", [False, True])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fp16_output_random(kind, split_k):
    counts = [4096, 0, 8192, 256] if split_k else [512, 0, 768, 256]
    wl = workloads.make_operands(counts, 320, 384, kind, torch.float16, False, seed=82, device=DEV)
    if split_k:
        assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts), fp8=kind == "fp8") > 0
    out = nan_filled((4, 320, 384), torch.float16)
    if kind == "bf16":
        kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out, split_k=split_k)
    else:
        kgw.kgw_wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out, split_k=split_k)
    torch.cuda.synchronize()
    ref = oracle_dense(wl)
    got = to_f64(out)
    assert np.all(got[1] == 0.0) and not np.any(np.signbit(got[1]))
    assert_fp16_close(got, ref, f"{kind} fp16 split_k={split_k}")


# ----------------------------------------------------------------------------
# split-K: few output tiles, many tokens -> chunked K with an fp32 workspace
# ----------------------------------------------------------------------------
SPLIT_COUNTS = [4096, 0, 8192, 256]     # E=4; partial M and N tiles below: 2 x 2 tiles per expert


def _split_case(kind, out_dtype, accumulate, seed, integer_range=None):
    wl = workloads.make_operands(SPLIT_COUNTS, 320, 384, kind, out_dtype, accumulate, seed=seed, device=DEV,
                                 integer_range=integer_range)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(SPLIT_COUNTS), fp8=kind == "fp8") > 0, "case must split"
    return wl


def _run(wl, out, path, split_k):
    if wl.kind == "bf16":
        kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out, accumulate=wl.accumulate, split_k=split_k)
    else:
        fn = kgw.kgw_wgrad_fp8_native if path == "native" else kgw.kgw_wgrad_fp8
        fn(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out, accumulate=wl.accumulate, split_k=split_k)
    torch.cuda.synchronize()


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_split_k_random(kind, out_dtype, accumulate):
    wl = _split_case(kind, out_dtype, accumulate, seed=61)
    out = wl.C0.clone() if accumulate else nan_filled((4, 320, 384), out_dtype)
    _run(wl, out, "exact", True)
    W = oracle_dense(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    if accumulate:
        assert torch.equal(out[1].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           wl.C0[1].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    else:
        assert np.all(got[1] == 0.0) and not np.any(np.signbit(got[1]))
    if out_dtype == torch.float32:
        assert_fp32_close(got, ref, f"split-K {kind} fp32")
    else:
        assert_bf16_close(got, ref, f"split-K {kind} bf16")


@pytest.mark.parametrize("kind,path", [("bf16", "exact"), ("fp8", "exact"), ("fp8", "native")])
def test_split_k_integer_bit_exact_and_same_as_one_pass(kind, path):
    wl = _split_case(kind, torch.float32, False, seed=62, integer_range=4)
    split = nan_filled((4, 320, 384), torch.float32)
    _run(wl, split, path, True)
    one = nan_filled((4, 320, 384), torch.float32)
    _run(wl, one, path, False)
    W = oracle_dense(wl)
    assert np.array_equal(to_f64(split), W)
    assert torch.equal(split, one)


def test_split_k_native_random_within_its_bound():
    wl = _split_case("fp8", torch.float32, False, seed=63)
    out = nan_filled((4, 320, 384), torch.float32)
    _run(wl, out, "native", True)
    W = oracle_dense(wl)
    got = to_f64(out)
    for e in (0, 2, 3):
        assert rel_frob(got[e], W[e]) <= NATIVE_FP8_REL_FROB
    assert np.all(got[1] == 0.0)


# ----------------------------------------------------------------------------
# fp8 block-scaled path
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fp8_random_small(out_dtype):
    counts = [128, 0, 384, 256, 640]
    wl = workloads.make_operands(counts, 264, 400, "fp8", out_dtype, False, seed=31, device=DEV)
    out = nan_filled((5, 264, 400), out_dtype)
    run_fp8(wl, out=out)
    ref = oracle_dense(wl)
    if out_dtype == torch.float32:
        assert_fp32_close(to_f64(out), ref, "fp8 fp32")
    else:
        assert_bf16_close(to_f64(out), ref, "fp8 bf16")


@pytest.mark.parametrize("native", [False, True])
@pytest.mark.parametrize("accumulate", [False, True])
def test_fp8_integer_inputs_with_scales_bit_exact(accumulate, native):
    counts = [256, 128, 0, 512]
    hidden, n = 200, 272
    wl = workloads.make_operands(counts, hidden, n, "fp8", torch.float32, accumulate, seed=41, device=DEV,
                                 integer_range=8)
    g = torch.Generator(device=DEV).manual_seed(42)
    # scales 2^j, |j| <= 2: every product and partial sum stays exact in fp32
    wl.sfa = torch.randint(125, 130, wl.sfa.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    wl.sfb = torch.randint(125, 130, wl.sfb.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    out = wl.C0.clone() if accumulate else nan_filled((4, hidden, n), torch.float32)
    run_fp8(wl, out=out, accumulate=accumulate, native=native)
    W = oracle_dense(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


@pytest.mark.parametrize("native", [False, True])
def test_fp8_every_code_dequantised_exactly(native):
    """A holds every finite e4m3fn code under per-row scales 2^-20 .. 2^20 and B is one-hot
    (the code of 1.0 on its diagonal, scale 2^0), so each output element is one dequantised
    A value: the device's dequantisation of every code at each of those scales must equal
    the oracle's bit for bit (fp32 output)."""
    T, hidden, n = 128, 256, 128
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 0x7F, 0xFF: NaN
    a = codes[(np.arange(hidden)[:, None] * T + np.arange(T)[None, :]) % len(codes)]
    b = np.zeros((T, n), np.uint8)
    b[np.arange(n), np.arange(n)] = 0x38                                             # e4m3fn 1.0
    sfa = (127 + (np.arange(hidden) % 41) - 20).astype(np.uint8)[None, :]
    sfb = np.full((1, n), 127, np.uint8)
    off = torch.tensor([T], dtype=torch.int32)
    assert len(np.unique(a)) == 254
    fn = kgw.kgw_wgrad_fp8_native if native else kgw.kgw_wgrad_fp8
    out = fn(torch.from_numpy(a).to(DEV), torch.from_numpy(sfa).to(DEV), torch.from_numpy(b).to(DEV),
             torch.from_numpy(sfb).to(DEV), off.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.wgrad_fp8(a, sfa, b, sfb, off)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


def test_fp8_native_random_small_within_its_bound():
    counts = [128, 0, 384, 256, 640]
    wl = workloads.make_operands(counts, 264, 400, "fp8", torch.float32, False, seed=31, device=DEV)
    out = nan_filled((5, 264, 400), torch.float32)
    run_fp8(wl, out=out, native=True)
    ref = oracle_dense(wl)
    got = to_f64(out)
    assert np.all(got[1] == 0.0)
    for e in (0, 2, 3, 4):
        err = rel_frob(got[e], ref[e])
        assert err <= NATIVE_FP8_REL_FROB, f"expert {e}: {err:.3e}"


# ----------------------------------------------------------------------------
# the persistent schedule at mid size, every element: more items than CUs
# ----------------------------------------------------------------------------
# The host picks the schedule from the counts (kgw_host.hip): with at least 1024
# tokens per expert on average ("long experts") the bf16 kernel remaps workgroups
# so each XCD owns a contiguous run of items, walks each expert's tiles in columns
# of four M tiles and takes odd rounds of the persistent stride in reverse; below
# that ("short experts") it uses columns of eight M tiles and no remap.  Both
# branches run here with more items than the 256 CUs hold, so every workgroup
# takes several rounds, and every element is compared with the oracle.
def _long_expert_counts(E, seed):
    counts = workloads.counts_uniform(E, 2048, 256, seed)
    assert sum(counts) >= 1024 * E, "long-expert branch"
    return counts


def _short_expert_counts(E, seed):
    rng = np.random.default_rng(seed)
    counts = (256 * rng.integers(0, 4, size=E)).tolist()      # 0 .. 768 tokens, about a quarter empty
    assert sum(counts) < 1024 * E, "short-expert branch"
    return counts


def _items(counts, hidden, n):
    return len(counts) * ((hidden + 255) // 256) * ((n + 255) // 256)


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("branch", ["long", "short"])
def test_bf16_multi_round_schedule_integer_every_element(branch, accumulate):
    if branch == "long":
        counts, hidden, n = _long_expert_counts(6, 7), 2048, 2048          # 384 items: 2 rounds
    else:
        counts, hidden, n = _short_expert_counts(40, 8), 2048, 1024        # 1280 items: 5 rounds
    assert _items(counts, hidden, n) > 256
    wl = workloads.make_operands(counts, hidden, n, "bf16", torch.float32, accumulate, seed=71, device=DEV,
                                 integer_range=4)
    out = wl.C0.clone() if accumulate else nan_filled((len(counts), hidden, n), torch.float32)
    run_bf16(wl, out=out, accumulate=accumulate)
    W = oracle_dense(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


@pytest.mark.parametrize("branch", ["long", "short"])
def test_bf16_multi_round_schedule_random_bf16_out(branch):
    if branch == "long":
        counts, hidden, n = _long_expert_counts(6, 17), 2048, 2048
    else:
        counts, hidden, n = _short_expert_counts(40, 18), 2048, 1024
    wl = workloads.make_operands(counts, hidden, n, "bf16", torch.bfloat16, False, seed=72, device=DEV)
    out = nan_filled((len(counts), hidden, n), torch.bfloat16)
    run_bf16(wl, out=out)
    W = oracle_dense(wl)
    assert_bf16_close(to_f64(out), oracle.apply_output_mode(W, False), f"{branch} bf16")


def _dynamic_counts(seed):
    # 32 experts, lognormal sizes in 256-token units, two empty, about 36k tokens: at least
    # 1024 tokens on average and 32 x 64 = 2048 tiles of 2048 x 2048, the dynamic schedule
    rng = np.random.default_rng(seed)
    units = np.maximum(1, np.rint(rng.lognormal(np.log(3.0), 1.0, size=32))).astype(np.int64)
    units = np.maximum(1, (units * 160) // units.sum())
    units[rng.choice(32, 2, replace=False)] = 0
    counts = (256 * units).tolist()
    assert sum(counts) >= 1024 * 32 and kgw.kgw_workspace_bytes(32, 2048, 2048, sum(counts)) == 256
    return counts


@pytest.mark.parametrize("accumulate", [False, True])
def test_bf16_dynamic_schedule_integer_every_element(accumulate):
    counts = _dynamic_counts(81 + accumulate)
    wl = workloads.make_operands(counts, 2048, 2048, "bf16", torch.float32, accumulate, seed=83, device=DEV,
                                 integer_range=4)
    out = wl.C0.clone() if accumulate else nan_filled((32, 2048, 2048), torch.float32)
    run_bf16(wl, out=out, accumulate=accumulate)
    W = oracle_dense(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


def test_bf16_dynamic_schedule_same_bits_as_static():
    # every tile is computed whole by one workgroup either way: identical outputs, with the
    # workspace (dynamic) and without (static), on random operands, bf16 output
    counts = _dynamic_counts(85)
    wl = workloads.make_operands(counts, 2048, 2048, "bf16", torch.bfloat16, False, seed=86, device=DEV)
    dyn = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=torch.bfloat16)
    sta = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=torch.bfloat16, split_k=False)
    again = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dyn.view(torch.int16), sta.view(torch.int16))
    assert torch.equal(dyn.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("native", [False, True])
def test_fp8_multi_round_schedule_integer_every_element(native):
    counts = workloads.counts_uniform(6, 2048, 128, 9)                    # 384 items: 2 rounds
    hidden, n = 2048, 2048
    wl = workloads.make_operands(counts, hidden, n, "fp8", torch.float32, False, seed=73, device=DEV,
                                 integer_range=8)
    g = torch.Generator(device=DEV).manual_seed(74)
    wl.sfa = torch.randint(125, 130, wl.sfa.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    wl.sfb = torch.randint(125, 130, wl.sfb.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    out = nan_filled((len(counts), hidden, n), torch.float32)
    run_fp8(wl, out=out, native=native)
    W = oracle_dense(wl)
    got = to_f64(out)
    mism = np.argwhere(got != W)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {W[tuple(mism[0])]}"


# ----------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration
# ----------------------------------------------------------------------------
# Overwrite-mode outputs start as NaN, so a tile the schedule drops or misplaces
# shows up in the whole-tensor NaN check; the values are then compared with the
# oracle on every element (balanced) or on sampled rows that the oracle computes
# one by one (the larger workloads).
def check_sampled(wl, out, experts, rows_per_expert=6, seed=0):
    Ah, Bh, off = wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu()
    if wl.kind == "fp8":
        sah, sbh = wl.sfa.cpu(), wl.sfb.cpu()
    for e in experts:
        rows = sample_rows(wl.hidden, rows_per_expert, seed + int(e))
        if wl.kind == "bf16":
            W = oracle.wgrad_rows_bf16(Ah, Bh, off, int(e), rows)
        else:
            W = oracle.wgrad_rows_fp8(Ah, sah, Bh, sbh, off, int(e), rows)
        C0 = to_f64(wl.C0[e][rows]) if wl.accumulate else None
        ref = oracle.apply_output_mode(W, wl.accumulate, C0)
        got = to_f64(out[e][torch.from_numpy(rows).to(out.device)])
        if out.dtype == torch.float32:
            err = rel_frob(got, ref)
            assert err <= FP32_REL_FROB, f"{wl.name} expert {e}: rel Frobenius {err:.3e}"
        else:
            rms = np.sqrt(np.mean(W * W)) if np.any(W) else np.sqrt(np.mean(ref * ref))
            assert_bf16_close(got[None], ref[None], f"{wl.name} expert {e}", rms=np.array([rms]))


def empty_experts(wl):
    return [e for e, c in enumerate(wl.counts) if c == 0]


def nonempty_experts(wl):
    return [e for e, c in enumerate(wl.counts) if c > 0]


def full_out(wl, dtype=None):
    return nan_filled((wl.num_experts, wl.hidden, wl.n), dtype or wl.out_dtype)


def assert_every_element_written(out):
    assert not torch.isnan(out).any().item(), "NaN left in the output: some elements were never written"


def assert_empty_experts_zero(wl, out):
    emp = empty_experts(wl)
    if not emp:
        return
    z = out.index_select(0, torch.tensor(emp, device=out.device))
    assert torch.count_nonzero(z).item() == 0 and not torch.signbit(z).any().item()


def test_full_balanced_bf16_every_element():
    wl = workloads.make_workload("balanced", seed=1, device=DEV)
    out = run_bf16(wl, out=full_out(wl))
    assert_every_element_written(out)
    W = oracle_dense(wl)
    rms = np.sqrt(np.mean(W * W, axis=(1, 2)))
    assert_bf16_close(to_f64(out), W, "balanced", rms=rms)


def test_full_skewed_accumulate():
    wl = workloads.make_workload("skewed", seed=1, device=DEV)
    out = run_bf16(wl)
    for e in empty_experts(wl):
        assert torch.equal(out[e].view(torch.int32), wl.C0[e].view(torch.int32)), f"expert {e} touched"
    check_sampled(wl, out, nonempty_experts(wl), rows_per_expert=4)


def test_full_skewed_overwrite_writes_every_element():
    # the skewed workload's schedule in overwrite mode: every element written, empties +0.0
    wl = workloads.make_workload("skewed", seed=1, device=DEV)
    out = run_bf16(wl, out=full_out(wl), accumulate=False)
    assert_every_element_written(out)
    assert_empty_experts_zero(wl, out)
    wl.accumulate = False
    check_sampled(wl, out, nonempty_experts(wl)[::3], rows_per_expert=3, seed=5)


def test_full_fp8():
    wl = workloads.make_workload("fp8", seed=1, device=DEV)
    out = run_fp8(wl, out=full_out(wl))
    assert_every_element_written(out)
    check_sampled(wl, out, nonempty_experts(wl)[::2], rows_per_expert=4)


def test_full_fp8_native_within_its_bound():
    wl = workloads.make_workload("fp8", seed=1, device=DEV)
    out = run_fp8(wl, out=full_out(wl, torch.float32), native=True)
    assert_every_element_written(out)
    Ah, Bh, sah, sbh, off = wl.A.cpu(), wl.B.cpu(), wl.sfa.cpu(), wl.sfb.cpu(), wl.offsets.cpu()
    for e in nonempty_experts(wl)[::4]:
        rows = sample_rows(wl.hidden, 4, e)
        ref = oracle.wgrad_rows_fp8(Ah, sah, Bh, sbh, off, e, rows)
        got = to_f64(out[e][torch.from_numpy(rows).to(out.device)])
        err = rel_frob(got, ref)
        assert err <= NATIVE_FP8_REL_FROB, f"expert {e}: {err:.3e}"


def test_full_many_small():
    wl = workloads.make_workload("many_small", seed=1, device=DEV)
    out = run_bf16(wl, out=full_out(wl))
    assert_every_element_written(out)
    assert_empty_experts_zero(wl, out)
    ne = nonempty_experts(wl)
    rng = np.random.default_rng(0)
    pick = sorted(set([ne[0], ne[-1]] + rng.choice(ne, 16, replace=False).tolist()))
    check_sampled(wl, out, pick, rows_per_expert=4)


def test_mfma_ceiling_helper_runs():
    # the measurement helper: a finite rate and a clock in the chip's range for every kind
    g = torch.Generator(device=DEV).manual_seed(9)
    x = workloads.randn_bf16((256, 4096), 1.0, g, DEV)
    codes, _ = workloads.quantize_token_blocks(x, token_axis=1)
    fp4 = torch.randint(0, 256, (256, 4096), generator=g, device=DEV, dtype=torch.uint8)
    for src, kind in ((x, 0), (codes, 1), (codes, 2), (fp4, 3)):
        tflops, ghz = kgw.kgw_mfma_ceiling(src, kind, iters=200, workgroups=256)
        assert 1.0 < tflops < 12000.0 and 0.3 < ghz < 3.5, (kind, tflops, ghz)
