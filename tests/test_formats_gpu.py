"""GPU parity of the scale-layout and output-form variants against the CPU oracle.

  * packed UE8M0 scale words (four 128-token blocks per int32) and 32-token
    (MX-style) blocks packed one word per 128 tokens, on both fp8 paths;
  * discrete per-expert outputs through a device pointer array (None entries
    skip their expert), one-pass and split-K, overwrite and accumulate;
  * the quantiser's packed outputs, byte for byte.

Integer-valued operands with power-of-two scales keep every product and
partial sum exact in fp32 (and inside the native MFMA's aligned group sums),
so those cases are compared bit for bit; Gaussian cases use the tolerances of
the other parity tests.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, assert_fp32_close, rel_frob, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
NATIVE_FP8_REL_FROB = 1e-4     # the native MFMA's in-group alignment; see test_parity_gpu.py


def nan_filled(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def fmt_block(fmt):
    return 32 if fmt == kgw.KGW_SCALES_PACKED_32 else 128


def scales_for(wl, fmt):
    """The workload's uint8 scales (one byte per fmt_block tokens) in layout fmt."""
    if fmt == kgw.KGW_SCALES_U8:
        return wl.sfa, wl.sfb
    sfa = workloads.pack_scale_words(wl.sfa)
    sfb = workloads.pack_scale_words(wl.sfb)
    if fmt == kgw.KGW_SCALES_PACKED_32:
        assert sfa.shape[0] == wl.tokens_sum // 128
    return sfa, sfb


def fp8_oracle(wl):
    return oracle.wgrad_fp8(wl.A.cpu(), wl.sfa.cpu(), wl.B.cpu(), wl.sfb.cpu(), wl.offsets.cpu(),
                            block=wl.scale_block)


def integer_fp8_case(counts, hidden, n, fmt, accumulate, seed):
    """Integers in [-4, 4] with random scales 2^j, -1 <= j <= 2, per scale block: exact in fp32."""
    wl = workloads.make_operands(counts, hidden, n, "fp8", torch.float32, accumulate, seed=seed, device=DEV,
                                 integer_range=4, scale_block=fmt_block(fmt))
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    wl.sfa = torch.randint(126, 130, wl.sfa.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    wl.sfb = torch.randint(126, 130, wl.sfb.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    return wl


FORMATS = [kgw.KGW_SCALES_PACKED, kgw.KGW_SCALES_PACKED_32]


# ----------------------------------------------------------------------------
# scale layouts
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("native", [False, True])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("accumulate", [False, True])
def test_scale_formats_integer_bit_exact(fmt, native, accumulate):
    # ragged M and N tails, an empty expert, a 128-token expert, 13 blocks of 128 (a partial
    # last packed word for the 128-token format)
    counts = [256, 0, 128, 896, 384]
    wl = integer_fp8_case(counts, 264, 400, fmt, accumulate, seed=81)
    sfa, sfb = scales_for(wl, fmt)
    out = wl.C0.clone() if accumulate else nan_filled((5, 264, 400), torch.float32)
    kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=fmt, native=native, out=out,
                         accumulate=accumulate)
    torch.cuda.synchronize()
    W = fp8_oracle(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


def test_packed_128_matches_byte_scales_bit_for_bit():
    # the packed layout carries the same bytes: both fp8 paths give identical results
    counts = [384, 0, 1152, 256]
    wl = workloads.make_operands(counts, 320, 272, "fp8", torch.float32, False, seed=82, device=DEV)
    sfa, sfb = scales_for(wl, kgw.KGW_SCALES_PACKED)
    for native in (False, True):
        a = kgw.kgw_wgrad_fp8_ex(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, native=native, out_dtype=torch.float32)
        b = kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED,
                                 native=native, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"native={native}"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mx32_random_exact_path(out_dtype):
    counts = [128, 0, 640, 384, 1024]
    wl = workloads.make_operands(counts, 328, 400, "fp8", out_dtype, False, seed=83, device=DEV, scale_block=32)
    sfa, sfb = scales_for(wl, kgw.KGW_SCALES_PACKED_32)
    out = nan_filled((5, 328, 400), out_dtype)
    kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED_32, out=out)
    torch.cuda.synchronize()
    ref = fp8_oracle(wl)
    if out_dtype == torch.float32:
        assert_fp32_close(to_f64(out), ref, "mx32 fp32")
    else:
        assert_bf16_close(to_f64(out), ref, "mx32 bf16")
    # reading the 32-token scales as if each covered 128 tokens must not pass
    wrong = oracle.wgrad_fp8(wl.A.cpu(), wl.sfa[::4].contiguous().cpu(), wl.B.cpu(), wl.sfb[::4].contiguous().cpu(),
                             wl.offsets.cpu(), block=128)
    assert rel_frob(wrong, ref) > 1e-2


def test_mx32_random_native_path_within_its_bound():
    counts = [128, 0, 640, 384, 1024]
    wl = workloads.make_operands(counts, 328, 400, "fp8", torch.float32, False, seed=84, device=DEV, scale_block=32)
    sfa, sfb = scales_for(wl, kgw.KGW_SCALES_PACKED_32)
    out = kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED_32,
                               native=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = fp8_oracle(wl)
    got = to_f64(out)
    assert np.all(got[1] == 0.0)
    for e in (0, 2, 3, 4):
        err = rel_frob(got[e], ref[e])
        assert err <= NATIVE_FP8_REL_FROB, f"expert {e}: {err:.2e}"


@pytest.mark.parametrize("native", [False, True])
def test_mx32_split_k_integer_bit_exact(native):
    counts = [4096, 0, 8192, 256]
    wl = integer_fp8_case(counts, 320, 384, kgw.KGW_SCALES_PACKED_32, False, seed=85)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts), fp8=True) > 0
    sfa, sfb = scales_for(wl, kgw.KGW_SCALES_PACKED_32)
    out = kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED_32,
                               native=native, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(out), fp8_oracle(wl))


def test_mx32_full_fp8_workload_sampled_rows():
    # the fp8 workload's shape (E=32, hidden 7168, n 4096) with 32-token scales, sampled rows
    spec = workloads.config_spec("fp8", 1)
    wl = workloads.make_operands(spec["counts"], spec["hidden"], spec["n"], "fp8", torch.bfloat16, False, seed=1,
                                 device=DEV, scale_block=32)
    sfa, sfb = scales_for(wl, kgw.KGW_SCALES_PACKED_32)
    out = kgw.kgw_wgrad_fp8_ex(wl.A, sfa, wl.B, sfb, wl.offsets, scale_format=kgw.KGW_SCALES_PACKED_32)
    torch.cuda.synchronize()
    A, B, sa, sb, off = wl.A.cpu(), wl.B.cpu(), wl.sfa.cpu(), wl.sfb.cpu(), wl.offsets.cpu()
    rows = np.array([0, 1, 255, 256, 3001, 7167])
    for e in (0, 13, 31):
        ref = oracle.wgrad_rows_fp8(A, sa, B, sb, off, e, rows, block=32)
        got = to_f64(out[e][torch.from_numpy(rows).to(DEV)])
        assert_bf16_close(got[None], ref[None], f"mx32 full expert {e}",
                          rms=np.array([np.sqrt(np.mean(ref * ref))]))


# ----------------------------------------------------------------------------
# discrete outputs (pointer array)
# ----------------------------------------------------------------------------
def _discrete(hidden, n, dtype, E, skip=(), fill=float("nan")):
    return [None if e in skip else torch.full((hidden, n), fill, dtype=dtype, device=DEV) for e in range(E)]


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_discrete_outputs_match_dense(kind, accumulate):
    counts = [256, 0, 768, 512, 256]
    dtype = torch.bfloat16
    wl = workloads.make_operands(counts, 296, 400, kind, dtype, accumulate, seed=86, device=DEV)
    dense = wl.C0.clone() if accumulate else nan_filled((5, 296, 400), dtype)
    outs = [wl.C0[e].clone() for e in range(5)] if accumulate else _discrete(296, 400, dtype, 5)
    outs[3] = None                                  # skipped expert
    if kind == "bf16":
        kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, dense, accumulate=accumulate)
        kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=outs, accumulate=accumulate)
    else:
        kgw.kgw_wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, dense, accumulate=accumulate)
        kgw.kgw_wgrad_fp8_ex(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, outs=outs, accumulate=accumulate)
    torch.cuda.synchronize()
    for e in (0, 1, 2, 4):
        assert torch.equal(outs[e].view(torch.int16), dense[e].view(torch.int16)), f"expert {e}"
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu()) if kind == "bf16" else fp8_oracle(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = np.stack([to_f64(outs[e]) for e in (0, 2, 4)])
    assert_bf16_close(got, ref[[0, 2, 4]], f"discrete {kind}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_discrete_outputs_other_dtypes(dtype):
    counts = [512, 256, 512]
    wl = workloads.make_operands(counts, 256, 264, "bf16", dtype, False, seed=87, device=DEV)
    outs = _discrete(256, 264, dtype, 3, skip=(1,))
    dense = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=dtype)
    kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=outs)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    for e in (0, 2):
        assert torch.equal(outs[e].view(bits), dense[e].view(bits)), f"expert {e}"
    if dtype == torch.float32:
        W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
        assert_fp32_close(np.stack([to_f64(outs[0]), to_f64(outs[2])]), W[[0, 2]], "discrete fp32")


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_discrete_outputs_split_k_integer_bit_exact(kind, accumulate):
    counts = [4096, 0, 8192, 256]
    wl = workloads.make_operands(counts, 320, 384, kind, torch.float32, accumulate, seed=88, device=DEV,
                                 integer_range=4)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts), fp8=kind == "fp8") > 0
    outs = [wl.C0[e].clone() for e in range(4)] if accumulate else _discrete(320, 384, torch.float32, 4)
    outs[2] = None
    if kind == "bf16":
        kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=outs, accumulate=accumulate)
        W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
    else:
        kgw.kgw_wgrad_fp8_ex(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, outs=outs, accumulate=accumulate)
        W = fp8_oracle(wl)
    torch.cuda.synchronize()
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    for e in (0, 1, 3):
        assert np.array_equal(to_f64(outs[e]), ref[e]), f"expert {e}"
    if not accumulate:
        assert not torch.signbit(outs[1]).any() and torch.all(outs[1] == 0)


def test_discrete_outputs_all_skipped_and_no_tokens():
    wl = workloads.make_operands([0, 0], 64, 64, "bf16", torch.float32, False, seed=89, device=DEV)
    kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=[None, None])
    outs = _discrete(64, 64, torch.float32, 2)
    kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=outs)
    torch.cuda.synchronize()
    for t in outs:
        assert torch.all(t == 0) and not torch.signbit(t).any()


def test_discrete_outputs_many_experts_mostly_empty():
    # 300 experts of one 256x256 tile each, 40 with tokens: enough items for a full grid,
    # where workgroups of their own zero-fill the empty experts.  Skipped (None) experts,
    # empty or not, take no work; every other empty expert is +0.0.
    E, hidden, n = 300, 256, 256
    rng = np.random.default_rng(90)
    counts = [0] * E
    for e in rng.choice(E, 40, replace=False):
        counts[e] = 256 * int(rng.integers(1, 4))
    wl = workloads.make_operands(counts, hidden, n, "bf16", torch.float32, False, seed=90, device=DEV,
                                 integer_range=4)
    skip = set(rng.choice(E, 30, replace=False).tolist())
    outs = _discrete(hidden, n, torch.float32, E, skip=skip)
    kgw.kgw_wgrad_bf16_ex(wl.A, wl.B, wl.offsets, outs=outs)
    torch.cuda.synchronize()
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
    for e in range(E):
        if e in skip:
            continue
        if counts[e]:
            assert np.array_equal(to_f64(outs[e]), W[e]), f"expert {e}"
        else:
            assert torch.all(outs[e] == 0) and not torch.signbit(outs[e]).any(), f"expert {e}"
    # the same call into one dense output: identical values, empty experts +0.0
    dense = nan_filled((E, hidden, n), torch.float32)
    kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, dense)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(dense), W)
    empty = torch.tensor([e for e in range(E) if not counts[e]], device=DEV)
    assert not torch.signbit(dense.index_select(0, empty)).any()


# ----------------------------------------------------------------------------
# quantiser scale layouts
# ----------------------------------------------------------------------------
def _spread_bf16(shape, token_axis, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    other = shape[0] if token_axis else shape[1]
    mag = torch.exp2(torch.randint(-30, 31, (other,), generator=g).float())
    x = x * (mag[:, None] if token_axis else mag[None, :])
    # a few non-finite values poison their own (32- or 128-token) blocks only
    flat = x.view(-1)
    flat[(torch.arange(5) * 7919) % flat.numel()] = float("nan")
    flat[1234 % flat.numel()] = float("inf")
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("fmt", [kgw.KGW_SCALES_PACKED, kgw.KGW_SCALES_PACKED_32])
@pytest.mark.parametrize("token_axis,shape", [(1, (264, 1664)), (1, (3, 640)), (0, (1664, 200)), (0, (640, 72))])
def test_quantizer_scale_formats_bit_exact(fmt, token_axis, shape):
    x = _spread_bf16(shape, token_axis, seed=90)
    q, s = kgw.kgw_quantize_fp8(x.to(DEV), token_axis, scale_format=fmt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_fp8_tokens(x, token_axis, block=fmt_block(fmt))
    assert np.array_equal(q.cpu().numpy(), q_ref), "e4m3 bytes"
    words = s.cpu().numpy()
    assert words.dtype == np.int32
    assert np.array_equal(words, oracle.pack_scales(s_ref)), "packed scale words"
    assert np.array_equal(oracle.unpack_scales(words, s_ref.shape[0]), s_ref)


@pytest.mark.parametrize("fmt", [kgw.KGW_SCALES_PACKED, kgw.KGW_SCALES_PACKED_32])
def test_quantizer_to_gemm_round_trip(fmt):
    # quantise on the device, multiply on the device, compare with the oracle on the same bytes
    counts = [128, 384, 0, 640]
    T = sum(counts)
    g = torch.Generator().manual_seed(91)
    a = torch.randn(200, T, generator=g).to(torch.bfloat16).to(DEV)
    b = torch.randn(T, 272, generator=g).to(torch.bfloat16).to(DEV)
    off = torch.from_numpy(workloads.offsets_from_counts(counts)).to(DEV)
    qa, sa = kgw.kgw_quantize_fp8(a, 1, scale_format=fmt)
    qb, sb = kgw.kgw_quantize_fp8(b, 0, scale_format=fmt)
    out = kgw.kgw_wgrad_fp8_ex(qa, sa, qb, sb, off, scale_format=fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nb = T // fmt_block(fmt)
    ua = oracle.unpack_scales(sa.cpu().numpy(), nb)
    ub = oracle.unpack_scales(sb.cpu().numpy(), nb)
    ref = oracle.wgrad_fp8(qa.cpu(), ua, qb.cpu(), ub, off.cpu(), block=fmt_block(fmt))
    assert_fp32_close(to_f64(out), ref, "quantise -> gemm")
