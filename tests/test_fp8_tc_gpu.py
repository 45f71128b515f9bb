"""GPU parity of the fp8 products in the operand layouts other than kgw_wgrad_fp8's default:

  * the k-grouped weight gradient with A stored M-major (tokens_sum, hidden) and / or B stored
    K-major (n, tokens_sum), or as per-expert K-contiguous blocks (ragged) -- the same logical
    operands as kgw_wgrad_fp8, stored by plain copies; the MFMAs see the same token sets in the
    same order as the default layout, so the results must be identical bit for bit, besides
    matching the oracle;
  * the m-grouped forward product with fp8 operands and one UE8M0 scale per 1x128 block
    along K (kgw_mgrouped_fp8), against the oracle's mgrouped_fp8.

Integer-valued operands with power-of-two scales 2^-1 .. 2^2 keep every product and partial
sum exact in fp32, so those cases are compared bit for bit (and pin which scale byte meets
which element); Gaussian block-quantised cases use the fp32 / bf16 tolerances of the other
parity tests.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, assert_fp16_close, assert_fp32_close, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
# (a_major, b_major): both token-contiguous; both token-major; A token-major, B token-contiguous;
# "r": per-expert K-contiguous blocks back to back (ragged)
LAYOUTS = [("k", "k"), ("m", "n"), ("m", "k"), ("r", "r")]


def nan_filled(shape, dtype=torch.float32):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def random_scales(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randint(126, 130, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)


def first_mismatch(got, ref):
    mism = np.argwhere(~((got == ref) | (np.isnan(got) & np.isnan(ref))))
    return "" if mism.size == 0 else (f"{len(mism)} mismatches, first {tuple(mism[0])}: "
                                      f"{got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}")


# ----------------------------------------------------------------------------
# weight gradient, other operand layouts
# ----------------------------------------------------------------------------
def fp8_oracle(wl):
    return oracle.wgrad_fp8(wl.A.cpu(), wl.sfa.cpu(), wl.B.cpu(), wl.sfb.cpu(), wl.offsets.cpu())


def run_layout(wl, layout, out=None, outs=None, accumulate=False, split_k=True, out_dtype=torch.float32):
    a_major, b_major = layout
    if a_major == "r":
        # expert e's A block (hidden, n_e) and B block (n, n_e), row-major, back to back
        off = [0] + wl.offsets.tolist()
        a = torch.cat([wl.A[:, off[e]:off[e + 1]].contiguous().reshape(-1) for e in range(len(off) - 1)])
        b = torch.cat([wl.B[off[e]:off[e + 1]].t().contiguous().reshape(-1) for e in range(len(off) - 1)])
        r = kgw.kgw_wgrad_fp8_ex(a, wl.sfa, b, wl.sfb, wl.offsets, a_major="k", b_major="k", ragged=True,
                                 hidden=wl.hidden, n=wl.n, out=out, outs=outs, out_dtype=out_dtype,
                                 accumulate=accumulate, split_k=split_k)
    else:
        a = wl.A.t().contiguous() if a_major == "m" else wl.A
        b = wl.B.t().contiguous() if b_major == "k" else wl.B
        r = kgw.kgw_wgrad_fp8_ex(a, wl.sfa, b, wl.sfb, wl.offsets, a_major=a_major, b_major=b_major, out=out,
                                 outs=outs, out_dtype=out_dtype, accumulate=accumulate, split_k=split_k)
    torch.cuda.synchronize()
    return r


def integer_wgrad_case(counts, hidden, n, accumulate, seed):
    wl = workloads.make_operands(counts, hidden, n, "fp8", torch.float32, accumulate, seed=seed, device=DEV,
                                 integer_range=4)
    wl.sfa = random_scales(wl.sfa.shape, seed + 1)
    wl.sfb = random_scales(wl.sfb.shape, seed + 2)
    return wl


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_integer_bit_exact(layout, accumulate):
    # ragged hidden and n tails, an empty expert, one- and odd-block experts (the K loop's
    # two-step remainder), 7 blocks
    counts = [256, 0, 128, 896, 384]
    wl = integer_wgrad_case(counts, 272, 400, accumulate, seed=201)
    out = wl.C0.clone() if accumulate else nan_filled((5, 272, 400))
    run_layout(wl, layout, out=out, accumulate=accumulate)
    W = fp8_oracle(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    msg = first_mismatch(to_f64(out), ref)
    assert not msg, msg


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_equals_default_layout_and_oracle(layout, out_dtype):
    counts = [384, 0, 1152, 256, 640]
    wl = workloads.make_operands(counts, 336, 400, "fp8", out_dtype, False, seed=202, device=DEV)
    base = kgw.kgw_wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out_dtype=out_dtype)
    out = run_layout(wl, layout, out=nan_filled((5, 336, 400), out_dtype))
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(out.view(bits), base.view(bits))
    ref = fp8_oracle(wl)
    if out_dtype == torch.float32:
        assert_fp32_close(to_f64(out), ref, f"fp8 {layout} fp32")
    elif out_dtype == torch.bfloat16:
        assert_bf16_close(to_f64(out), ref, f"fp8 {layout} bf16")
    else:
        assert_fp16_close(to_f64(out), ref, f"fp8 {layout} fp16")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_malformed_offsets_stay_in_bounds(layout):
    # decreasing and past-the-end offsets: wrong values allowed for those experts, but the call
    # completes without leaving the operands and the well-formed first expert is exact
    counts = [256, 256, 256]
    wl = integer_wgrad_case(counts, 272, 256, False, seed=205)
    good = oracle.wgrad_fp8(wl.A.cpu(), wl.sfa.cpu(), wl.B.cpu(), wl.sfb.cpu(), wl.offsets.cpu())
    wl.offsets = torch.tensor([256, 4096, 128], dtype=torch.int32, device=DEV)
    out = run_layout(wl, layout, out=nan_filled((3, 272, 256)))
    assert np.array_equal(to_f64(out[0]), good[0])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_split_k_integer_bit_exact(layout):
    counts = [4096, 0, 8192, 256]
    wl = integer_wgrad_case(counts, 320, 384, False, seed=203)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts), fp8=True) > 0
    out = run_layout(wl, layout, out=nan_filled((4, 320, 384)))
    one = run_layout(wl, layout, out=nan_filled((4, 320, 384)), split_k=False)
    assert np.array_equal(to_f64(out), fp8_oracle(wl)) and torch.equal(out, one)


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_discrete_outputs(layout, accumulate):
    counts = [256, 0, 640, 384]
    wl = integer_wgrad_case(counts, 272, 256, accumulate, seed=204)
    c0 = wl.C0 if accumulate else None
    outs = [None if e == 3 else (c0[e].clone() if accumulate else nan_filled((272, 256))) for e in range(4)]
    run_layout(wl, layout, outs=outs, accumulate=accumulate)
    W = fp8_oracle(wl)
    ref = oracle.apply_output_mode(W, accumulate, to_f64(c0) if accumulate else None)
    for e in (0, 1, 2):
        msg = first_mismatch(to_f64(outs[e]), ref[e])
        assert not msg, f"expert {e}: {msg}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wgrad_layout_full_fp8_workload_every_element(layout):
    # the fp8 workload (E=32, hidden 7168, n 4096, n_e = roundup128(8192 * U(0.7, 1.3))):
    # every element written (NaN prefill), identical to the default layout, sampled rows
    # against the oracle
    spec = workloads.config_spec("fp8", 1)
    wl = workloads.make_operands(spec["counts"], spec["hidden"], spec["n"], "fp8", torch.bfloat16, False, seed=1,
                                 device=DEV)
    out = nan_filled((32, 7168, 4096), torch.bfloat16)
    run_layout(wl, layout, out=out, out_dtype=torch.bfloat16)
    assert not torch.isnan(out).any()
    base = kgw.kgw_wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    del base
    A, B, sa, sb, off = wl.A.cpu(), wl.B.cpu(), wl.sfa.cpu(), wl.sfb.cpu(), wl.offsets.cpu()
    rows = np.array([0, 255, 256, 4095, 7167])
    for e in (0, 31):
        ref = oracle.wgrad_rows_fp8(A, sa, B, sb, off, e, rows)
        got = to_f64(out[e][torch.from_numpy(rows).to(DEV)])
        assert_bf16_close(got[None], ref[None], f"{layout} full expert {e}",
                          rms=np.array([np.sqrt(np.mean(ref * ref))]))


# ----------------------------------------------------------------------------
# m-grouped forward product, fp8
# ----------------------------------------------------------------------------
# groups [0,128) [128,512) (empty) [512,896) [896,1408), 128 pad rows: output tiles 0 and 3
# hold two groups (the two-pass path), tile 5 half a group and half pad rows
COUNTS = [128, 384, 0, 384, 512]
PAD = 128


def run_mg(wl, grouping, out, accumulate=False, layout="nt"):
    """The product with W passed in `layout`: "nn" stores the same logical weight as (E, K, N)
    (a transposed copy; the scales are the same (E, K/128, N) bytes)."""
    kw = {"offsets": wl.offsets} if grouping == "offsets" else {"m_indices": wl.m_indices}
    W = wl.W if layout == "nt" else wl.W.transpose(1, 2).contiguous()
    kgw.kgw_mgrouped_fp8(wl.A, wl.sa, W, wl.sw, layout=layout, out=out, accumulate=accumulate, **kw)
    torch.cuda.synchronize()
    return out


def mg_oracle(wl, m_indices=None):
    idx = wl.m_indices if m_indices is None else m_indices
    return oracle.mgrouped_fp8(wl.A.cpu(), wl.sa.cpu(), wl.W.cpu(), wl.sw.cpu(), m_indices=idx.cpu())


@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("grouping", ["offsets", "m_indices"])
@pytest.mark.parametrize("K", [128, 384, 640])
def test_mgrouped_fp8_integer_bit_exact(K, grouping, accumulate, layout):
    N = 264 if layout == "nt" else 272          # nn: N a multiple of 16
    wl = workloads.make_mgrouped_fp8(COUNTS, K, N, seed=211, device=DEV, pad_rows=PAD, integer_range=4)
    wl.sa = random_scales(wl.sa.shape, 212)
    wl.sw = random_scales(wl.sw.shape, 213)
    M = wl.M
    if accumulate:
        g = torch.Generator(device=DEV).manual_seed(214)
        c0 = torch.randint(-8, 9, (M, N), generator=g, device=DEV, dtype=torch.int32).float()
    else:
        c0 = nan_filled((M, N))
    out = run_mg(wl, grouping, c0.clone(), accumulate, layout)
    ref = mg_oracle(wl)
    valid = ~np.isnan(ref[:, 0])
    assert valid.sum() == sum(COUNTS)
    exp = ref + to_f64(c0) if accumulate else ref
    got = to_f64(out)
    msg = first_mismatch(got[valid], exp[valid])
    assert not msg, msg
    # rows of no group are left as they were
    msg = first_mismatch(got[~valid], to_f64(c0)[~valid])
    assert not msg, f"rows of no group: {msg}"


@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_mgrouped_fp8_random_against_oracle(out_dtype, layout):
    wl = workloads.make_mgrouped_fp8(COUNTS, 896, 400, seed=215, device=DEV, pad_rows=PAD)
    out = run_mg(wl, "offsets", nan_filled((wl.M, 400), out_dtype), layout=layout)
    if layout == "nn":
        # the same logical product: identical to the forward layout bit for bit
        fwd = run_mg(wl, "offsets", nan_filled((wl.M, 400), out_dtype))
        bits = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(bits), fwd.view(bits))
    ref = mg_oracle(wl)
    valid = ~np.isnan(ref[:, 0])
    got = to_f64(out)
    assert np.all(np.isnan(got[~valid]))
    if out_dtype == torch.float32:
        assert_fp32_close(got[valid][None], ref[valid][None], "mgrouped fp8 fp32")
    elif out_dtype == torch.bfloat16:
        assert_bf16_close(got[valid][None], ref[valid][None], "mgrouped fp8 bf16")
    else:
        assert_fp16_close(got[valid][None], ref[valid][None], "mgrouped fp8 fp16")


def test_mgrouped_fp8_two_group_tile_matches_single_group_runs():
    wl = workloads.make_mgrouped_fp8([128, 128], 512, 256, seed=216, device=DEV)
    both = run_mg(wl, "offsets", torch.empty((256, 256), device=DEV))
    for h in (0, 1):
        sub = workloads.MGroupedWorkload(counts=[128], K=512, N=256, layout="nt",
                                         A=wl.A[128 * h:128 * (h + 1)].contiguous(), W=wl.W[h:h + 1].contiguous(),
                                         offsets=torch.tensor([128], dtype=torch.int32, device=DEV),
                                         sa=wl.sa[:, 128 * h:128 * (h + 1)].contiguous(),
                                         sw=wl.sw[h:h + 1].contiguous())
        one = run_mg(sub, "offsets", torch.empty((128, 256), device=DEV))
        assert torch.equal(both[128 * h:128 * (h + 1)], one)


def test_mgrouped_fp8_k_zero_and_unknown_group_ids():
    wl = workloads.make_mgrouped_fp8([128, 256], 256, 64, seed=217, device=DEV, pad_rows=128)
    idx = wl.m_indices.clone()
    idx[128:256] = 7                     # ids outside [0, E): no group
    out = nan_filled((wl.M, 64))
    kgw.kgw_mgrouped_fp8(wl.A, wl.sa, wl.W, wl.sw, m_indices=idx, out=out)
    torch.cuda.synchronize()
    ref = mg_oracle(wl, m_indices=idx)
    valid = ~np.isnan(ref[:, 0])
    assert valid.sum() == 256 and np.all(np.isnan(to_f64(out)[~valid]))
    assert_fp32_close(to_f64(out)[valid][None], ref[valid][None], "unknown ids")
    # K == 0: rows of a group become +0.0, others untouched
    A0 = torch.empty((wl.M, 0), dtype=torch.uint8, device=DEV)
    W0 = torch.empty((2, 64, 0), dtype=torch.uint8, device=DEV)
    s0 = torch.empty((0, wl.M), dtype=torch.uint8, device=DEV)
    w0 = torch.empty((2, 0, 64), dtype=torch.uint8, device=DEV)
    out0 = nan_filled((wl.M, 64))
    kgw.kgw_mgrouped_fp8(A0, s0, W0, w0, offsets=wl.offsets, out=out0)
    torch.cuda.synchronize()
    assert torch.all(out0[:384] == 0) and not torch.signbit(out0[:384]).any() and torch.all(out0[384:].isnan())


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_mgrouped_fp8_full_layer_every_element_sampled_rows(layout):
    # the fp8 workload's layer: X (T, 7168) @ W^T with W (32, 4096, 7168) -- forward, and the
    # same product with W stored (32, 7168, 4096) as dgrad reads it -- 32 local experts of
    # roundup128(8192 * U(0.7, 1.3)) rows; every element written (NaN prefill)
    counts = workloads.counts_uniform(32, 8192, 128, 1)
    wl = workloads.make_mgrouped_fp8(counts, 7168, 4096, seed=1, device=DEV)
    out = run_mg(wl, "offsets", nan_filled((wl.M, 4096), torch.bfloat16), layout=layout)
    assert not torch.isnan(out).any()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 127, 128, wl.M - 1], rng.integers(0, wl.M, 12)]))
    groups = oracle.row_groups_from_offsets(wl.offsets.cpu(), wl.M)[rows]
    r = torch.from_numpy(rows).to(DEV)
    ref = oracle.mgrouped_fp8(wl.A[r].cpu(), wl.sa[:, r].cpu(), wl.W.cpu(), wl.sw.cpu(),
                              m_indices=torch.from_numpy(groups))
    got = to_f64(out[r])
    assert_bf16_close(got[None], ref[None], "mgrouped fp8 full", rms=np.array([np.sqrt(np.mean(ref * ref))]))
