"""Parity of the on-device token-axis fp8 quantiser (kgw_quantize_fp8) with the CPU oracle.

Bytes are compared bit for bit: e4m3fn codes and UE8M0 scale bytes are integer outputs.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import helpers
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _spread_bf16(shape, token_axis, seed):
    """Gaussian values whose scale varies by 2^[-30, 30] across the non-token axis."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    other = shape[0] if token_axis else shape[1]
    mag = torch.exp2(torch.randint(-30, 31, (other,), generator=g).float())
    x = x * (mag[:, None] if token_axis else mag[None, :])
    return x.to(torch.bfloat16)


def _check(x_cpu, token_axis):
    q, s = kgw.kgw_quantize_fp8(x_cpu.to(DEV), token_axis)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_fp8_tokens(x_cpu, token_axis)
    s_got, q_got = s.cpu().numpy(), q.cpu().numpy()
    bad_s = np.argwhere(s_got != s_ref)
    assert bad_s.size == 0, f"{len(bad_s)} scale mismatches, first {tuple(bad_s[0])}"
    bad_q = np.argwhere(q_got != q_ref)
    assert bad_q.size == 0, (f"{len(bad_q)} byte mismatches, first {tuple(bad_q[0])}: "
                             f"{q_got[tuple(bad_q[0])]:#x} vs {q_ref[tuple(bad_q[0])]:#x}")


@pytest.mark.parametrize("shape", [(264, 640), (64, 128), (3, 1536)])
def test_tokens_along_columns_random(shape):
    _check(_spread_bf16(shape, 1, seed=71), 1)


@pytest.mark.parametrize("shape", [(384, 200), (1280, 72), (128, 8)])
def test_tokens_along_rows_random(shape):
    _check(_spread_bf16(shape, 0, seed=72), 0)


def test_every_bf16_value_under_a_fixed_scale():
    """Every finite bf16 value with |x| <= 448, shuffled into 128-token blocks whose maximum
    is 448 (scale 2^0), the whole row then scaled by 2^k for eight k from -40 to 30: each
    value meets the e4m3fn rounding at its block's scale (subnormals and ties included), on
    both token axes."""
    v = helpers.every_bf16_up_to(448.0)
    ks = (0, -12, 9, -40, 30, 1, -1, 5)
    rows = [helpers.anchored_blocks(v, 448.0, 128, 128, seed=200 + i) * 2.0 ** k for i, k in enumerate(ks)]
    x = torch.stack(rows).to(torch.bfloat16)                                 # (8, T): tokens along the columns
    _check(x.contiguous(), 1)
    _check(x.t().contiguous(), 0)


def _special_column(n=128):
    """One 128-token block per column kind: zeros, NaN, inf, subnormal bf16, -0, midpoints."""
    cols = []
    z = torch.zeros(n)
    cols.append(z.clone())                                         # all zero -> 127
    c = torch.randn(n); c[17] = float("nan"); cols.append(c)       # NaN block
    c = torch.randn(n); c[3] = float("-inf"); cols.append(c)       # inf block
    c = torch.full((n,), 2.0 ** -130) * torch.arange(1, n + 1); cols.append(c)   # tiny: clamps to 1
    c = -torch.zeros(n); c[0] = 1.0; cols.append(c)                # negative zeros
    # exact e4m3 midpoints at scale 2^0 (amax 448): ties must go to even
    mids = torch.tensor([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -6 + 2.0 ** -10, 240.0, 416.0, 232.0, 448.0])
    c = mids.repeat(n // len(mids)); cols.append(c)
    c = torch.randn(n) * 1e30; cols.append(c)                       # large magnitudes
    c = torch.randn(n) * 1e-30; cols.append(c)                      # small normal magnitudes
    return torch.stack(cols, dim=1)                                # (128, 8)


def test_special_blocks_both_axes():
    xb = _special_column().to(torch.bfloat16)                      # tokens along the rows
    _check(torch.cat([xb, xb], dim=0).contiguous(), 0)
    _check(torch.cat([xb, xb], dim=0).t().contiguous(), 1)


def test_rejects_bad_shapes():
    x = torch.zeros((64, 200), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        kgw.kgw_quantize_fp8(x, 1)                                 # 200 tokens: not a multiple of 128
    x = torch.zeros((128, 12), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        kgw.kgw_quantize_fp8(x, 0)                                 # 12 columns: not a multiple of 8


def test_full_size_fp8_operands_sampled():
    # the fp8 workload's operand shapes (hidden 7168, n 4096, tokens_sum 264320), sampled rows of
    # A and column slices of B against the oracle
    spec = workloads.config_spec("fp8", 1)
    T, H, N = sum(spec["counts"]), spec["hidden"], spec["n"]
    g = torch.Generator(device=DEV).manual_seed(73)
    A = torch.randn((H, T), generator=g, device=DEV).to(torch.bfloat16)
    qa, sa = kgw.kgw_quantize_fp8(A, 1)
    rows = np.array([0, 1, 777, 4096, H - 1])
    ref_q, ref_s = oracle.quantize_fp8_tokens(A[torch.from_numpy(rows).to(DEV)].cpu(), 1)
    assert np.array_equal(qa[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref_q)
    assert np.array_equal(sa[:, torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref_s)
    del A, qa, sa
    B = torch.randn((T, N), generator=g, device=DEV).to(torch.bfloat16)
    qb, sb = kgw.kgw_quantize_fp8(B, 0)
    for c0 in (0, 1984, N - 64):
        ref_q, ref_s = oracle.quantize_fp8_tokens(B[:, c0:c0 + 64].cpu().contiguous(), 0)
        assert np.array_equal(qb[:, c0:c0 + 64].cpu().numpy(), ref_q)
        assert np.array_equal(sb[:, c0:c0 + 64].cpu().numpy(), ref_s)


def test_quantised_operands_feed_the_fp8_wgrad():
    # end to end on the device: quantise bf16 A and B, then kgw_wgrad_fp8 on those bytes equals
    # the oracle's fp8 weight gradient of the same bytes
    counts = [256, 0, 384]
    wl = workloads.make_operands(counts, 192, 256, "bf16", torch.float32, False, seed=74, device=DEV)
    qa, sa = kgw.kgw_quantize_fp8(wl.A, 1)
    qb, sb = kgw.kgw_quantize_fp8(wl.B, 0)
    out = kgw.kgw_wgrad_fp8(qa, sa, qb, sb, wl.offsets, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.wgrad_fp8(qa.cpu(), sa.cpu(), qb.cpu(), sb.cpu(), wl.offsets.cpu())
    got = out.cpu().double().numpy()
    for e in (0, 2):
        err = np.linalg.norm(got[e] - ref[e]) / np.linalg.norm(ref[e])
        assert err <= 1e-5, f"expert {e}: {err:.2e}"
    assert np.all(got[1] == 0.0)
