"""Parity of the on-device FP4 (e2m1) quantiser (kgw_quantize_fp4) with the CPU oracle.

Codes and UE8M0 scale bytes are integer outputs: compared bit for bit against
oracle.quantize_fp4_tokens (tokens along the columns; for tokens along the rows the oracle
quantises the transposed tensor, which is the layout the device writes).  Packed scales
are compared with the oracle's bytes packed four to a word by oracle.pack_scales.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import helpers
import oracle
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]
DEV = "cuda"
FORMATS = [kgw.KGW_SCALES_U8, kgw.KGW_SCALES_PACKED_32]


def _spread_bf16(shape, token_axis, seed):
    """Gaussian values whose scale varies by 2^[-30, 30] across the non-token axis."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    other = shape[0] if token_axis else shape[1]
    mag = torch.exp2(torch.randint(-30, 31, (other,), generator=g).float())
    x = x * (mag[:, None] if token_axis else mag[None, :])
    return x.to(torch.bfloat16)


def _check(x_cpu, token_axis, fmt):
    q, s = kgw.kgw_quantize_fp4(x_cpu.to(DEV), token_axis, scale_format=fmt)
    torch.cuda.synchronize()
    src = x_cpu if token_axis else x_cpu.t().contiguous()
    q_ref, s_ref = oracle.quantize_fp4_tokens(src)
    if fmt == kgw.KGW_SCALES_PACKED_32:
        s_ref = oracle.pack_scales(s_ref)
    s_got, q_got = s.cpu().numpy(), q.cpu().numpy()
    assert s_got.shape == s_ref.shape and q_got.shape == q_ref.shape
    bad_s = np.argwhere(s_got != s_ref)
    assert bad_s.size == 0, f"{len(bad_s)} scale mismatches, first {tuple(bad_s[0])}"
    bad_q = np.argwhere(q_got != q_ref)
    assert bad_q.size == 0, (f"{len(bad_q)} byte mismatches, first {tuple(bad_q[0])}: "
                             f"{q_got[tuple(bad_q[0])]:#x} vs {q_ref[tuple(bad_q[0])]:#x}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(264, 640), (64, 2048), (3, 2176), (70, 4224)])
def test_tokens_along_columns_random(shape, fmt):
    # ragged row blocks (not multiples of 16 or 64) and partial 2048-token chunks
    _check(_spread_bf16(shape, 1, seed=91), 1, fmt)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(384, 200), (1280, 72), (128, 8), (256, 136)])
def test_tokens_along_rows_random(shape, fmt):
    # column counts that leave partial 128-column tiles
    _check(_spread_bf16(shape, 0, seed=92), 0, fmt)


def _special_column(n=128):
    """One 32-token block per kind, four per column: zeros, NaN, inf, subnormal bf16, -0,
    exact e2m1 midpoints (ties to the even code), saturation at the block maximum."""
    blocks = []
    blocks.append(torch.zeros(32))                                           # all zero -> 127
    c = torch.randn(32); c[5] = float("nan"); blocks.append(c)               # NaN block
    c = torch.randn(32); c[9] = float("-inf"); blocks.append(c)              # inf block
    blocks.append(torch.full((32,), 2.0 ** -130) * torch.arange(1, 33))      # tiny: clamps to 1
    c = -torch.zeros(32); c[0] = 1.0; blocks.append(c)                       # negative zeros
    # amax 6 fixes the scale at 2^0: every midpoint 0.25 .. 5 is a tie
    mids = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                         0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.375, 0.625, 2.25, 2.75, 4.5, 5.5, 0.125, 1.125,
                         3.25, 3.75])
    blocks.append(mids)
    blocks.append(torch.randn(32) * 1e30)                                    # large magnitudes
    blocks.append(torch.randn(32) * 1e-30)                                   # small normal magnitudes
    col = torch.cat(blocks[:4])
    col2 = torch.cat(blocks[4:])
    return torch.stack([col, col2, col.flip(0), col2.flip(0), col * 3, col2 * 0.75, col2 * 1.5, -col2], dim=1)


@pytest.mark.parametrize("fmt", FORMATS)
def test_special_blocks_both_axes(fmt):
    xb = _special_column().to(torch.bfloat16)                                # (128, 8): tokens along rows
    _check(xb.contiguous(), 0, fmt)
    _check(xb.t().contiguous(), 1, fmt)


def _tie_neighbour_column():
    """Blocks whose maximum is 6 * 2^k (so the scale is 2^k) holding every e2m1 rounding
    midpoint 0.25 .. 5 times 2^k and the bf16 values one unit in the last place either
    side of it, both signs, for k = -3, 0 and 5: the encoder's tie and near-tie cases
    away from scale 1."""
    ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=torch.bfloat16)
    bits = ties.view(torch.int16)
    near = torch.cat([ties, (bits + 1).view(torch.bfloat16), (bits - 1).view(torch.bfloat16)]).float()
    vals = torch.cat([near, -near])                                          # 42 values
    blocks = []
    for k in (-3, 0, 5):
        for part in (vals[:31], vals[31:]):
            b = torch.zeros(32)
            b[0] = 6.0
            b[1:1 + len(part)] = part
            blocks.append(b * 2.0 ** k)
    col = torch.cat(blocks + [torch.zeros(32)] * 2)                          # 8 blocks = 256 tokens
    perm = torch.randperm(32, generator=torch.Generator().manual_seed(95))
    shuffled = col.view(8, 32)[:, perm].reshape(-1)
    return torch.stack([col, -col, shuffled, -shuffled, col.flip(0), shuffled.flip(0), col * 0.5, shuffled * 4],
                       dim=1)


@pytest.mark.parametrize("fmt", FORMATS)
def test_tie_neighbours_at_several_scales(fmt):
    xb = _tie_neighbour_column().to(torch.bfloat16)                          # (256, 8): tokens along rows
    assert torch.equal(xb.float(), _tie_neighbour_column())                  # every value exact in bf16
    _check(xb.contiguous(), 0, fmt)
    _check(xb.t().contiguous(), 1, fmt)


@pytest.mark.parametrize("fmt", FORMATS)
def test_every_bf16_value_under_a_fixed_scale(fmt):
    """Every finite bf16 value with |x| <= 6, shuffled into 32-token blocks whose maximum is
    6 (scale 2^0), the whole row then scaled by 2^k for eight k from -40 to 30: each value
    meets the e2m1 encoding at its block's scale, on both token axes."""
    v = helpers.every_bf16_up_to(6.0)
    ks = (0, -12, 9, -40, 30, 1, -1, 5)
    rows = [helpers.anchored_blocks(v, 6.0, 32, 256, seed=100 + i) * 2.0 ** k for i, k in enumerate(ks)]
    x = torch.stack(rows).to(torch.bfloat16)                                 # (8, T): tokens along the columns
    _check(x.contiguous(), 1, fmt)
    _check(x.t().contiguous(), 0, fmt)


def test_quantised_operands_feed_the_fp4_wgrad():
    # end to end on the device: quantise bf16 A (hidden, T) and B (T, n), then kgw_wgrad_fp4 on
    # those bytes equals the oracle's FP4 weight gradient of the same bytes
    counts = [256, 0, 512]
    g = torch.Generator(device=DEV).manual_seed(93)
    T, hidden, n = sum(counts), 192, 264
    A = torch.randn((hidden, T), generator=g, device=DEV).to(torch.bfloat16)
    B = torch.randn((T, n), generator=g, device=DEV).to(torch.bfloat16)
    qa, sa = kgw.kgw_quantize_fp4(A, 1)
    qb, sb = kgw.kgw_quantize_fp4(B, 0)
    off = torch.tensor(np.cumsum(counts), dtype=torch.int32, device=DEV)
    out = kgw.kgw_wgrad_fp4(qa, sa, qb, sb, off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.wgrad_fp4(qa.cpu(), oracle.unpack_scales(sa.cpu(), T // 32), qb.cpu(),
                           oracle.unpack_scales(sb.cpu(), T // 32), off.cpu())
    got = out.cpu().double().numpy()
    for e in (0, 2):
        err = np.linalg.norm(got[e] - ref[e]) / np.linalg.norm(ref[e])
        assert err <= 1e-5, f"expert {e}: {err:.2e}"
    assert np.all(got[1] == 0.0)


def test_full_size_fp4_operands_sampled():
    # the FP4 workload's operand shapes (hidden 7168, n 4096, 266,240 tokens): sampled rows
    # of A and column slices of B against the oracle
    T, H, N = 266240, 7168, 4096
    g = torch.Generator(device=DEV).manual_seed(94)
    A = torch.randn((H, T), generator=g, device=DEV).to(torch.bfloat16)
    qa, sa = kgw.kgw_quantize_fp4(A, 1, scale_format=kgw.KGW_SCALES_U8)
    rows = torch.tensor([0, 1, 777, 4096, H - 1], device=DEV)
    ref_q, ref_s = oracle.quantize_fp4_tokens(A[rows].cpu())
    assert np.array_equal(qa[rows].cpu().numpy(), ref_q)
    assert np.array_equal(sa[:, rows].cpu().numpy(), ref_s)
    del A, qa, sa
    B = torch.randn((T, N), generator=g, device=DEV).to(torch.bfloat16)
    qb, sb = kgw.kgw_quantize_fp4(B, 0)
    for c0 in (0, 1984, N - 64):
        ref_q, ref_s = oracle.quantize_fp4_tokens(B[:, c0:c0 + 64].t().contiguous().cpu())
        assert np.array_equal(qb[c0:c0 + 64].cpu().numpy(), ref_q)
        assert np.array_equal(sb[:, c0:c0 + 64].cpu().numpy(), oracle.pack_scales(ref_s))
