"""GPU parity of the weight gradient's other operand layouts (A M-major, B K-major, ragged blocks).

The same logical A (hidden, tokens_sum) and B (tokens_sum, n) are stored in each layout by
plain tensor copies; the oracle multiplies the logical operands.  Integer-valued operands are
compared bit for bit; every layout must also give exactly the default layout's result on random
data (the MFMAs see the same operands in the same order).
"""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import oracle
import workloads
from helpers import assert_bf16_close, sample_rows, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
LAYOUTS = [("m", "n", False), ("m", "k", False), ("k", "k", False), ("k", "k", True)]


def stored(wl, a_major, b_major, ragged):
    """The workload's operands in the given layout (copies; the values are unchanged)."""
    if ragged:
        off = [0] + wl.offsets.tolist()
        a = torch.cat([wl.A[:, off[e]:off[e + 1]].contiguous().reshape(-1) for e in range(len(off) - 1)])
        b = torch.cat([wl.B[off[e]:off[e + 1]].t().contiguous().reshape(-1) for e in range(len(off) - 1)])
        return a, b
    a = wl.A.t().contiguous() if a_major == "m" else wl.A
    b = wl.B.t().contiguous() if b_major == "k" else wl.B
    return a, b


def run(wl, a_major, b_major, ragged, out, accumulate=False, split_k=True):
    a, b = stored(wl, a_major, b_major, ragged)
    kgw.kgw_wgrad_bf16_ex(a, b, wl.offsets, a_major=a_major, b_major=b_major, ragged=ragged, hidden=wl.hidden,
                          n=wl.n, out=out, accumulate=accumulate, split_k=split_k)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("a_major,b_major,ragged", LAYOUTS)
def test_integer_bit_exact(a_major, b_major, ragged, accumulate):
    counts = [256, 0, 768, 512, 256]
    wl = workloads.make_operands(counts, 264, 392, "bf16", torch.float32, accumulate, seed=111, device=DEV,
                                 integer_range=4)
    out = wl.C0.clone() if accumulate else torch.full((5, 264, 392), float("nan"), device=DEV)
    run(wl, a_major, b_major, ragged, out, accumulate)
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
    ref = oracle.apply_output_mode(W, accumulate, to_f64(wl.C0) if accumulate else None)
    got = to_f64(out)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {tuple(mism[0])}: {got[tuple(mism[0])]} vs {ref[tuple(mism[0])]}"


@pytest.mark.parametrize("a_major,b_major,ragged", LAYOUTS)
def test_random_equals_default_layout_and_oracle(a_major, b_major, ragged):
    counts = [512, 256, 0, 1280, 256]
    wl = workloads.make_operands(counts, 328, 400, "bf16", torch.bfloat16, False, seed=112, device=DEV)
    base = kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out_dtype=torch.bfloat16)
    out = run(wl, a_major, b_major, ragged, torch.full((5, 328, 400), float("nan"), device=DEV, dtype=torch.bfloat16))
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
    assert_bf16_close(to_f64(out), W, f"layout {a_major}{b_major}{'r' if ragged else ''}")


@pytest.mark.parametrize("a_major,b_major,ragged", LAYOUTS)
def test_split_k_integer_bit_exact(a_major, b_major, ragged):
    counts = [4096, 0, 8192, 256]
    wl = workloads.make_operands(counts, 320, 384, "bf16", torch.float32, False, seed=113, device=DEV,
                                 integer_range=4)
    assert kgw.kgw_workspace_bytes(4, 320, 384, sum(counts)) > 0
    out = run(wl, a_major, b_major, ragged, torch.full((4, 320, 384), float("nan"), device=DEV))
    one = run(wl, a_major, b_major, ragged, torch.full((4, 320, 384), float("nan"), device=DEV), split_k=False)
    W = oracle.wgrad_bf16(wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu())
    assert np.array_equal(to_f64(out), W) and torch.equal(out, one)


def test_full_balanced_token_major_operands():
    # the headline workload with both operands stored token-major, as dY (T, hidden) and X (T, n)
    wl = workloads.make_workload("balanced", seed=1, device=DEV)
    out = run(wl, "m", "n", False, torch.empty((8, 4096, 2048), dtype=torch.bfloat16, device=DEV))
    Ah, Bh, off = wl.A.cpu(), wl.B.cpu(), wl.offsets.cpu()
    for e in (0, 3, 7):
        rows = sample_rows(wl.hidden, 4, e)
        W = oracle.wgrad_rows_bf16(Ah, Bh, off, e, rows)
        got = to_f64(out[e][torch.from_numpy(rows).to(DEV)])
        assert_bf16_close(got[None], W[None], f"balanced token-major expert {e}",
                          rms=np.array([np.sqrt(np.mean(W * W))]))
