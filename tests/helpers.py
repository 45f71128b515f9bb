"""Comparison helpers shared by the GPU parity tests.

Tolerances (floating point):
  * fp32 output: relative Frobenius error <= 1e-5, per non-empty expert and
    over the whole tensor; an expert whose exact result is zero must be
    exactly zero.
  * bf16 output: every element within 2 bf16 ulps of the exact value, the ulp
    taken at max(|exact|, 2^-8 * rms of that expert's exact result) so that
    near-cancelled elements are judged on the expert's scale.
  * fp16 output: the same with fp16 ulps, floor also 2^-8 * rms: near zero the
    fp32 accumulation the contract fixes errs by ~1e-6 of the rms over long
    token ranges, which a finer floor would count against fp16's resolution
    (2 fp16 ulps at 2^-8 * rms is ~8e-6 of the rms, in line with fp32's 1e-5).
Integer-valued inputs make every partial sum exact in fp32, so those cases
are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

FP32_REL_FROB = 1e-5
BF16_ULPS = 2.0
BF16_FLOOR = 2.0 ** -8
FP16_FLOOR = 2.0 ** -8


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_frob(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def assert_fp32_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """got/ref: (..., H, N) blocks of one or more experts (leading axis = expert)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    for e in range(ref.shape[0]):
        if not np.any(ref[e]):
            assert not np.any(got[e]), f"{what}: expert {e} should be exactly zero"
            continue
        err = rel_frob(got[e], ref[e])
        assert err <= FP32_REL_FROB, f"{what}: expert {e} rel Frobenius {err:.3e}"
    err = rel_frob(got, ref)
    assert err <= FP32_REL_FROB, f"{what}: whole rel Frobenius {err:.3e}"


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str = "", rms: np.ndarray = None):
    """Element-wise 2-ulp check; `rms` gives each expert's rms (defaults to ref's own)."""
    _assert_ulps(got, ref, what, rms, BF16_FLOOR, oracle.bf16_ulp, "bf16")


def assert_fp16_close(got: np.ndarray, ref: np.ndarray, what: str = "", rms: np.ndarray = None):
    """Element-wise 2-ulp check in fp16 units (floor 2^-8 * rms)."""
    _assert_ulps(got, ref, what, rms, FP16_FLOOR, oracle.fp16_ulp, "fp16")


def _assert_ulps(got, ref, what, rms, floor, ulp_fn, name):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    for e in range(ref.shape[0]):
        r = ref[e]
        s = float(np.sqrt(np.mean(r * r))) if rms is None else float(rms[e])
        if s == 0.0:
            assert not np.any(got[e]), f"{what}: expert {e} should be exactly zero"
            continue
        scale = np.maximum(np.abs(r), floor * s)
        tol = BF16_ULPS * ulp_fn(scale)
        bad = np.abs(got[e] - r) > tol
        nbad = int(bad.sum())
        if nbad:
            idx = np.argwhere(bad)[0]
            raise AssertionError(f"{what}: expert {e}: {nbad} elements beyond 2 {name} ulps, first at "
                                 f"{tuple(idx)} got {got[e][tuple(idx)]!r} want {r[tuple(idx)]!r}")


def sample_rows(hidden: int, k: int, seed: int) -> np.ndarray:
    """First, last and k-2 random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = {0, hidden - 1}
    rows.update(rng.integers(0, hidden, size=max(0, k - 2)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def every_bf16_up_to(limit: float) -> torch.Tensor:
    """Every finite bf16 value with |x| <= limit (both signs, zeros and subnormals
    included), as float32 in increasing bit-pattern order."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).float()
    return x[torch.isfinite(x) & (x.abs() <= limit)]


def anchored_blocks(values: torch.Tensor, anchor: float, block: int, multiple: int, seed: int) -> torch.Tensor:
    """`values` shuffled into blocks of `block` tokens whose first entry is `anchor`
    (the block maximum, which fixes the block's scale), zero-padded to a multiple of
    `multiple` tokens: every value meets the scale that the anchor selects."""
    g = torch.Generator().manual_seed(seed)
    v = values[torch.randperm(len(values), generator=g)]
    per = block - 1
    nblk = -(-len(v) // per)
    body = torch.zeros(nblk * per)
    body[:len(v)] = v
    out = torch.cat([torch.full((nblk, 1), anchor), body.view(nblk, per)], dim=1)
    flat = out.reshape(-1)
    pad = (-len(flat)) % multiple
    return torch.cat([flat, torch.zeros(pad)])
