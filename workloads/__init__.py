"""Seeded synthetic inputs for the K-grouped weight-gradient GEMM.

This module only *produces inputs*: per-expert token counts, the int32
inclusive-cumulative offsets built from them, random operand matrices, and
the fp8 test-data quantiser that turns bf16 operands into (e4m3 bytes,
UE8M0 scale bytes) pairs.  It holds none of the grouped GEMM's arithmetic;
both the CPU oracle (via the tests) and the HIP path consume what it makes.

Shapes follow the cuDNN "Grouped GEMM + WGrad (Unified)" page, section
"BF16 contract": A is (hidden, tokens_sum) with the token axis contiguous,
B is (tokens_sum, intermediate) row-major, offsets is int32 (num_experts,),
the dense output is (num_experts, hidden, intermediate).

Count distributions:
  * balanced / fp8: expected tokens per expert times U(0.7, 1.3), the
    generator quoted on the llm-infra-atlas page, section 2.1 (contiguous
    layout), rounded up to the alignment unit;
  * skewed: 256 * round(lognormal(ln 16, 1)), four experts forced empty,
    total capped at 262144 tokens;
  * many-small: 65536 tokens over 256 experts, ~40% empty, the rest spread
    by a Zipf(1.2) law over ranks (see ``counts_many_small``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

E4M3_MAX = 448.0          # largest finite OCP E4M3 ("fn") magnitude
E8M0_BIAS = 127
SCALE_BLOCK = 128         # tokens per fp8 scale block (1 x 128 along the token axis)


# ----------------------------------------------------------------------------
# per-expert token counts
# ----------------------------------------------------------------------------
def _roundup(x: np.ndarray, unit: int) -> np.ndarray:
    return ((x + unit - 1) // unit) * unit


def counts_tiny() -> List[int]:
    return [256, 0, 512, 256]


def counts_uniform(num_experts: int, expected: int, unit: int, seed: int) -> List[int]:
    """expected * U(0.7, 1.3) tokens per expert, rounded up to `unit`."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.7, 1.3, size=num_experts)
    n = np.ceil(expected * u).astype(np.int64)
    return _roundup(n, unit).astype(int).tolist()


def counts_skewed(seed: int, num_experts: int = 32, unit: int = 256,
                  forced_zeros: int = 4, cap_tokens: int = 262144) -> List[int]:
    """unit * round(lognormal(ln 16, 1)); `forced_zeros` experts emptied; total capped.

    The cap rescales unit counts by floor(units * cap_units / sum(units)) when
    the sum exceeds the cap; the forced-empty experts are drawn after sampling.
    """
    rng = np.random.default_rng(seed)
    units = np.rint(rng.lognormal(mean=math.log(16.0), sigma=1.0, size=num_experts)).astype(np.int64)
    zeros = rng.choice(num_experts, size=forced_zeros, replace=False)
    units[zeros] = 0
    cap_units = cap_tokens // unit
    total = int(units.sum())
    if total > cap_units:
        units = (units * cap_units) // total
    return (units * unit).astype(int).tolist()


def counts_many_small(seed: int, num_experts: int = 256, tokens_sum: int = 65536,
                      unit: int = 256, empty_frac: float = 0.4, zipf_s: float = 1.2) -> List[int]:
    """Many small experts with a Zipf(1.2) tail and about 40% empty experts.

    A seeded permutation picks round(empty_frac * E) empty experts; each of the
    others gets one `unit` of tokens, and the remaining units are spread with
    multinomial(remaining, p_r ~ r^-s) over the non-empty experts in permuted
    rank order.  The total is exactly `tokens_sum`.
    """
    rng = np.random.default_rng(seed)
    total_units = tokens_sum // unit
    n_empty = int(round(empty_frac * num_experts))
    perm = rng.permutation(num_experts)
    nonempty = perm[n_empty:]
    k = len(nonempty)
    ranks = np.arange(1, k + 1, dtype=np.float64)
    p = ranks ** (-zipf_s)
    p /= p.sum()
    units = np.ones(k, dtype=np.int64) + rng.multinomial(total_units - k, p)
    counts = np.zeros(num_experts, dtype=np.int64)
    counts[nonempty] = units * unit
    return counts.astype(int).tolist()


def offsets_from_counts(counts: List[int]) -> np.ndarray:
    """int32 inclusive cumulative sum of per-expert token counts."""
    return np.cumsum(np.asarray(counts, dtype=np.int64)).astype(np.int32)


# ----------------------------------------------------------------------------
# operands
# ----------------------------------------------------------------------------
def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, std: float, gen: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def randint_values(shape, lo: int, hi: int, gen: torch.Generator, device, dtype) -> torch.Tensor:
    """Integer values in [lo, hi] stored in a float dtype (exact in bf16 / e4m3 for small ranges)."""
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device, dtype=torch.int32).to(dtype)


def e8m0_exponent_for_block(amax: torch.Tensor) -> torch.Tensor:
    """Biased UE8M0 exponent e with amax / 2^(e-127) <= 448 (127 where the block is all zero)."""
    a = amax.to(torch.float64)
    safe = torch.where(a > 0, a, torch.ones_like(a))
    e = torch.ceil(torch.log2(safe / E4M3_MAX))
    # guard against log2 rounding: bump where the scaled max would still exceed the range
    e = torch.where(safe / torch.exp2(e) > E4M3_MAX, e + 1, e)
    e = torch.where(a > 0, e, torch.zeros_like(e)) + E8M0_BIAS
    return e.clamp_(1, 254).to(torch.uint8)


def quantize_token_blocks(x: torch.Tensor, token_axis: int, block: int = SCALE_BLOCK):
    """Quantise a bf16/fp32 matrix to OCP e4m3fn with one UE8M0 scale per `block` tokens.

    token_axis = 1 for A (hidden, tokens) and 0 for B (tokens, N).  Returns
    (q, s): q holds e4m3fn bytes (uint8) in x's layout; s holds the biased
    exponents (uint8) laid out (tokens/block, other_dim), i.e. mn-major.
    Rounding: round-to-nearest-even in the float8 conversion.
    """
    xf = x.to(torch.float32)
    if token_axis == 1:
        xf = xf.t()                      # (tokens, other)
    t, o = xf.shape
    assert t % block == 0, "token count must be a multiple of the scale block"
    blocks = xf.reshape(t // block, block, o)
    amax = blocks.abs().amax(dim=1)      # (t/block, o)
    s = e8m0_exponent_for_block(amax)    # (t/block, o) uint8
    scale = torch.exp2(s.to(torch.float32) - E8M0_BIAS)
    q = (blocks / scale[:, None, :]).reshape(t, o).to(torch.float8_e4m3fn).view(torch.uint8)
    if token_axis == 1:
        q = q.t()
    return q.contiguous(), s.contiguous()


def pack_scale_words(s: torch.Tensor) -> torch.Tensor:
    """(nblocks, mn) uint8 scale bytes -> (ceil(nblocks/4), mn) int32 words, four consecutive
    blocks per little-endian word (block 4w + j in byte j), zero bytes past the last block."""
    nb, mn = s.shape
    nw = (nb + 3) // 4
    padded = torch.zeros((4 * nw, mn), dtype=torch.uint8, device=s.device)
    padded[:nb] = s
    return padded.reshape(nw, 4, mn).permute(0, 2, 1).contiguous().view(torch.int32).reshape(nw, mn)


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    counts: List[int]
    hidden: int
    n: int
    kind: str                     # "bf16" or "fp8"
    out_dtype: torch.dtype
    accumulate: bool
    A: torch.Tensor = None        # bf16 (hidden, T) or uint8 e4m3 bytes
    B: torch.Tensor = None        # bf16 (T, n) or uint8 e4m3 bytes
    sfa: Optional[torch.Tensor] = None   # uint8 (T/scale_block, hidden)
    sfb: Optional[torch.Tensor] = None   # uint8 (T/scale_block, n)
    C0: Optional[torch.Tensor] = None    # initial output for accumulate mode
    offsets: torch.Tensor = None         # int32 (E,)
    scale_block: int = SCALE_BLOCK       # tokens per fp8 scale (128, or 32 for MX-style blocks)
    meta: Dict = field(default_factory=dict)

    @property
    def num_experts(self) -> int:
        return len(self.counts)

    @property
    def tokens_sum(self) -> int:
        return int(sum(self.counts))

    @property
    def flops(self) -> float:
        return 2.0 * self.hidden * self.n * self.tokens_sum


DESCRIPTIONS = {
    "tiny": "tiny bf16 E=4 H=256 N=512 counts [256,0,512,256], fp32 out, overwrite",
    "balanced": "balanced bf16 fc2-wgrad E=8 H=4096 N=2048 n_e=roundup256(4096*U(0.7,1.3)), bf16 out, overwrite",
    "skewed": "skewed bf16 fc1-wgrad E=32 H=7168 N=4096 lognormal counts, 4 empty, fp32 out, accumulate",
    "fp8": "fp8 e4m3 1x128 UE8M0 block-scaled E=32 H=7168 N=4096 n_e=roundup128(8192*U(0.7,1.3)), bf16 out, overwrite",
    "many_small": "many-small bf16 E=256 H=7168 N=2048 tokens_sum=65536 Zipf(1.2) ~40% empty, fp32 out, overwrite",
}


def config_spec(name: str, seed: int = 1) -> Dict:
    """Shape-only description of a named workload (no tensors)."""
    if name == "tiny":
        return dict(counts=counts_tiny(), hidden=256, n=512, kind="bf16", out_dtype=torch.float32,
                    accumulate=False, std=1.0)
    if name == "balanced":
        return dict(counts=counts_uniform(8, 4096, 256, seed), hidden=4096, n=2048, kind="bf16",
                    out_dtype=torch.bfloat16, accumulate=False, std=0.02)
    if name == "skewed":
        return dict(counts=counts_skewed(seed), hidden=7168, n=4096, kind="bf16", out_dtype=torch.float32,
                    accumulate=True, std=1.0)
    if name == "fp8":
        return dict(counts=counts_uniform(32, 8192, 128, seed), hidden=7168, n=4096, kind="fp8",
                    out_dtype=torch.bfloat16, accumulate=False, std=1.0)
    if name == "many_small":
        return dict(counts=counts_many_small(seed), hidden=7168, n=2048, kind="bf16", out_dtype=torch.float32,
                    accumulate=False, std=1.0)
    raise KeyError(name)


def make_operands(counts: List[int], hidden: int, n: int, kind: str, out_dtype: torch.dtype,
                  accumulate: bool, seed: int, device="cpu", std: float = 1.0,
                  integer_range: Optional[int] = None, name: str = "custom",
                  scale_block: int = SCALE_BLOCK) -> Workload:
    """Build a Workload with tensors on `device`.

    Draw order from one generator seeded with `seed`: A, then B, then the
    initial output C0 (accumulate mode only).  With `integer_range=r` the
    operands hold integers in [-r, r] instead of normals (for fp8 the integers
    are stored exactly as e4m3 values with unit scales).  fp8 operands get one
    scale per `scale_block` tokens.
    """
    T = int(sum(counts))
    g = _gen(seed, device)
    wl = Workload(name=name, counts=list(map(int, counts)), hidden=hidden, n=n, kind=kind,
                  out_dtype=out_dtype, accumulate=accumulate, scale_block=scale_block)
    if integer_range is None:
        A = randn_bf16((hidden, T), std, g, device)
        B = randn_bf16((T, n), std, g, device)
    else:
        A = randint_values((hidden, T), -integer_range, integer_range, g, device, torch.bfloat16)
        B = randint_values((T, n), -integer_range, integer_range, g, device, torch.bfloat16)
    if kind == "bf16":
        wl.A, wl.B = A, B
    elif kind == "fp8":
        if integer_range is None:
            wl.A, wl.sfa = quantize_token_blocks(A, token_axis=1, block=scale_block)
            wl.B, wl.sfb = quantize_token_blocks(B, token_axis=0, block=scale_block)
        else:
            wl.A = A.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
            wl.B = B.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
            wl.sfa = torch.full((T // scale_block, hidden), E8M0_BIAS, dtype=torch.uint8, device=device)
            wl.sfb = torch.full((T // scale_block, n), E8M0_BIAS, dtype=torch.uint8, device=device)
        del A, B
    else:
        raise ValueError(kind)
    if accumulate:
        E = len(counts)
        if integer_range is None:
            wl.C0 = torch.randn((E, hidden, n), generator=g, device=device, dtype=torch.float32).to(out_dtype)
        else:
            wl.C0 = randint_values((E, hidden, n), -integer_range, integer_range, g, device, out_dtype)
    wl.offsets = torch.from_numpy(offsets_from_counts(counts)).to(device)
    return wl


def make_workload(name: str, seed: int = 1, device="cpu") -> Workload:
    spec = config_spec(name, seed)
    std = spec.pop("std")
    wl = make_operands(seed=seed, device=device, std=std, name=name, **spec)
    wl.meta["description"] = DESCRIPTIONS[name]
    wl.meta["seed"] = seed
    return wl


CONFIG_NAMES = ["tiny", "balanced", "skewed", "fp8", "many_small"]


# ----------------------------------------------------------------------------
# m-grouped (forward / dgrad) inputs
# ----------------------------------------------------------------------------
@dataclass
class MGroupedWorkload:
    counts: List[int]              # rows per group (multiples of 128; zero allowed)
    K: int
    N: int
    layout: str                    # "nt": W (E, N, K) (forward); "nn": W (E, K, N) (dgrad)
    A: torch.Tensor = None         # bf16 (M, K), rows grouped contiguously
    W: torch.Tensor = None         # bf16, see layout
    offsets: torch.Tensor = None   # int32 (E,), inclusive cumulative row counts
    m_indices: torch.Tensor = None  # int32 (M,), group id per row (-1 for pad rows)
    sa: Optional[torch.Tensor] = None   # fp8: UE8M0 (K/128, M) scales of A
    sw: Optional[torch.Tensor] = None   # fp8: UE8M0 (E, K/128, N) scales of W

    @property
    def M(self) -> int:
        return int(self.A.shape[0])

    @property
    def flops(self) -> float:
        return 2.0 * sum(self.counts) * self.K * self.N


def make_mgrouped(counts: List[int], K: int, N: int, layout: str, seed: int, device="cpu", pad_rows: int = 0,
                  std: float = 1.0, integer_range: Optional[int] = None) -> MGroupedWorkload:
    """Seeded operands of the m-grouped GEMM: A then W from one generator; `pad_rows` extra rows
    after the last group (group id -1 in m_indices, beyond the last offset)."""
    g = _gen(seed, device)
    M = int(sum(counts)) + pad_rows
    E = len(counts)
    wshape = (E, N, K) if layout == "nt" else (E, K, N)
    if integer_range is None:
        A = randn_bf16((M, K), std, g, device)
        W = randn_bf16(wshape, std, g, device)
    else:
        A = randint_values((M, K), -integer_range, integer_range, g, device, torch.bfloat16)
        W = randint_values(wshape, -integer_range, integer_range, g, device, torch.bfloat16)
    idx = np.concatenate([np.repeat(np.arange(E), counts), -np.ones(pad_rows, dtype=np.int64)]).astype(np.int32)
    return MGroupedWorkload(counts=list(map(int, counts)), K=K, N=N, layout=layout, A=A, W=W,
                            offsets=torch.from_numpy(offsets_from_counts(counts)).to(device),
                            m_indices=torch.from_numpy(idx).to(device))


def make_mgrouped_fp8(counts: List[int], K: int, N: int, seed: int, device="cpu", pad_rows: int = 0,
                      integer_range: Optional[int] = None) -> MGroupedWorkload:
    """fp8 operands of the m-grouped forward ("nt") product: the bf16 draws of make_mgrouped
    quantised to e4m3fn with one UE8M0 scale per 1x128 block along K (llm-infra-atlas section 3),
    scales mn-major: A -> (codes (M, K), sa (K/128, M)), W -> (codes (E, N, K), sw (E, K/128, N)).
    With `integer_range` the values are small integers stored exactly with unit scales."""
    wl = make_mgrouped(counts, K, N, "nt", seed, device, pad_rows=pad_rows, integer_range=integer_range)
    E = len(counts)
    if integer_range is None:
        qa, sa = quantize_token_blocks(wl.A, token_axis=1)
        qs = [quantize_token_blocks(wl.W[e], token_axis=1) for e in range(E)]
        qw = torch.stack([q for q, _ in qs]) if E else torch.empty((0, N, K), dtype=torch.uint8, device=device)
        sw = torch.stack([s for _, s in qs]) if E else torch.empty((0, K // 128, N), dtype=torch.uint8, device=device)
    else:
        qa = wl.A.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
        qw = wl.W.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
        sa = torch.full((K // 128, qa.shape[0]), E8M0_BIAS, dtype=torch.uint8, device=device)
        sw = torch.full((E, K // 128, N), E8M0_BIAS, dtype=torch.uint8, device=device)
    wl.A, wl.W = qa, qw.contiguous()
    wl.sa, wl.sw = sa.contiguous(), sw.contiguous()
    return wl


# ----------------------------------------------------------------------------
# FP4 (e2m1) test operands: token-contiguous, two tokens per byte (even token in
# the low nibble), one UE8M0 scale per 32 tokens
# ----------------------------------------------------------------------------
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code, magnitudes above 6 saturate), sign bit 8."""
    a = np.abs(v)
    idx = np.clip(np.searchsorted(E2M1_MAGNITUDES, a, side="right") - 1, 0, 7)
    lo = E2M1_MAGNITUDES[idx]
    hi = E2M1_MAGNITUDES[np.minimum(idx + 1, 7)]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & (idx % 2 == 1))
    code = np.where(idx == 7, 7, np.where(up, idx + 1, idx))
    return (code + 8 * np.signbit(v)).astype(np.uint8)


def quantize_fp4_token_blocks(x: torch.Tensor):
    """bf16/fp32 (rows, tokens) -> (packed e2m1 bytes (rows, tokens/2), UE8M0 bytes (tokens/32, rows))."""
    xf = x.to(torch.float32).cpu().numpy().astype(np.float64)
    rows, t = xf.shape
    assert t % 32 == 0
    blocks = xf.reshape(rows, t // 32, 32)
    amax = np.abs(blocks).max(axis=2)                       # (rows, t/32)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / E2M1_MAX))
    e = np.where(safe / np.exp2(e) > E2M1_MAX, e + 1, e)
    e = np.where(amax > 0, e, 0.0)
    s = np.clip(e + E8M0_BIAS, 1, 254).astype(np.uint8)      # (rows, t/32)
    scaled = blocks / np.exp2(s.astype(np.float64) - E8M0_BIAS)[:, :, None]
    codes = e2m1_codes(scaled).reshape(rows, t)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(packed), torch.from_numpy(np.ascontiguousarray(s.T))


def make_fp4_operands(counts: List[int], hidden: int, n: int, seed: int, device="cpu", integer_range=None,
                      random_codes: bool = False):
    """Seeded FP4 operands of the weight gradient: A (hidden, T/2) and B (n, T/2) packed e2m1,
    sfa (T/32, hidden) and sfb (T/32, n).  Draw order: A then B (bf16 normals quantised per
    32-token block, or integers in [-integer_range, integer_range] taken to e2m1 exactly (no 5)
    with unit scales).  random_codes=True draws every byte uniformly (each byte is two valid
    e2m1 codes) and the scale bytes uniformly in [122, 132], on `device` -- for full-size shapes,
    where quantising billions of values on the host would take minutes."""
    T = int(sum(counts))
    if random_codes:
        g = _gen(seed, device)
        qa = torch.randint(0, 256, (hidden, T // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        qb = torch.randint(0, 256, (n, T // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        sa = torch.randint(122, 133, (T // 32, hidden), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        sb = torch.randint(122, 133, (T // 32, n), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
        off = torch.from_numpy(offsets_from_counts(counts)).to(device)
        return dict(A=qa, sfa=sa, B=qb, sfb=sb, offsets=off, counts=list(map(int, counts)), hidden=hidden, n=n)
    g = _gen(seed, "cpu")
    if integer_range is None:
        a = randn_bf16((hidden, T), 1.0, g, "cpu")
        b = randn_bf16((n, T), 1.0, g, "cpu")
        qa, sa = quantize_fp4_token_blocks(a)
        qb, sb = quantize_fp4_token_blocks(b)
    else:
        vals = torch.tensor([-6.0, -4.0, -3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0, 4.0, 6.0])
        keep = vals[vals.abs() <= integer_range]
        ia = keep[torch.randint(0, keep.numel(), (hidden, T), generator=g)]
        ib = keep[torch.randint(0, keep.numel(), (n, T), generator=g)]
        ca, cb = e2m1_codes(ia.numpy()), e2m1_codes(ib.numpy())
        qa = torch.from_numpy((ca[:, 0::2] | (ca[:, 1::2] << 4)).astype(np.uint8))
        qb = torch.from_numpy((cb[:, 0::2] | (cb[:, 1::2] << 4)).astype(np.uint8))
        sa = torch.full((T // 32, hidden), E8M0_BIAS, dtype=torch.uint8)
        sb = torch.full((T // 32, n), E8M0_BIAS, dtype=torch.uint8)
    off = torch.from_numpy(offsets_from_counts(counts))
    return dict(A=qa.to(device), sfa=sa.to(device), B=qb.to(device), sfb=sb.to(device), offsets=off.to(device),
                counts=list(map(int, counts)), hidden=hidden, n=n)
