"""CPU oracle for the K-grouped MoE weight-gradient GEMM (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the
HIP library and its Python binding) never imports this package, and this
package never imports the product.

The arithmetic lives in ``kgw_oracle.c`` (plain C, IEEE double, OpenMP over
output rows).  This module builds it with gcc, loads it with ctypes, and
adds the output semantics of the cuDNN "Grouped GEMM + WGrad (Unified)"
page, section "Operation": overwrite writes Wgrad[e] (an empty expert gives
zero); accumulate adds Wgrad[e] onto the caller-initialised output.

Every function here is pinned by tests/test_oracle.py against brute force,
closed forms, library decoders or invariants; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kgw_oracle.c")
_LIB = os.path.join(_HERE, "libkgw_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kgw_oracle.c into libkgw_oracle.so next to it (gcc, OpenMP)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3fn_value.restype = ctypes.c_double
    lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_expert_range.restype = None
    lib.oracle_expert_range.argtypes = [p, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_wgrad_rows_bf16.restype = ctypes.c_int
    lib.oracle_wgrad_rows_bf16.argtypes = [p, p, i64, i64, i64, i64, p, i64, p]
    lib.oracle_wgrad_rows_fp8.restype = ctypes.c_int
    lib.oracle_wgrad_rows_fp8.argtypes = [p, p, i64, p, p, i64, i64, i64, i64, p, i64, p, i64]
    lib.oracle_wgrad_bf16.restype = ctypes.c_int
    lib.oracle_wgrad_bf16.argtypes = [p, p, p, i32, i64, i64, i64, p]
    lib.oracle_wgrad_fp8.restype = ctypes.c_int
    lib.oracle_wgrad_fp8.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p, i64]
    lib.oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_double]
    lib.oracle_e8m0_for_amax.restype = ctypes.c_uint8
    lib.oracle_e8m0_for_amax.argtypes = [ctypes.c_double]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_e8m0_for_amax_fp4.restype = ctypes.c_uint8
    lib.oracle_e8m0_for_amax_fp4.argtypes = [ctypes.c_double]
    lib.oracle_wgrad_rows_fp4.restype = ctypes.c_int
    lib.oracle_wgrad_rows_fp4.argtypes = [p, p, i64, p, p, i64, i64, i64, i64, p, i64, p]
    lib.oracle_wgrad_fp4.restype = ctypes.c_int
    lib.oracle_wgrad_fp4.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p]
    lib.oracle_quantize_fp4_tokens.restype = ctypes.c_int
    lib.oracle_quantize_fp4_tokens.argtypes = [p, i64, i64, p, p]
    lib.oracle_mgrouped_bf16.restype = ctypes.c_int
    lib.oracle_mgrouped_bf16.argtypes = [p, p, p, i64, i64, i64, i32, ctypes.c_int, p]
    lib.oracle_mgrouped_fp8.restype = ctypes.c_int
    lib.oracle_mgrouped_fp8.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p]
    lib.oracle_quantize_fp8_tokens.restype = ctypes.c_int
    lib.oracle_quantize_fp8_tokens.argtypes = [p, i64, i64, ctypes.c_int, p, p, i64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _u16(a) -> np.ndarray:
    a = _as_numpy(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def _u8(a) -> np.ndarray:
    a = _as_numpy(a)
    if a.dtype == np.int8:
        a = a.view(np.uint8)
    assert a.dtype == np.uint8, a.dtype
    return np.ascontiguousarray(a)


def _as_numpy(a) -> np.ndarray:
    """Raw storage of a host array or CPU torch tensor (bf16 viewed as its bit pattern)."""
    if isinstance(a, np.ndarray):
        return a
    import torch  # only for accepting CPU tensors; no torch arithmetic is used
    t = a.detach()
    assert t.device.type == "cpu", "the oracle works on host memory"
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn,):
        return t.view(torch.uint8).numpy()
    return t.numpy()


# ----------------------------------------------------------------------------
# decoders and offsets
# ----------------------------------------------------------------------------
def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def e4m3fn_value(bits: int) -> float:
    return _load().oracle_e4m3fn_value(bits)


def e8m0_value(bits: int) -> float:
    return _load().oracle_e8m0_value(bits)


def expert_range(offsets, e: int):
    off = np.ascontiguousarray(_as_numpy(offsets).astype(np.int32))
    b, t = ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_expert_range(_ptr(off), int(e), ctypes.byref(b), ctypes.byref(t))
    return b.value, t.value


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------------------
# the grouped product
# ----------------------------------------------------------------------------
def wgrad_rows_bf16(A, B, offsets, e: int, rows: Sequence[int]) -> np.ndarray:
    """Rows `rows` of Wgrad[e] in float64 (bf16 operands)."""
    a, b = _u16(A), _u16(B)
    hidden, T = a.shape
    n = b.shape[1]
    begin, end = expert_range(offsets, e)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.size == 0 or (r.min() >= 0 and r.max() < hidden)
    out = np.empty((r.size, n), dtype=np.float64)
    rc = _load().oracle_wgrad_rows_bf16(_ptr(a), _ptr(b), T, n, begin, end, _ptr(r), r.size, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle: bad token range [{begin}, {end}) for tokens_sum {T}")
    return out


def wgrad_rows_fp8(A, sfa, B, sfb, offsets, e: int, rows: Sequence[int], block: int = 128) -> np.ndarray:
    """Rows `rows` of Wgrad[e] in float64 (e4m3 operands, one UE8M0 byte per `block` tokens)."""
    a, sa, b, sb = _u8(A), _u8(sfa), _u8(B), _u8(sfb)
    hidden, T = a.shape
    n = b.shape[1]
    begin, end = expert_range(offsets, e)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.size == 0 or (r.min() >= 0 and r.max() < hidden)
    out = np.empty((r.size, n), dtype=np.float64)
    assert sa.shape == (T // block, hidden) and sb.shape == (T // block, n), "scale shape"
    rc = _load().oracle_wgrad_rows_fp8(_ptr(a), _ptr(sa), hidden, _ptr(b), _ptr(sb), T, n, begin, end,
                                       _ptr(r), r.size, _ptr(out), int(block))
    if rc != 0:
        raise ValueError(f"oracle: bad token range [{begin}, {end}) for tokens_sum {T}")
    return out


def wgrad_bf16(A, B, offsets) -> np.ndarray:
    """Dense Wgrad (E, hidden, n) in float64 for bf16 operands."""
    a, b = _u16(A), _u16(B)
    off = np.ascontiguousarray(_as_numpy(offsets).astype(np.int32))
    hidden, T = a.shape
    n = b.shape[1]
    out = np.empty((off.size, hidden, n), dtype=np.float64)
    rc = _load().oracle_wgrad_bf16(_ptr(a), _ptr(b), _ptr(off), off.size, hidden, n, T, _ptr(out))
    if rc != 0:
        raise ValueError("oracle: malformed offsets")
    return out


def wgrad_fp8(A, sfa, B, sfb, offsets, block: int = 128) -> np.ndarray:
    """Dense Wgrad (E, hidden, n) in float64 for e4m3 operands with one UE8M0 byte per `block`
    tokens: sfa (tokens_sum/block, hidden), sfb (tokens_sum/block, n)."""
    a, sa, b, sb = _u8(A), _u8(sfa), _u8(B), _u8(sfb)
    off = np.ascontiguousarray(_as_numpy(offsets).astype(np.int32))
    hidden, T = a.shape
    n = b.shape[1]
    out = np.empty((off.size, hidden, n), dtype=np.float64)
    assert sa.shape == (T // block, hidden) and sb.shape == (T // block, n), "scale shape"
    rc = _load().oracle_wgrad_fp8(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(off), off.size, hidden, n, T,
                                  _ptr(out), int(block))
    if rc != 0:
        raise ValueError("oracle: malformed offsets")
    return out


def e4m3fn_encode(v: float) -> int:
    """e4m3fn byte of v, round to nearest, ties to even (0x7F for NaN or beyond 448)."""
    return int(_load().oracle_e4m3fn_encode(float(v)))


def e8m0_for_amax(amax: float) -> int:
    """Biased UE8M0 exponent of the smallest 2^k with amax <= 448 * 2^k, clamped to [1, 254]
    (127 for 0, 255 for NaN/inf)."""
    return int(_load().oracle_e8m0_for_amax(float(amax)))


def quantize_fp8_tokens(x, token_axis: int, block: int = 128):
    """Quantise bf16 x (rows, cols) to e4m3fn with one UE8M0 scale per `block` tokens.

    token_axis 1: tokens along the columns (A (hidden, tokens)), scales (cols/block, rows);
    token_axis 0: tokens along the rows (B (tokens, n)), scales (rows/block, cols).
    Returns (q uint8 in x's layout, s uint8).
    """
    xb = _u16(x)
    rows, cols = xb.shape
    tokens = cols if token_axis else rows
    other = rows if token_axis else cols
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((tokens // block, other), dtype=np.uint8)
    rc = _load().oracle_quantize_fp8_tokens(_ptr(xb), rows, cols, int(token_axis), _ptr(q), _ptr(s), int(block))
    if rc != 0:
        raise ValueError(f"the token length must be a multiple of {block}")
    return q, s


# ----------------------------------------------------------------------------
# packed UE8M0 scale layout
# ----------------------------------------------------------------------------
# The pages name a packed UE8M0 scale tensor (the DeepGEMM k-grouped page's
# use_packed_ue8m0 flag; the llm-infra-atlas page, section 3, mn-major scales
# whose 8-bit exponents are packed) without printing its layout.  Reading used
# here: four consecutive blocks along the token axis share one little-endian
# 32-bit word, mn-major -- word (w, m) holds the scale byte of block 4w + j for
# mn index m in its byte j (bits 8j .. 8j+7); bytes of blocks past the last one
# are zero.
def pack_scales(s) -> np.ndarray:
    """(nblocks, mn) uint8 scale bytes -> (ceil(nblocks/4), mn) int32 packed words."""
    s = _u8(s)
    nb, mn = s.shape
    nw = (nb + 3) // 4
    padded = np.zeros((4 * nw, mn), dtype=np.uint32)
    padded[:nb] = s
    words = np.zeros((nw, mn), dtype=np.uint32)
    for j in range(4):
        words |= padded[j::4] << np.uint32(8 * j)
    return words.view(np.int32)


def unpack_scales(words, nblocks: int) -> np.ndarray:
    """Inverse of pack_scales: (ceil(nblocks/4), mn) int32 words -> (nblocks, mn) uint8 bytes."""
    w = np.ascontiguousarray(_as_numpy(words)).view(np.uint32)
    nw, mn = w.shape
    assert nw == (nblocks + 3) // 4, "word count"
    out = np.zeros((4 * nw, mn), dtype=np.uint8)
    for j in range(4):
        out[j::4] = ((w >> np.uint32(8 * j)) & np.uint32(0xFF)).astype(np.uint8)
    return out[:nblocks]


# ----------------------------------------------------------------------------
# FP4 (e2m1) operands, one UE8M0 scale per 32 tokens, both operands token-contiguous
# (two tokens per byte, the even token in the low nibble)
# ----------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code) & 15)


def e2m1_encode(v: float) -> int:
    """e2m1 code of v: round to nearest, ties to the even code, saturating at 6."""
    return int(_load().oracle_e2m1_encode(float(v)))


def e8m0_for_amax_fp4(amax: float) -> int:
    """Biased UE8M0 exponent of the smallest 2^k with amax <= 6 * 2^k, clamped to [1, 254]."""
    return int(_load().oracle_e8m0_for_amax_fp4(float(amax)))


def wgrad_fp4(A, sfa, B, sfb, offsets) -> np.ndarray:
    """Dense Wgrad (E, hidden, n) in float64 for e2m1 operands: A (hidden, T/2) and B (n, T/2)
    packed bytes (token axis contiguous), sfa (T/32, hidden), sfb (T/32, n) UE8M0 bytes."""
    a, sa, b, sb = _u8(A), _u8(sfa), _u8(B), _u8(sfb)
    off = np.ascontiguousarray(_as_numpy(offsets).astype(np.int32))
    hidden, half = a.shape
    n = b.shape[0]
    T = 2 * half
    assert b.shape == (n, half) and sa.shape == (T // 32, hidden) and sb.shape == (T // 32, n), "shapes"
    out = np.empty((off.size, hidden, n), dtype=np.float64)
    rc = _load().oracle_wgrad_fp4(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(off), off.size, hidden, n, T, _ptr(out))
    if rc != 0:
        raise ValueError("oracle: malformed offsets")
    return out


def wgrad_rows_fp4(A, sfa, B, sfb, offsets, e: int, rows: Sequence[int]) -> np.ndarray:
    """Rows `rows` of Wgrad[e] for e2m1 operands (layouts as wgrad_fp4)."""
    a, sa, b, sb = _u8(A), _u8(sfa), _u8(B), _u8(sfb)
    hidden, half = a.shape
    n = b.shape[0]
    T = 2 * half
    begin, end = expert_range(offsets, e)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((r.size, n), dtype=np.float64)
    rc = _load().oracle_wgrad_rows_fp4(_ptr(a), _ptr(sa), hidden, _ptr(b), _ptr(sb), T, n, begin, end, _ptr(r),
                                       r.size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle: bad token range")
    return out


def quantize_fp4_tokens(x):
    """bf16 x (rows, cols), tokens along the columns -> (q (rows, cols/2) packed e2m1 bytes,
    s (cols/32, rows) UE8M0 bytes).  Scale: the smallest 2^k with amax <= 6 * 2^k."""
    xb = _u16(x)
    rows, cols = xb.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((cols // 32, rows), dtype=np.uint8)
    if _load().oracle_quantize_fp4_tokens(_ptr(xb), rows, cols, _ptr(q), _ptr(s)) != 0:
        raise ValueError("the token length must be a multiple of 32")
    return q, s


# ----------------------------------------------------------------------------
# m-grouped GEMM (forward / dgrad of the same experts)
# ----------------------------------------------------------------------------
def row_groups_from_offsets(offsets, M: int) -> np.ndarray:
    """Group of every row of an M-row contiguous layout: row m is in group e when
    offsets[e-1] <= m < offsets[e] (offsets[-1] read as 0); rows at or past the last offset
    belong to no group (-1)."""
    off = np.asarray(_as_numpy(offsets), dtype=np.int64)
    g = np.searchsorted(off, np.arange(M), side="right").astype(np.int32)
    g[g >= off.size] = -1
    return g


def mgrouped_bf16(A, W, *, offsets=None, m_indices=None, layout: str = "nt") -> np.ndarray:
    """(M, N) float64 result of the m-grouped product; rows of no group are NaN.

    A bf16 (M, K); W bf16 (E, N, K) for layout "nt" (forward, out = A_g @ W_g^T) or
    (E, K, N) for "nn" (dgrad, out = A_g @ W_g).  Groups from inclusive cumulative
    `offsets` (E,) or from per-row `m_indices` (M,) (an id outside [0, E) = no group).
    """
    a, w = _u16(A), _u16(W)
    M, K = a.shape
    E = w.shape[0]
    nt = layout == "nt"
    assert layout in ("nt", "nn")
    N = w.shape[1] if nt else w.shape[2]
    assert (w.shape[2] if nt else w.shape[1]) == K, "W does not match A's K"
    if m_indices is not None:
        grp = np.ascontiguousarray(np.asarray(_as_numpy(m_indices), dtype=np.int32))
    else:
        grp = row_groups_from_offsets(offsets, M)
    assert grp.shape == (M,)
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_mgrouped_bf16(_ptr(a), _ptr(w), _ptr(grp), M, K, N, E, int(nt), _ptr(out))
    return out


def mgrouped_fp8(A, sa, W, sw, *, offsets=None, m_indices=None) -> np.ndarray:
    """(M, N) float64 result of the fp8 m-grouped forward product; rows of no group are NaN.

    A e4m3 bytes (M, K), sa UE8M0 bytes (K/128, M); W e4m3 bytes (E, N, K), sw UE8M0 bytes
    (E, K/128, N): each value is e4m3(code) * 2^(scale - 127) with the scale of its 1x128 block
    along K.  Groups from inclusive cumulative `offsets` or per-row `m_indices`.
    """
    a, s_a, w, s_w = _u8(A), _u8(sa), _u8(W), _u8(sw)
    M, K = a.shape
    E, N = w.shape[0], w.shape[1]
    assert K % 128 == 0 and w.shape[2] == K, "K must be a multiple of 128 and match W"
    assert s_a.shape == (K // 128, M) and s_w.shape == (E, K // 128, N), "scale shapes"
    if m_indices is not None:
        grp = np.ascontiguousarray(np.asarray(_as_numpy(m_indices), dtype=np.int32))
    else:
        grp = row_groups_from_offsets(offsets, M)
    assert grp.shape == (M,)
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_mgrouped_fp8(_ptr(a), _ptr(s_a), _ptr(w), _ptr(s_w), _ptr(grp), M, K, N, E, _ptr(out))
    return out


def apply_output_mode(W: np.ndarray, accumulate: bool, C0: Optional[np.ndarray] = None) -> np.ndarray:
    """Exact (float64) value the output should hold before rounding to its dtype.

    overwrite: Wgrad itself (an empty expert's sum is over no tokens: zero);
    accumulate: the caller's initial output plus Wgrad.
    """
    if not accumulate:
        return W
    assert C0 is not None and C0.shape == W.shape
    return C0.astype(np.float64) + W


# ----------------------------------------------------------------------------
# output rounding (for exactness pins) and the bf16 unit in the last place
# ----------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even), returned as float64.

    Goes through float32 first, which is exact for every value the exactness
    pins use (integers below 2^24); NaN stays NaN.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE binary16 (numpy's cast: nearest, ties to even; overflow to
    infinity), returned as float64.  Goes through float32 first, exact for the exactness pins'
    values (integers below 2^24)."""
    with np.errstate(over="ignore"):                 # overflow to infinity is the defined result
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def fp16_ulp(x: np.ndarray) -> np.ndarray:
    """Unit in the last place of binary16 at |x| (2^(e-10) for normal x, 2^-24 below 2^-14)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -14)))
    return np.exp2(e - 10)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 7)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    tiny = 2.0 ** -126
    ax = np.maximum(ax, tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7.0)
