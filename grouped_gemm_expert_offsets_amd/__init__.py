"""Python binding of libkgw: the K-grouped MoE weight-gradient GEMM for MI355X.

For expert e with token range [begin, end) from int32 inclusive cumulative
offsets (begin = 0 for the first expert, offsets[e-1] otherwise; end =
offsets[e]) the library computes

    Wgrad[e] = A[:, begin:end] @ B[begin:end, :]

into a dense (num_experts, hidden, n) output, overwriting it or accumulating
into it (cuDNN "Grouped GEMM + WGrad (Unified)", section "Operation").

Every function here only marshals arguments (tensor shapes, dtypes, device
pointers, the current HIP stream) and calls the C-ABI entry point of the
same name in libkgw.so; all arithmetic runs in the library's HIP kernels.
Status codes 1-4 raise ValueError, 5 raises RuntimeError (the cuDNN page,
section "Scheduling, cache, and errors", splits errors the same way).
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "kgw_wgrad_bf16", "kgw_wgrad_bf16_noalloc", "kgw_wgrad_bf16_ex", "kgw_wgrad_fp8", "kgw_wgrad_fp8_native", "kgw_wgrad_fp8_ex",
    "kgw_wgrad_fp4", "FP4_TOKEN_ALIGN",
    "kgw_quantize_fp8", "kgw_quantize_fp4", "kgw_mgrouped_bf16", "kgw_mgrouped_fp8", "kgw_workspace_bytes",
    "KGW_LAYOUT_NT",
    "KGW_LAYOUT_NN",
    "KGW_A_M_MAJOR", "KGW_B_K_MAJOR", "KGW_RAGGED",
    "kgw_validate_offsets", "kgw_check_offsets", "kgw_mfma_ceiling",
    "kgw_validate_offsets_host", "kgw_status_string", "kgw_device_info", "wgrad",
    "KGW_SUCCESS", "KGW_ERROR_INVALID_VALUE", "KGW_ERROR_MISALIGNED", "KGW_ERROR_BAD_OFFSETS",
    "KGW_ERROR_UNSUPPORTED", "KGW_ERROR_DEVICE", "KGW_OUT_FP32", "KGW_OUT_BF16", "KGW_OUT_FP16",
    "KGW_SCALES_U8", "KGW_SCALES_PACKED", "KGW_SCALES_PACKED_32", "scale_shape",
    "BF16_TOKEN_ALIGN", "FP8_TOKEN_ALIGN", "library_path", "load_library",
]

KGW_SUCCESS = 0
KGW_ERROR_INVALID_VALUE = 1
KGW_ERROR_MISALIGNED = 2
KGW_ERROR_BAD_OFFSETS = 3
KGW_ERROR_UNSUPPORTED = 4
KGW_ERROR_DEVICE = 5
KGW_OUT_FP32 = 0
KGW_OUT_BF16 = 1
KGW_OUT_FP16 = 2
KGW_A_M_MAJOR = 1          # weight-gradient A stored (tokens_sum, hidden)
KGW_B_K_MAJOR = 2          # weight-gradient B stored (n, tokens_sum)
KGW_RAGGED = 4             # per-expert K-contiguous blocks back to back (with KGW_B_K_MAJOR)
KGW_LAYOUT_NT = 0          # m-grouped forward: W (E, N, K)
KGW_LAYOUT_NN = 1          # m-grouped dgrad:   W (E, K, N)
KGW_SCALES_U8 = 0          # uint8 (tokens/128, mn)
KGW_SCALES_PACKED = 1      # int32 (ceil(tokens/512), mn): four 128-token blocks per word
KGW_SCALES_PACKED_32 = 2   # int32 (tokens/128, mn): four 32-token blocks per word
BF16_TOKEN_ALIGN = 256
FP8_TOKEN_ALIGN = 128
FP4_TOKEN_ALIGN = 256

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkgw.so")
_lib = None

# Every symbol include/kgw.h declares.
EXPORTED_SYMBOLS = ("kgw_wgrad_bf16", "kgw_wgrad_bf16_noalloc", "kgw_wgrad_bf16_ex", "kgw_wgrad_fp8", "kgw_wgrad_fp8_native",
                    "kgw_wgrad_fp8_ex", "kgw_wgrad_fp4", "kgw_quantize_fp8", "kgw_quantize_fp4", "kgw_mgrouped_bf16",
                    "kgw_mgrouped_fp8", "kgw_workspace_bytes", "kgw_validate_offsets_host", "kgw_validate_offsets", "kgw_check_offsets",
                    "kgw_mfma_ceiling", "kgw_status_string", "kgw_device_info")


def load_library():
    """Load libkgw.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is missing: build it with "
                           "`python -m grouped_gemm_expert_offsets_amd.build`")
    lib = ctypes.CDLL(library_path)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kgw_wgrad_bf16.restype = ctypes.c_int
    lib.kgw_wgrad_bf16.argtypes = [p, p, p, i32, i64, i64, i64, p, i32, i32, p, sz, p]
    lib.kgw_wgrad_bf16_noalloc.restype = ctypes.c_int
    lib.kgw_wgrad_bf16_noalloc.argtypes = [p, p, p, i32, i64, i64, i64, p, i32, i32, p]
    lib.kgw_wgrad_fp8.restype = ctypes.c_int
    lib.kgw_wgrad_fp8.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p, i32, i32, p, sz, p]
    lib.kgw_wgrad_fp8_native.restype = ctypes.c_int
    lib.kgw_wgrad_fp8_native.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p, i32, i32, p, sz, p]
    lib.kgw_wgrad_bf16_ex.restype = ctypes.c_int
    lib.kgw_wgrad_bf16_ex.argtypes = [p, p, i32, p, i32, i64, i64, i64, p, p, i32, i32, p, sz, p]
    lib.kgw_wgrad_fp8_ex.restype = ctypes.c_int
    lib.kgw_wgrad_fp8_ex.argtypes = [p, p, p, p, i32, i32, i32, p, i32, i64, i64, i64, p, p, i32, i32, p, sz, p]
    lib.kgw_wgrad_fp4.restype = ctypes.c_int
    lib.kgw_wgrad_fp4.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p, p, i32, i32, p, sz, p]
    lib.kgw_mgrouped_bf16.restype = ctypes.c_int
    lib.kgw_mgrouped_bf16.argtypes = [p, p, i32, p, p, i32, i64, i64, i64, p, i32, i32, p]
    lib.kgw_mgrouped_fp8.restype = ctypes.c_int
    lib.kgw_mgrouped_fp8.argtypes = [p, p, p, p, i32, p, p, i32, i64, i64, i64, p, i32, i32, p]
    lib.kgw_quantize_fp8.restype = ctypes.c_int
    lib.kgw_quantize_fp8.argtypes = [p, i64, i64, i32, i32, p, p, p]
    lib.kgw_quantize_fp4.restype = ctypes.c_int
    lib.kgw_quantize_fp4.argtypes = [p, i64, i64, i32, i32, p, p, p]
    lib.kgw_workspace_bytes.restype = sz
    lib.kgw_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.kgw_validate_offsets_host.restype = ctypes.c_int
    lib.kgw_validate_offsets_host.argtypes = [p, i32, i64, i32, ctypes.POINTER(i32)]
    lib.kgw_validate_offsets.restype = ctypes.c_int
    lib.kgw_validate_offsets.argtypes = [p, i32, i64, i32, ctypes.POINTER(i32), p]
    lib.kgw_check_offsets.restype = ctypes.c_int
    lib.kgw_check_offsets.argtypes = [p, i32, i64, i32, p, p]
    lib.kgw_mfma_ceiling.restype = ctypes.c_int
    lib.kgw_mfma_ceiling.argtypes = [p, i64, i32, i32, i32, p, p]
    lib.kgw_status_string.restype = ctypes.c_char_p
    lib.kgw_status_string.argtypes = [ctypes.c_int]
    lib.kgw_device_info.restype = ctypes.c_int
    lib.kgw_device_info.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    _lib = lib
    return lib


def kgw_status_string(status: int) -> str:
    return load_library().kgw_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status == KGW_SUCCESS:
        return
    msg = f"{what}: {kgw_status_string(status)} (status {status})"
    if status == KGW_ERROR_DEVICE:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _workspace(E: int, hidden: int, n: int, T: int, fp8: bool, device, stream, split_k: bool):
    """Device workspace for the call (None when it runs in one pass or split_k is False)."""
    if not split_k:
        return None, 0
    nbytes = kgw_workspace_bytes(E, hidden, n, T, fp8)
    if nbytes == 0:
        return None, 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)   # keep it alive for the launch stream's pending work
    return ws, nbytes


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _out_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return KGW_OUT_FP32
    if dtype == torch.bfloat16:
        return KGW_OUT_BF16
    if dtype == torch.float16:
        return KGW_OUT_FP16
    raise ValueError(f"output dtype must be float32, bfloat16 or float16, got {dtype}")


def _prepare_out(out, E, hidden, n, out_dtype, accumulate, device):
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an initialised `out`")
        return torch.empty((E, hidden, n), dtype=out_dtype, device=device)
    if tuple(out.shape) != (E, hidden, n):
        raise ValueError(f"out must have shape {(E, hidden, n)}, got {tuple(out.shape)}")
    if not out.is_contiguous() or out.device != device:
        raise ValueError("out must be a contiguous tensor on the operands' device")
    return out


def _prepare_outs(outs, E, hidden, n, out_dtype, device, stream):
    """Per-expert outputs -> (list, device int64 array of their addresses, 0 for None)."""
    outs = list(outs)
    if len(outs) != E:
        raise ValueError(f"need one output (or None) per expert: {E}, got {len(outs)}")
    for t in outs:
        if t is None:
            continue
        if tuple(t.shape) != (hidden, n) or t.dtype != out_dtype or t.device != device or not t.is_contiguous():
            raise ValueError(f"each output must be a contiguous {(hidden, n)} {out_dtype} tensor on {device}")
    addrs = torch.tensor([0 if t is None else int(t.data_ptr()) for t in outs], dtype=torch.int64)
    s = torch.cuda.current_stream(device) if stream is None else stream
    with torch.cuda.stream(s):
        ptrs = addrs.to(device)
    ptrs.record_stream(s)
    return outs, ptrs


def _check_offsets(offsets: torch.Tensor, device):
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous 1-D int32 tensor")
    if offsets.device != device:
        raise ValueError("offsets must live on the operands' device")
    if offsets.numel() < 1:
        raise ValueError("need at least one expert")


def kgw_wgrad_bf16(A: torch.Tensor, B: torch.Tensor, offsets: torch.Tensor, out: Optional[torch.Tensor] = None,
                   *, out_dtype: torch.dtype = torch.float32, accumulate: bool = False, validate: bool = False,
                   stream=None, split_k: bool = True) -> torch.Tensor:
    """bf16 A (hidden, tokens_sum) token-contiguous, B (tokens_sum, n) row-major -> out (E, hidden, n).

    validate=True first checks the offsets on the host (one synchronising copy).  The
    workspace kgw_workspace_bytes asks for is allocated here; split_k=False passes none
    (one pass).
    """
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("kgw_wgrad_bf16 takes bfloat16 A and B")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (A token-contiguous, B row-major)")
    device = A.device
    if B.device != device:
        raise ValueError("A and B must be on the same device")
    _check_offsets(offsets, device)
    hidden, T = A.shape
    n = B.shape[1]
    E = offsets.numel()
    if out is not None:
        out_dtype = out.dtype
    code = _out_code(out_dtype)
    out = _prepare_out(out, E, hidden, n, out_dtype, accumulate, device)
    if validate:
        kgw_validate_offsets(offsets, T, BF16_TOKEN_ALIGN, stream=stream)
    ws, ws_bytes = _workspace(E, hidden, n, T, False, device, stream, split_k)
    st = load_library().kgw_wgrad_bf16(_ptr(A), _ptr(B), _ptr(offsets), E, hidden, n, T, _ptr(out), code,
                                       int(bool(accumulate)), _ptr(ws), ws_bytes, _stream_ptr(stream))
    _check(st, "kgw_wgrad_bf16")
    return out


def kgw_wgrad_bf16_noalloc(A: torch.Tensor, B: torch.Tensor, offsets: torch.Tensor, out: torch.Tensor, *,
                           accumulate: bool = False, stream=None) -> torch.Tensor:
    """kgw_wgrad_bf16 that allocates nothing, here or in the library: `out` must be given
    (its dtype selects the output type), and split-K partials use the library's fixed
    per-device scratch.  Calls that overlap in time on one device race on that scratch."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("kgw_wgrad_bf16_noalloc takes bfloat16 A and B")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (A token-contiguous, B row-major)")
    if out is None:
        raise ValueError("kgw_wgrad_bf16_noalloc needs `out` (it allocates nothing)")
    device = A.device
    if B.device != device:
        raise ValueError("A and B must be on the same device")
    _check_offsets(offsets, device)
    hidden, T = A.shape
    n = B.shape[1]
    E = offsets.numel()
    code = _out_code(out.dtype)
    out = _prepare_out(out, E, hidden, n, out.dtype, accumulate, device)
    st = load_library().kgw_wgrad_bf16_noalloc(_ptr(A), _ptr(B), _ptr(offsets), E, hidden, n, T, _ptr(out), code,
                                               int(bool(accumulate)), _stream_ptr(stream))
    _check(st, "kgw_wgrad_bf16_noalloc")
    return out


def kgw_wgrad_bf16_ex(A: torch.Tensor, B: torch.Tensor, offsets: torch.Tensor, *, a_major: str = "k",
                      b_major: str = "n", ragged: bool = False, hidden: Optional[int] = None,
                      n: Optional[int] = None, out: Optional[torch.Tensor] = None, outs=None,
                      out_dtype: torch.dtype = torch.float32, accumulate: bool = False, validate: bool = False,
                      stream=None, split_k: bool = True):
    """kgw_wgrad_bf16 with a choice of operand layout and output form.

    a_major "k": A is (hidden, tokens_sum) (the default); "m": A is stored (tokens_sum, hidden).
    b_major "n": B is (tokens_sum, n) (the default); "k": B is stored (n, tokens_sum).
    ragged=True (with a_major "k", b_major "k"): A and B hold per-expert blocks (hidden, n_e) and
    (n, n_e) back to back; pass them as flat buffers with `hidden` and `n`.
    `outs` is a list of num_experts (hidden, n) tensors (None skips that expert) whose addresses
    go to the device as the pointer array (returned); otherwise `out` as for kgw_wgrad_bf16.
    """
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("kgw_wgrad_bf16_ex takes bfloat16 A and B")
    if a_major not in ("k", "m") or b_major not in ("n", "k"):
        raise ValueError("a_major is 'k' or 'm', b_major is 'n' or 'k'")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous in their declared layout")
    layout = (KGW_A_M_MAJOR if a_major == "m" else 0) | (KGW_B_K_MAJOR if b_major == "k" else 0)
    if ragged:
        if a_major != "k" or b_major != "k":
            raise ValueError("ragged input needs K-major A and B (a_major='k', b_major='k')")
        if hidden is None or n is None or hidden <= 0 or n <= 0 or A.numel() % hidden:
            raise ValueError("ragged input needs hidden and n, and A.numel() a multiple of hidden")
        layout |= KGW_RAGGED
        T = A.numel() // hidden
        if B.numel() != T * n:
            raise ValueError(f"B must hold tokens_sum * n = {T * n} elements")
    else:
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        hidden, T = A.shape if a_major == "k" else (A.shape[1], A.shape[0])
        Tb, n = B.shape if b_major == "n" else (B.shape[1], B.shape[0])
        if Tb != T:
            raise ValueError(f"shape mismatch: A {tuple(A.shape)} ({a_major}-major), B {tuple(B.shape)} ({b_major}-major)")
    device = A.device
    if B.device != device:
        raise ValueError("A and B must be on the same device")
    _check_offsets(offsets, device)
    E = offsets.numel()
    out, outs, ptrs, code = _outputs(out, outs, E, hidden, n, out_dtype, accumulate, device, stream)
    if validate:
        kgw_validate_offsets(offsets, T, BF16_TOKEN_ALIGN, stream=stream)
    ws, ws_bytes = _workspace(E, hidden, n, T, False, device, stream, split_k)
    st = load_library().kgw_wgrad_bf16_ex(_ptr(A), _ptr(B), layout, _ptr(offsets), E, hidden, n, T, _ptr(out),
                                          _ptr(ptrs), code, int(bool(accumulate)), _ptr(ws), ws_bytes,
                                          _stream_ptr(stream))
    _check(st, "kgw_wgrad_bf16_ex")
    return out if outs is None else outs


def _outputs(out, outs, E, hidden, n, out_dtype, accumulate, device, stream):
    """Resolve the dense / discrete output forms: (out, outs, pointer array, dtype code)."""
    if out is not None and outs is not None:
        raise ValueError("pass either out or outs, not both")
    if outs is not None:
        outs = list(outs)
        given = [t for t in outs if t is not None]
        if given:
            out_dtype = given[0].dtype
        code = _out_code(out_dtype)
        outs, ptrs = _prepare_outs(outs, E, hidden, n, out_dtype, device, stream)
        return None, outs, ptrs, code
    if out is not None:
        out_dtype = out.dtype
    code = _out_code(out_dtype)
    return _prepare_out(out, E, hidden, n, out_dtype, accumulate, device), None, None, code


def kgw_wgrad_fp8(A: torch.Tensor, sfa: torch.Tensor, B: torch.Tensor, sfb: torch.Tensor, offsets: torch.Tensor,
                  out: Optional[torch.Tensor] = None, *, out_dtype: torch.dtype = torch.bfloat16,
                  accumulate: bool = False, validate: bool = False, stream=None, split_k: bool = True) -> torch.Tensor:
    """e4m3 A (hidden, T) with UE8M0 sfa (T/128, hidden); e4m3 B (T, n) with sfb (T/128, n)."""
    return _fp8_call("kgw_wgrad_fp8", A, sfa, B, sfb, offsets, out, out_dtype, accumulate, validate, stream,
                     split_k)


def kgw_wgrad_fp8_native(A: torch.Tensor, sfa: torch.Tensor, B: torch.Tensor, sfb: torch.Tensor,
                         offsets: torch.Tensor, out: Optional[torch.Tensor] = None, *,
                         out_dtype: torch.dtype = torch.bfloat16, accumulate: bool = False, validate: bool = False,
                         stream=None, split_k: bool = True) -> torch.Tensor:
    """kgw_wgrad_fp8 on the native scaled fp8 MFMA (faster, ~13-bit in-group alignment; see include/kgw.h)."""
    return _fp8_call("kgw_wgrad_fp8_native", A, sfa, B, sfb, offsets, out, out_dtype, accumulate, validate,
                     stream, split_k)


def kgw_wgrad_fp8_ex(A: torch.Tensor, sfa: torch.Tensor, B: torch.Tensor, sfb: torch.Tensor,
                     offsets: torch.Tensor, *, scale_format: int = KGW_SCALES_U8, native: bool = False,
                     a_major: str = "k", b_major: str = "n", ragged: bool = False, hidden: Optional[int] = None,
                     n: Optional[int] = None, out: Optional[torch.Tensor] = None, outs=None,
                     out_dtype: torch.dtype = torch.bfloat16, accumulate: bool = False, validate: bool = False,
                     stream=None, split_k: bool = True):
    """fp8 product with a scale layout (KGW_SCALES_*: uint8 per 128 tokens, packed int32 words of
    four 128-token blocks, or packed words of four 32-token blocks) and a dense `out` or discrete
    `outs` (see kgw_wgrad_bf16_ex); native=True uses the scaled fp8 MFMA.  Operand layouts as for
    kgw_wgrad_bf16_ex: a_major "k" (A is (hidden, T), the default) or "m" (A stored (T, hidden));
    b_major "n" (B is (T, n), the default) or "k" (B stored (n, T)); ragged=True (with a_major
    "k", b_major "k"): per-expert K-contiguous blocks back to back, passed as flat buffers with
    `hidden` and `n`.  Layouts other than the default take the exact path with uint8 scales;
    the scales keep their (T/128, mn) shapes."""
    if a_major not in ("k", "m") or b_major not in ("n", "k"):
        raise ValueError("a_major is 'k' or 'm', b_major is 'n' or 'k'")
    if ragged and (a_major != "k" or b_major != "k"):
        raise ValueError("ragged input needs K-major A and B (a_major='k', b_major='k')")
    return _fp8_call("kgw_wgrad_fp8_ex", A, sfa, B, sfb, offsets, out, out_dtype, accumulate, validate, stream,
                     split_k, scale_format=scale_format, native=native, outs=outs, a_m_major=a_major == "m",
                     b_k_major=b_major == "k", ragged_dims=(hidden, n) if ragged else None)


def kgw_wgrad_fp4(A: torch.Tensor, sfa: torch.Tensor, B: torch.Tensor, sfb: torch.Tensor, offsets: torch.Tensor,
                  *, out: Optional[torch.Tensor] = None, outs=None, out_dtype: torch.dtype = torch.bfloat16,
                  accumulate: bool = False, validate: bool = False, stream=None, split_k: bool = True):
    """FP4 (e2m1) operands, both token-contiguous and packed two tokens per byte: A (hidden, T/2)
    and B (n, T/2) uint8; scales one UE8M0 per 32 tokens, packed: sfa (T/128, hidden) and
    sfb (T/128, n) int32 (KGW_SCALES_PACKED_32)."""
    if A.dtype != torch.uint8 or B.dtype != torch.uint8 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("kgw_wgrad_fp4 takes packed e2m1 bytes: A (hidden, T/2), B (n, T/2) uint8")
    if A.shape[1] != B.shape[1]:
        raise ValueError(f"A {tuple(A.shape)} and B {tuple(B.shape)} must hold the same token count")
    hidden, T = A.shape[0], 2 * A.shape[1]
    n = B.shape[0]
    (sa_shape, sdtype), (sb_shape, _) = (scale_shape(T, hidden, KGW_SCALES_PACKED_32),
                                         scale_shape(T, n, KGW_SCALES_PACKED_32))
    if sfa.dtype != sdtype or sfb.dtype != sdtype or tuple(sfa.shape) != sa_shape or tuple(sfb.shape) != sb_shape:
        raise ValueError(f"scales must be int32 {sa_shape} and {sb_shape}")
    for t in (A, B, sfa, sfb):
        if not t.is_contiguous():
            raise ValueError("fp4 operands and scales must be contiguous")
    device = A.device
    if any(t.device != device for t in (B, sfa, sfb)):
        raise ValueError("operands and scales must be on the same device")
    _check_offsets(offsets, device)
    E = offsets.numel()
    out, outs, ptrs, code = _outputs(out, outs, E, hidden, n, out_dtype, accumulate, device, stream)
    if validate:
        kgw_validate_offsets(offsets, T, FP4_TOKEN_ALIGN, stream=stream)
    ws, ws_bytes = _workspace(E, hidden, n, T, True, device, stream, split_k)
    st = load_library().kgw_wgrad_fp4(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(offsets), E, hidden, n, T,
                                      _ptr(out), _ptr(ptrs), code, int(bool(accumulate)), _ptr(ws), ws_bytes,
                                      _stream_ptr(stream))
    _check(st, "kgw_wgrad_fp4")
    return out if outs is None else outs


def scale_shape(tokens: int, mn: int, scale_format: int) -> Tuple[Tuple[int, int], torch.dtype]:
    """Shape and dtype of the scale tensor of an operand with `tokens` tokens and mn other extent."""
    if scale_format == KGW_SCALES_U8:
        return (tokens // FP8_TOKEN_ALIGN, mn), torch.uint8
    if scale_format == KGW_SCALES_PACKED:
        return ((tokens // FP8_TOKEN_ALIGN + 3) // 4, mn), torch.int32
    if scale_format == KGW_SCALES_PACKED_32:
        return (tokens // FP8_TOKEN_ALIGN, mn), torch.int32
    raise ValueError(f"unknown scale_format {scale_format}")


def _fp8_call(name, A, sfa, B, sfb, offsets, out, out_dtype, accumulate, validate, stream, split_k,
              scale_format=KGW_SCALES_U8, native=None, outs=None, a_m_major=False, b_k_major=False,
              ragged_dims=None):
    fp8_types = (torch.uint8, torch.float8_e4m3fn)
    if A.dtype not in fp8_types or B.dtype not in fp8_types:
        raise ValueError(f"{name} takes e4m3fn (or raw uint8) A and B")
    if sfa is None or sfb is None:
        raise ValueError(f"{name} needs both scale tensors sfa and sfb")
    if ragged_dims is not None:
        hidden, n = ragged_dims
        if hidden is None or n is None or hidden <= 0 or n <= 0 or A.numel() % hidden:
            raise ValueError("ragged input needs hidden and n, and A.numel() a multiple of hidden")
        T = A.numel() // hidden
        if B.numel() != T * n:
            raise ValueError(f"B must hold tokens_sum * n = {T * n} elements")
    else:
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        hidden, T = (A.shape[1], A.shape[0]) if a_m_major else (A.shape[0], A.shape[1])
        Tb, n = (B.shape[1], B.shape[0]) if b_k_major else (B.shape[0], B.shape[1])
        if Tb != T:
            raise ValueError(f"shape mismatch: A {tuple(A.shape)}{' (stored (T, hidden))' if a_m_major else ''}, "
                             f"B {tuple(B.shape)}{' (stored (n, T))' if b_k_major else ''}")
    (sa_shape, sdtype), (sb_shape, _) = scale_shape(T, hidden, scale_format), scale_shape(T, n, scale_format)
    if sfa.dtype != sdtype or sfb.dtype != sdtype:
        raise ValueError(f"this scale format takes {sdtype} scale tensors")
    if tuple(sfa.shape) != sa_shape or tuple(sfb.shape) != sb_shape:
        raise ValueError(f"scale shapes must be {sa_shape} and {sb_shape}")
    for t in (A, B, sfa, sfb):
        if not t.is_contiguous():
            raise ValueError("fp8 operands and scales must be contiguous")
    device = A.device
    if any(t.device != device for t in (B, sfa, sfb)):
        raise ValueError("operands and scales must be on the same device")
    _check_offsets(offsets, device)
    E = offsets.numel()
    out, outs, ptrs, code = _outputs(out, outs, E, hidden, n, out_dtype, accumulate, device, stream)
    if validate:
        kgw_validate_offsets(offsets, T, FP8_TOKEN_ALIGN, stream=stream)
    fn = getattr(load_library(), name)
    ws, ws_bytes = _workspace(E, hidden, n, T, True, device, stream, split_k)
    if native is None:
        st = fn(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(offsets), E, hidden, n, T, _ptr(out), code,
                int(bool(accumulate)), _ptr(ws), ws_bytes, _stream_ptr(stream))
    else:
        st = fn(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), int(scale_format), int(bool(native)),
                (KGW_A_M_MAJOR if a_m_major else 0) | (KGW_B_K_MAJOR if b_k_major else 0) |
                (KGW_RAGGED if ragged_dims is not None else 0), _ptr(offsets), E,
                hidden, n, T, _ptr(out), _ptr(ptrs), code,
                int(bool(accumulate)), _ptr(ws), ws_bytes, _stream_ptr(stream))
    _check(st, name)
    return out if outs is None else outs


def kgw_quantize_fp8(x: torch.Tensor, token_axis: int, stream=None,
                     scale_format: int = KGW_SCALES_U8) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 x (rows, cols) -> (e4m3fn bytes as uint8 (rows, cols), UE8M0 scales in `scale_format`).

    token_axis 1: tokens along the columns (A (hidden, tokens)), scales with mn = rows;
    token_axis 0: tokens along the rows (B (tokens, n)), scales with mn = cols.  See
    scale_shape for the scale tensor of each format.
    """
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("kgw_quantize_fp8 takes a contiguous 2-D bfloat16 tensor")
    if token_axis not in (0, 1):
        raise ValueError("token_axis must be 0 or 1")
    rows, cols = x.shape
    tokens, other = (cols, rows) if token_axis else (rows, cols)
    if tokens % FP8_TOKEN_ALIGN != 0:
        raise ValueError(f"the token length ({tokens}) must be a multiple of {FP8_TOKEN_ALIGN}")
    shape, sdtype = scale_shape(tokens, other, scale_format)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty(shape, dtype=sdtype, device=x.device)
    st = load_library().kgw_quantize_fp8(_ptr(x), rows, cols, int(token_axis), int(scale_format), _ptr(q), _ptr(s),
                                         _stream_ptr(stream))
    _check(st, "kgw_quantize_fp8")
    return q, s


def kgw_quantize_fp4(x: torch.Tensor, token_axis: int, stream=None,
                     scale_format: int = KGW_SCALES_PACKED_32) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 x (rows, cols) -> (packed e2m1 bytes, UE8M0 scales per 32 tokens), the operands of
    kgw_wgrad_fp4.

    token_axis 1: tokens along the columns (A (hidden, tokens)): codes (rows, cols/2), scales
    with mn = rows; token_axis 0: tokens along the rows (B (tokens, n)): codes (cols, rows/2)
    (token-contiguous), scales with mn = cols.  scale_format KGW_SCALES_PACKED_32 (int32
    (tokens/128, mn), what kgw_wgrad_fp4 takes) or KGW_SCALES_U8 (uint8 (tokens/32, mn)).
    """
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("kgw_quantize_fp4 takes a contiguous 2-D bfloat16 tensor")
    if token_axis not in (0, 1):
        raise ValueError("token_axis must be 0 or 1")
    if scale_format not in (KGW_SCALES_U8, KGW_SCALES_PACKED_32):
        raise ValueError("FP4 scales are KGW_SCALES_U8 or KGW_SCALES_PACKED_32")
    rows, cols = x.shape
    tokens, other = (cols, rows) if token_axis else (rows, cols)
    if tokens % 128 != 0:
        raise ValueError(f"the token length ({tokens}) must be a multiple of 128")
    if scale_format == KGW_SCALES_U8:
        shape, sdtype = (tokens // 32, other), torch.uint8
    else:
        shape, sdtype = scale_shape(tokens, other, scale_format)
    q = torch.empty((other, tokens // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty(shape, dtype=sdtype, device=x.device)
    st = load_library().kgw_quantize_fp4(_ptr(x), rows, cols, int(token_axis), int(scale_format), _ptr(q), _ptr(s),
                                         _stream_ptr(stream))
    _check(st, "kgw_quantize_fp4")
    return q, s


def kgw_mgrouped_bf16(A: torch.Tensor, W: torch.Tensor, *, offsets: Optional[torch.Tensor] = None,
                      m_indices: Optional[torch.Tensor] = None, layout: str = "nt",
                      out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                      accumulate: bool = False, stream=None) -> torch.Tensor:
    """m-grouped product: out[r] = A[r] @ W[g(r)]^T ("nt", W (E, N, K), the forward) or
    A[r] @ W[g(r)] ("nn", W (E, K, N), dgrad); groups from `offsets` (inclusive cumulative
    rows) or per-row `m_indices`; rows of no group are left untouched."""
    if A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("kgw_mgrouped_bf16 takes bfloat16 A and W")
    if A.dim() != 2 or W.dim() != 3 or not A.is_contiguous() or not W.is_contiguous():
        raise ValueError("A must be a contiguous (M, K) and W a contiguous (E, ., .) tensor")
    if layout not in ("nt", "nn"):
        raise ValueError("layout is 'nt' (forward) or 'nn' (dgrad)")
    M, K = A.shape
    E = W.shape[0]
    N = W.shape[1] if layout == "nt" else W.shape[2]
    if (W.shape[2] if layout == "nt" else W.shape[1]) != K:
        raise ValueError(f"W {tuple(W.shape)} does not match A's K = {K} for layout {layout}")
    device = A.device
    if W.device != device:
        raise ValueError("A and W must be on the same device")
    if (offsets is None) == (m_indices is None):
        raise ValueError("pass exactly one of offsets and m_indices")
    idx = offsets if offsets is not None else m_indices
    if idx.dtype != torch.int32 or idx.dim() != 1 or not idx.is_contiguous() or idx.device != device:
        raise ValueError("offsets / m_indices must be a contiguous 1-D int32 tensor on the operands' device")
    if offsets is not None and offsets.numel() != E:
        raise ValueError(f"offsets must have one entry per group ({E})")
    if m_indices is not None and m_indices.numel() != M:
        raise ValueError(f"m_indices must have one entry per row ({M})")
    if out is not None:
        out_dtype = out.dtype
    code = _out_code(out_dtype)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an initialised `out`")
        out = torch.empty((M, N), dtype=out_dtype, device=device)
    elif tuple(out.shape) != (M, N) or not out.is_contiguous() or out.device != device:
        raise ValueError(f"out must be a contiguous {(M, N)} tensor on the operands' device")
    st = load_library().kgw_mgrouped_bf16(_ptr(A), _ptr(W), KGW_LAYOUT_NT if layout == "nt" else KGW_LAYOUT_NN,
                                          _ptr(offsets), _ptr(m_indices), E, M, K, N, _ptr(out), code,
                                          int(bool(accumulate)), _stream_ptr(stream))
    _check(st, "kgw_mgrouped_bf16")
    return out


def kgw_mgrouped_fp8(A: torch.Tensor, sa: torch.Tensor, W: torch.Tensor, sw: torch.Tensor, *,
                     offsets: Optional[torch.Tensor] = None, m_indices: Optional[torch.Tensor] = None,
                     layout: str = "nt", out: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.bfloat16, accumulate: bool = False, stream=None) -> torch.Tensor:
    """m-grouped product with fp8 operands: A is e4m3 (M, K) with UE8M0 sa (K/128, M); W is e4m3
    (E, N, K) for layout "nt" (forward, out[r] = a(r) @ w(g(r))^T) or (E, K, N) for "nn" (dgrad,
    out[r] = a(r) @ w(g(r))), with UE8M0 sw (E, K/128, N) either way, one scale per 1x128 block
    along K; groups from `offsets` or `m_indices` as for kgw_mgrouped_bf16; rows of no group
    are left untouched."""
    fp8_types = (torch.uint8, torch.float8_e4m3fn)
    if A.dtype not in fp8_types or W.dtype not in fp8_types:
        raise ValueError("kgw_mgrouped_fp8 takes e4m3fn (or raw uint8) A and W")
    if sa is None or sw is None or sa.dtype != torch.uint8 or sw.dtype != torch.uint8:
        raise ValueError("kgw_mgrouped_fp8 needs uint8 scale tensors sa and sw")
    if A.dim() != 2 or W.dim() != 3:
        raise ValueError("A must be (M, K) and W (E, N, K)")
    for t in (A, W, sa, sw):
        if not t.is_contiguous():
            raise ValueError("fp8 operands and scales must be contiguous")
    if layout not in ("nt", "nn"):
        raise ValueError("layout is 'nt' (forward) or 'nn' (dgrad)")
    M, K = A.shape
    E = W.shape[0]
    N = W.shape[1] if layout == "nt" else W.shape[2]
    if (W.shape[2] if layout == "nt" else W.shape[1]) != K:
        raise ValueError(f"W {tuple(W.shape)} does not match A's K = {K} for layout {layout}")
    if K % FP8_TOKEN_ALIGN != 0:
        raise ValueError(f"K ({K}) must be a multiple of {FP8_TOKEN_ALIGN}")
    if tuple(sa.shape) != (K // FP8_TOKEN_ALIGN, M) or tuple(sw.shape) != (E, K // FP8_TOKEN_ALIGN, N):
        raise ValueError(f"scale shapes must be {(K // FP8_TOKEN_ALIGN, M)} and {(E, K // FP8_TOKEN_ALIGN, N)}")
    device = A.device
    if any(t.device != device for t in (W, sa, sw)):
        raise ValueError("operands and scales must be on the same device")
    if (offsets is None) == (m_indices is None):
        raise ValueError("pass exactly one of offsets and m_indices")
    idx = offsets if offsets is not None else m_indices
    if idx.dtype != torch.int32 or idx.dim() != 1 or not idx.is_contiguous() or idx.device != device:
        raise ValueError("offsets / m_indices must be a contiguous 1-D int32 tensor on the operands' device")
    if offsets is not None and offsets.numel() != E:
        raise ValueError(f"offsets must have one entry per group ({E})")
    if m_indices is not None and m_indices.numel() != M:
        raise ValueError(f"m_indices must have one entry per row ({M})")
    if out is not None:
        out_dtype = out.dtype
    code = _out_code(out_dtype)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an initialised `out`")
        out = torch.empty((M, N), dtype=out_dtype, device=device)
    elif tuple(out.shape) != (M, N) or not out.is_contiguous() or out.device != device:
        raise ValueError(f"out must be a contiguous {(M, N)} tensor on the operands' device")
    st = load_library().kgw_mgrouped_fp8(_ptr(A), _ptr(sa), _ptr(W), _ptr(sw),
                                         KGW_LAYOUT_NT if layout == "nt" else KGW_LAYOUT_NN, _ptr(offsets),
                                         _ptr(m_indices), E, M, K, N, _ptr(out), code, int(bool(accumulate)),
                                         _stream_ptr(stream))
    _check(st, "kgw_mgrouped_fp8")
    return out


def kgw_workspace_bytes(num_experts: int, hidden: int, n: int, tokens_sum: int, fp8: bool = False) -> int:
    return int(load_library().kgw_workspace_bytes(num_experts, hidden, n, tokens_sum, int(bool(fp8))))


def kgw_validate_offsets_host(offsets, tokens_sum: int, alignment: int) -> Tuple[int, int]:
    """Check host offsets (sequence or CPU tensor); returns (status, first bad expert or -1)."""
    t = torch.as_tensor(offsets, dtype=torch.int32).contiguous()
    if t.device.type != "cpu":
        raise ValueError("kgw_validate_offsets_host takes host offsets")
    bad = ctypes.c_int32(-1)
    st = load_library().kgw_validate_offsets_host(t.data_ptr(), t.numel(), int(tokens_sum), int(alignment),
                                                  ctypes.byref(bad))
    return int(st), int(bad.value)


def kgw_validate_offsets(offsets: torch.Tensor, tokens_sum: int, alignment: int, stream=None) -> None:
    """Check device offsets (synchronising); raises ValueError naming the first bad expert."""
    bad = ctypes.c_int32(-1)
    st = load_library().kgw_validate_offsets(_ptr(offsets), offsets.numel(), int(tokens_sum), int(alignment),
                                             ctypes.byref(bad), _stream_ptr(stream))
    if st != KGW_SUCCESS:
        _check(st, f"kgw_validate_offsets (first bad expert {bad.value})")


def kgw_check_offsets(offsets: torch.Tensor, tokens_sum: int, alignment: int,
                      result: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Queue the offsets check on the device (no synchronisation): returns a one-element
    int32 device tensor that will hold the first bad expert, or -1 (`result` if given)."""
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous 1-D int32 tensor")
    if result is None:
        result = torch.empty(1, dtype=torch.int32, device=offsets.device)
    elif result.dtype != torch.int32 or result.numel() < 1 or result.device != offsets.device:
        raise ValueError("result must be an int32 tensor on the offsets' device")
    st = load_library().kgw_check_offsets(_ptr(offsets), offsets.numel(), int(tokens_sum), int(alignment),
                                          _ptr(result), _stream_ptr(stream))
    _check(st, "kgw_check_offsets")
    return result


def kgw_mfma_ceiling(src: torch.Tensor, kind: int, iters: int = 20000, workgroups: int = 1024,
                     stream=None) -> Tuple[float, float]:
    """Time MFMA-only loops on the bytes of `src` (kind 0 bf16, 1 e4m3 as bf16, 2 e4m3 on the scaled
    fp8 MFMA, 3 e2m1 pairs on the scaled MFMA's FP4 mode): returns (TFLOP/s from HIP events around the launch, mean clock in GHz the loop ran
    at).  A measurement helper: it synchronises."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    cycles = torch.zeros(2 * workgroups, dtype=torch.int64, device=src.device)
    s = torch.cuda.current_stream(src.device) if stream is None else stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    st = load_library().kgw_mfma_ceiling(_ptr(src), src.numel() * src.element_size(), int(kind), int(iters),
                                         int(workgroups), _ptr(cycles), int(s.cuda_stream))
    end.record(s)
    _check(st, "kgw_mfma_ceiling")
    end.synchronize()
    ms = start.elapsed_time(end)
    c = cycles.view(-1, 2).double().cpu()
    ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1
    flop_per_mfma = 131072.0 if kind in (2, 3) else 32768.0
    flops = 16.0 * iters * workgroups * 4 * flop_per_mfma
    return flops / (ms * 1e-3) / 1e12, ghz


def kgw_device_info() -> dict:
    cus, g950, xcds = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().kgw_device_info(ctypes.byref(cus), ctypes.byref(g950), ctypes.byref(xcds)),
           "kgw_device_info")
    return {"num_cus": cus.value, "is_gfx950": bool(g950.value), "num_xcds": xcds.value}


def wgrad(a: torch.Tensor, b: torch.Tensor, offsets: torch.Tensor, *, sfa: Optional[torch.Tensor] = None,
          sfb: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
          out_dtype: Optional[torch.dtype] = None, accumulate: bool = False, check: bool = True) -> torch.Tensor:
    """Dispatch on operand dtype like the cuDNN wrapper: bf16 operands take no scales
    (any scale is a ValueError, section "BF16 contract"); fp8 operands need both.

    check=True (the default, like the cuDNN page's wrapper, which rejects malformed or
    unaligned offsets: section "Scheduling, cache, and errors") validates the offsets first,
    which costs one synchronising copy of them to the host; check=False skips it and the
    kernels clamp malformed ranges instead (see kgw_check_offsets for an asynchronous flag)."""
    if a.dtype == torch.bfloat16 and b.dtype == torch.bfloat16:
        if sfa is not None or sfb is not None:
            raise ValueError("bf16 operands take no scale tensors")
        return kgw_wgrad_bf16(a, b, offsets, out, out_dtype=out_dtype or torch.float32, accumulate=accumulate,
                              validate=check)
    if a.dtype in (torch.float8_e4m3fn, torch.uint8) and b.dtype in (torch.float8_e4m3fn, torch.uint8):
        return kgw_wgrad_fp8(a, sfa, b, sfb, offsets, out, out_dtype=out_dtype or torch.bfloat16,
                             accumulate=accumulate, validate=check)
    raise ValueError(f"unsupported operand dtypes {a.dtype}, {b.dtype}")
