"""C-ABI library checks that need no GPU: symbols, host validation, argument errors.

Every call made here is rejected by the host-side argument checks (or is a
pure host function), so nothing is ever enqueued on a device.
"""
import ctypes
import json
import os
import re

import pytest

import grouped_gemm_expert_offsets_amd as kgw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def header_functions():
    text = open(os.path.join(ROOT, "include", "kgw.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kgw_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kgw.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 7
    for name in names:
        assert hasattr(lib, name), f"libkgw.so does not export {name}"
    assert sorted(kgw.EXPORTED_SYMBOLS) == names


def test_status_strings(lib):
    for code in range(6):
        s = kgw.kgw_status_string(code)
        assert isinstance(s, str) and s
    assert kgw.kgw_status_string(99) == "unknown status"


def test_workspace_is_zero(lib):
    assert kgw.kgw_workspace_bytes(8, 4096, 2048, 35584) == 0
    assert kgw.kgw_workspace_bytes(32, 7168, 4096, 264320, fp8=True) == 0


def test_workspace_bytes_split_k_plan():
    # the five workload shapes have enough tiles to fill the chip: no split; only the skewed one
    # (32 long experts, 49 rounds of tiles) takes the dynamic schedule's 256 bytes of counters
    import workloads
    for name in workloads.CONFIG_NAMES:
        spec = workloads.config_spec(name, 1)
        want = 256 if name == "skewed" else 0
        assert kgw.kgw_workspace_bytes(len(spec["counts"]), spec["hidden"], spec["n"], sum(spec["counts"]),
                                       fp8=spec["kind"] == "fp8") == want, name
    # few tiles and many tokens: split-K into chunks * E * hidden * n fp32 partials
    # (256 CUs when no device is visible: 4 tiles -> up to 16 chunks, 8 by tokens/(E*1024))
    assert kgw.kgw_workspace_bytes(2, 256, 512, 16384) == 8 * 2 * 256 * 512 * 4
    assert kgw.kgw_workspace_bytes(2, 256, 512, 16384, fp8=True) == 8 * 2 * 256 * 512 * 4
    # too few tokens per expert for two chunks of 1024 on average
    assert kgw.kgw_workspace_bytes(2, 256, 512, 4096 - 256) == 0
    # more than half of the CUs already have a tile
    assert kgw.kgw_workspace_bytes(1, 256 * 16, 256 * 9, 1 << 20) == 0


def test_workspace_bytes_dynamic_schedule_plan():
    # 256 bytes of counters: bf16 only, long experts (>= 1024 tokens on average), at most 64 of
    # them, and at least 8 rounds of tiles on 256 CUs (2048 items)
    assert kgw.kgw_workspace_bytes(32, 2048, 2048, 32 * 1024) == 256          # 2048 items
    assert kgw.kgw_workspace_bytes(32, 2048, 2048 - 256, 32 * 1024) == 0      # 1792 items
    assert kgw.kgw_workspace_bytes(32, 2048, 2048, 32 * 1024 - 256) == 0      # short experts
    assert kgw.kgw_workspace_bytes(65, 2048, 2048, 65 * 1024) == 0            # more than 64 experts
    assert kgw.kgw_workspace_bytes(32, 2048, 2048, 32 * 1024, fp8=True) == 0  # fp8 kernels: static


def validate(offsets, tokens_sum, align=256):
    return kgw.kgw_validate_offsets_host(offsets, tokens_sum, align)


def test_validate_offsets_host_accepts_contract():
    assert validate([256, 256, 768, 1024], 1024) == (kgw.KGW_SUCCESS, -1)
    assert validate([0, 0, 0], 0) == (kgw.KGW_SUCCESS, -1)
    assert validate([128, 384], 384, 128) == (kgw.KGW_SUCCESS, -1)


def test_validate_offsets_host_rejections():
    assert validate([512, 256, 1024], 1024) == (kgw.KGW_ERROR_BAD_OFFSETS, 1)      # decreasing
    assert validate([256, 300, 512], 512) == (kgw.KGW_ERROR_BAD_OFFSETS, 1)        # unaligned count
    assert validate([256, 512], 768) == (kgw.KGW_ERROR_BAD_OFFSETS, 1)             # last != tokens_sum
    assert validate([-256, 0], 0) == (kgw.KGW_ERROR_BAD_OFFSETS, 0)                # negative count
    assert validate([128, 256], 256, 256)[0] == kgw.KGW_ERROR_BAD_OFFSETS          # fp8-aligned, bf16 rule
    st, _ = kgw.kgw_validate_offsets_host([256], 256, 0)
    assert st == kgw.KGW_ERROR_INVALID_VALUE


def test_page_example_counts_are_rejected():
    g = json.load(open(os.path.join(GOLDEN, "p1_example_counts.json")))
    counts = g["tokens_per_expert"]
    offs, acc = [], 0
    for c in counts:
        acc += c
        offs.append(acc)
    st, bad = validate(offs, acc, 256)
    assert st == kgw.KGW_ERROR_BAD_OFFSETS and bad == g["first_bad_expert"]


# ----------------------------------------------------------------------------
# argument errors of the compute entry points (rejected before any HIP call)
# ----------------------------------------------------------------------------
FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced on these paths


def call_bf16(lib, A=FAKE, B=FAKE, off=FAKE, E=4, H=256, N=512, T=1024, out=FAKE, dt=0, acc=0):
    return lib.kgw_wgrad_bf16(A, B, off, E, H, N, T, out, dt, acc, None, 0, None)


def call_fp8(lib, A=FAKE, sa=FAKE, B=FAKE, sb=FAKE, off=FAKE, E=4, H=256, N=512, T=1024, out=FAKE, dt=1, acc=0):
    return lib.kgw_wgrad_fp8(A, sa, B, sb, off, E, H, N, T, out, dt, acc, None, 0, None)


def test_bf16_argument_errors(lib):
    assert call_bf16(lib, E=0) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, H=-1) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, dt=7) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, acc=2) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, off=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, A=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, out=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16(lib, A=FAKE + 8) == kgw.KGW_ERROR_MISALIGNED
    assert call_bf16(lib, out=FAKE + 4) == kgw.KGW_ERROR_MISALIGNED
    assert call_bf16(lib, N=500) == kgw.KGW_ERROR_MISALIGNED
    assert call_bf16(lib, T=1000) == kgw.KGW_ERROR_BAD_OFFSETS
    assert call_bf16(lib, E=65537) == kgw.KGW_ERROR_UNSUPPORTED


def test_fp8_argument_errors(lib):
    assert call_fp8(lib, sa=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8(lib, sb=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8(lib, T=1000) == kgw.KGW_ERROR_BAD_OFFSETS
    assert call_fp8(lib, N=520) == kgw.KGW_ERROR_MISALIGNED    # multiple of 8 but not 16
    assert call_fp8(lib, B=FAKE + 1) == kgw.KGW_ERROR_MISALIGNED


def test_empty_shapes_return_before_device(lib):
    # no output elements: nothing to do, no device needed
    assert call_bf16(lib, H=0, A=None, out=None) == kgw.KGW_SUCCESS
    assert call_bf16(lib, N=0, B=None, out=None) == kgw.KGW_SUCCESS
    # accumulate with no tokens adds nothing
    assert call_bf16(lib, T=0, A=None, B=None, acc=1) == kgw.KGW_SUCCESS


def test_python_binding_rejects_bad_tensors():
    import torch
    A = torch.zeros(4, 256, dtype=torch.bfloat16)
    B = torch.zeros(256, 8, dtype=torch.bfloat16)
    off = torch.tensor([256], dtype=torch.int32)
    with pytest.raises(ValueError):
        kgw.wgrad(A, B, off, sfa=torch.zeros(2, 4, dtype=torch.uint8))       # bf16 rejects scales
    with pytest.raises(ValueError):
        kgw.kgw_wgrad_bf16(A.float(), B, off)                                  # wrong dtype
    with pytest.raises(ValueError):
        kgw.kgw_wgrad_bf16(A, B[:128], off)                                    # shape mismatch
    with pytest.raises(ValueError):
        kgw.kgw_wgrad_fp8(A.view(torch.uint8)[:, :256], None, B.view(torch.uint8), None, off)  # no scales
    with pytest.raises(ValueError):
        kgw.kgw_wgrad_bf16(A, B, off, accumulate=True)                         # accumulate needs out


def call_bf16_ex(lib, out=FAKE, ptrs=None, H=256, N=512, E=4, T=1024, layout=0):
    return lib.kgw_wgrad_bf16_ex(FAKE, FAKE, layout, FAKE, E, H, N, T, out, ptrs, 0, 0, None, 0, None)


def call_fp8_ex(lib, sa=FAKE, sb=FAKE, fmt=0, native=0, out=FAKE, ptrs=None, H=256, N=512, T=1024, layout=0):
    return lib.kgw_wgrad_fp8_ex(FAKE, sa, FAKE, sb, fmt, native, layout, FAKE, 4, H, N, T, out, ptrs, 1, 0, None, 0,
                                None)


def test_extended_entry_point_errors(lib):
    # exactly one output form
    assert call_bf16_ex(lib, out=FAKE, ptrs=FAKE) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16_ex(lib, out=None, ptrs=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16_ex(lib, out=None, ptrs=FAKE + 4) == kgw.KGW_ERROR_MISALIGNED   # pointer array alignment
    assert call_bf16_ex(lib, out=None, ptrs=None, H=0) == kgw.KGW_SUCCESS         # nothing to write
    assert call_bf16_ex(lib, H=1 << 28) == kgw.KGW_ERROR_UNSUPPORTED
    # operand layouts: unknown bits, ragged without both K-major, M-major A with hidden % 8
    assert call_bf16_ex(lib, layout=8) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16_ex(lib, layout=kgw.KGW_RAGGED) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16_ex(lib, layout=kgw.KGW_RAGGED | kgw.KGW_A_M_MAJOR | kgw.KGW_B_K_MAJOR) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_bf16_ex(lib, layout=kgw.KGW_A_M_MAJOR, H=260) == kgw.KGW_ERROR_MISALIGNED
    assert call_fp8_ex(lib, fmt=3) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, fmt=-1) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, native=2) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, sa=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, fmt=kgw.KGW_SCALES_PACKED_32, sa=FAKE + 2) == kgw.KGW_ERROR_MISALIGNED
    assert call_fp8_ex(lib, fmt=kgw.KGW_SCALES_PACKED, sa=FAKE + 2, T=1000) == kgw.KGW_ERROR_BAD_OFFSETS
    assert call_fp8_ex(lib, out=FAKE, ptrs=FAKE) == kgw.KGW_ERROR_INVALID_VALUE
    # fp8 layouts: A M-major and / or B K-major on the exact path with uint8 scales only
    AM, BK = kgw.KGW_A_M_MAJOR, kgw.KGW_B_K_MAJOR
    assert call_fp8_ex(lib, layout=8) == kgw.KGW_ERROR_INVALID_VALUE
    for lay in (AM, BK, AM | BK):
        assert call_fp8_ex(lib, layout=lay) == kgw.KGW_ERROR_DEVICE            # accepted, no GPU here
        assert call_fp8_ex(lib, layout=lay, native=1) == kgw.KGW_ERROR_UNSUPPORTED
        assert call_fp8_ex(lib, layout=lay, fmt=kgw.KGW_SCALES_PACKED) == kgw.KGW_ERROR_UNSUPPORTED
        assert call_fp8_ex(lib, layout=lay, fmt=kgw.KGW_SCALES_PACKED_32) == kgw.KGW_ERROR_UNSUPPORTED
        assert call_fp8_ex(lib, layout=lay, H=0) == kgw.KGW_SUCCESS           # nothing to write
        assert call_fp8_ex(lib, layout=lay, N=520) == kgw.KGW_ERROR_MISALIGNED
    assert call_fp8_ex(lib, layout=kgw.KGW_RAGGED | BK) == kgw.KGW_ERROR_DEVICE     # ragged blocks accepted
    assert call_fp8_ex(lib, layout=kgw.KGW_RAGGED | BK, native=1) == kgw.KGW_ERROR_UNSUPPORTED
    assert call_fp8_ex(lib, layout=kgw.KGW_RAGGED) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, layout=kgw.KGW_RAGGED | AM | BK) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_fp8_ex(lib, layout=AM, H=264) == kgw.KGW_ERROR_MISALIGNED      # fp8 M-major rows: hidden % 16
    assert call_fp8_ex(lib, layout=BK, H=264) == kgw.KGW_ERROR_DEVICE
    assert call_fp8_ex(lib, layout=AM, H=1 << 25) == kgw.KGW_ERROR_UNSUPPORTED  # 32-bit row offsets
    assert call_bf16_ex(lib, layout=AM, H=1 << 24) == kgw.KGW_ERROR_UNSUPPORTED


def test_quantizer_argument_errors(lib):
    q = lib.kgw_quantize_fp8
    assert q(FAKE, 256, 256, 1, 3, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # unknown format
    assert q(FAKE, 256, 256, 2, 0, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # unknown axis
    assert q(FAKE, 256, 200, 1, 2, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # tokens % 128
    assert q(FAKE, 256, 256, 0, 2, FAKE, FAKE + 4, None) == kgw.KGW_ERROR_MISALIGNED     # packed-32 needs 16 B
    assert q(FAKE, 256, 256, 0, 0, FAKE, FAKE + 4, None) == kgw.KGW_ERROR_MISALIGNED     # bytes, rows: 8 B
    assert q(FAKE, 0, 256, 1, 1, None, None, None) == kgw.KGW_SUCCESS                    # empty


def test_fp4_quantizer_argument_errors(lib):
    q = lib.kgw_quantize_fp4
    assert q(FAKE, 256, 256, 1, kgw.KGW_SCALES_PACKED, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE   # 128-token bytes
    assert q(FAKE, 256, 256, 1, 3, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # unknown format
    assert q(FAKE, 256, 256, 2, 0, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # unknown axis
    assert q(FAKE, 256, 224, 1, 0, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE      # tokens % 128
    assert q(FAKE, 96, 256, 0, 2, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE       # tokens (rows) % 128
    assert q(FAKE, 256, 252, 0, 0, FAKE, FAKE, None) == kgw.KGW_ERROR_MISALIGNED         # cols % 8
    assert q(FAKE, 256, 256, 0, 2, FAKE, FAKE + 4, None) == kgw.KGW_ERROR_MISALIGNED     # packed-32 needs 16 B
    assert q(FAKE, 256, 256, 0, 0, FAKE, FAKE + 4, None) == kgw.KGW_ERROR_MISALIGNED     # bytes, rows: 8 B
    assert q(FAKE + 8, 256, 256, 1, 2, FAKE, FAKE, None) == kgw.KGW_ERROR_MISALIGNED     # x needs 16 B
    assert q(FAKE, 0, 256, 1, 2, None, None, None) == kgw.KGW_SUCCESS                    # empty
    assert q(None, 256, 256, 1, 2, FAKE, FAKE, None) == kgw.KGW_ERROR_INVALID_VALUE


def test_scale_shapes():
    import torch
    assert kgw.scale_shape(1280, 7, kgw.KGW_SCALES_U8) == ((10, 7), torch.uint8)
    assert kgw.scale_shape(1280, 7, kgw.KGW_SCALES_PACKED) == ((3, 7), torch.int32)
    assert kgw.scale_shape(1280, 7, kgw.KGW_SCALES_PACKED_32) == ((10, 7), torch.int32)
    with pytest.raises(ValueError):
        kgw.scale_shape(1280, 7, 5)


def call_mg(lib, A=FAKE, W=FAKE, layout=0, off=FAKE, idx=None, E=4, M=1024, K=256, N=512, out=FAKE, dt=1, acc=0):
    return lib.kgw_mgrouped_bf16(A, W, layout, off, idx, E, M, K, N, out, dt, acc, None)


def test_mgrouped_argument_errors(lib):
    assert call_mg(lib, layout=2) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg(lib, E=0) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg(lib, off=None, idx=None) == kgw.KGW_ERROR_INVALID_VALUE     # no grouping
    assert call_mg(lib, off=FAKE, idx=FAKE) == kgw.KGW_ERROR_INVALID_VALUE     # both
    assert call_mg(lib, dt=5) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg(lib, acc=3) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg(lib, K=96) == kgw.KGW_ERROR_MISALIGNED                      # K % 64
    assert call_mg(lib, N=500) == kgw.KGW_ERROR_MISALIGNED                     # N % 8
    assert call_mg(lib, A=FAKE + 8) == kgw.KGW_ERROR_MISALIGNED
    assert call_mg(lib, off=FAKE + 2) == kgw.KGW_ERROR_MISALIGNED
    assert call_mg(lib, K=1 << 22) == kgw.KGW_ERROR_UNSUPPORTED
    assert call_mg(lib, E=65537) == kgw.KGW_ERROR_UNSUPPORTED
    assert call_mg(lib, out=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg(lib, M=0, out=None, A=None) == kgw.KGW_SUCCESS              # nothing to do
    assert call_mg(lib, K=0, acc=1, A=None, W=None) == kgw.KGW_SUCCESS          # adds nothing


def call_mg8(lib, A=FAKE, sa=FAKE, W=FAKE, sw=FAKE, off=FAKE, idx=None, E=4, M=1024, K=256, N=512, out=FAKE, dt=1,
             acc=0, layout=0):
    return lib.kgw_mgrouped_fp8(A, sa, W, sw, layout, off, idx, E, M, K, N, out, dt, acc, None)


def test_mgrouped_fp8_argument_errors(lib):
    assert call_mg8(lib, E=0) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, layout=2) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, layout=kgw.KGW_LAYOUT_NN) == kgw.KGW_ERROR_DEVICE       # accepted, no GPU here
    assert call_mg8(lib, layout=kgw.KGW_LAYOUT_NN, N=520) == kgw.KGW_ERROR_MISALIGNED   # nn: N % 16
    assert call_mg8(lib, layout=kgw.KGW_LAYOUT_NT, N=520) == kgw.KGW_ERROR_DEVICE
    assert call_mg8(lib, off=None, idx=None) == kgw.KGW_ERROR_INVALID_VALUE    # no grouping
    assert call_mg8(lib, off=FAKE, idx=FAKE) == kgw.KGW_ERROR_INVALID_VALUE    # both
    assert call_mg8(lib, dt=5) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, acc=3) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, sa=None) == kgw.KGW_ERROR_INVALID_VALUE               # scales required
    assert call_mg8(lib, sw=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, K=192) == kgw.KGW_ERROR_MISALIGNED                    # K % 128 (one scale block)
    assert call_mg8(lib, N=500) == kgw.KGW_ERROR_MISALIGNED                    # N % 8
    assert call_mg8(lib, W=FAKE + 8) == kgw.KGW_ERROR_MISALIGNED
    assert call_mg8(lib, sa=FAKE + 1) != kgw.KGW_ERROR_MISALIGNED              # scale bytes: any address
    assert call_mg8(lib, idx=FAKE + 2, off=None) == kgw.KGW_ERROR_MISALIGNED
    assert call_mg8(lib, K=1 << 22) == kgw.KGW_ERROR_UNSUPPORTED
    assert call_mg8(lib, E=65537) == kgw.KGW_ERROR_UNSUPPORTED
    assert call_mg8(lib, out=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert call_mg8(lib, M=0, out=None, A=None) == kgw.KGW_SUCCESS             # nothing to do
    assert call_mg8(lib, K=0, acc=1, A=None, W=None, sa=None, sw=None) == kgw.KGW_SUCCESS   # adds nothing


def test_mgrouped_fp8_binding_rejects_bad_tensors():
    import torch
    A = torch.zeros(256, 256, dtype=torch.uint8)
    W = torch.zeros(2, 32, 256, dtype=torch.uint8)
    sa = torch.zeros(2, 256, dtype=torch.uint8)
    sw = torch.zeros(2, 2, 32, dtype=torch.uint8)
    off = torch.tensor([128, 256], dtype=torch.int32)
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa, W, sw)                                      # no grouping
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa.t().contiguous(), W, sw, offsets=off)        # scales must be (K/128, M)
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa, W, sw[:, :, :16].contiguous(), offsets=off)
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A[:, :192].contiguous(), sa[:1].contiguous(), W[:, :, :192].contiguous(),
                             sw[:, :1].contiguous(), offsets=off)               # K % 128
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A.to(torch.bfloat16), sa, W, sw, offsets=off)      # not fp8
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa, W, sw, offsets=off[:1])
    with pytest.raises(ValueError):
        kgw.kgw_wgrad_fp8_ex(A, sa, W[0], sw[0], off, b_major="m")
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa, W, sw, offsets=off, layout="tt")
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_fp8(A, sa, W, sw, offsets=off, layout="nn")           # K mismatch for nn


def test_mgrouped_binding_rejects_bad_tensors():
    import torch
    A = torch.zeros(256, 64, dtype=torch.bfloat16)
    W = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    off = torch.tensor([128, 256], dtype=torch.int32)
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_bf16(A, W)                                              # no grouping
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_bf16(A, W, offsets=off, layout="tt")
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_bf16(A, W, offsets=off, layout="nn")                    # K mismatch for nn
    with pytest.raises(ValueError):
        kgw.kgw_mgrouped_bf16(A, W, offsets=off[:1])


def test_fp4_argument_errors(lib):
    f = lambda **k: lib.kgw_wgrad_fp4(k.get("A", FAKE), k.get("sa", FAKE), FAKE, k.get("sb", FAKE), FAKE, 4,
                                      256, k.get("N", 512), k.get("T", 1024), FAKE, None, 1, 0, None, 0, None)
    assert f(T=896) == kgw.KGW_ERROR_BAD_OFFSETS            # 256-token alignment
    assert f(sa=None) == kgw.KGW_ERROR_INVALID_VALUE
    assert f(sa=FAKE + 2) == kgw.KGW_ERROR_MISALIGNED       # packed scale words
    assert f(N=500) == kgw.KGW_ERROR_MISALIGNED
    assert f(A=FAKE + 8) == kgw.KGW_ERROR_MISALIGNED


def test_check_offsets_argument_errors(lib):
    # kgw_check_offsets rejects bad arguments on the host before touching a device
    bad = kgw.KGW_ERROR_INVALID_VALUE
    assert lib.kgw_check_offsets(None, 4, 1024, 256, FAKE, None) == bad
    assert lib.kgw_check_offsets(FAKE, 4, 1024, 256, None, None) == bad
    assert lib.kgw_check_offsets(FAKE, 0, 1024, 256, FAKE, None) == bad
    assert lib.kgw_check_offsets(FAKE, 4, 1024, 0, FAKE, None) == bad
    assert lib.kgw_check_offsets(FAKE, 4, -1, 256, FAKE, None) == bad
    assert lib.kgw_check_offsets(FAKE + 2, 4, 1024, 256, FAKE, None) == kgw.KGW_ERROR_MISALIGNED
    assert lib.kgw_check_offsets(FAKE, 70000, 1024, 256, FAKE, None) == kgw.KGW_ERROR_UNSUPPORTED


def test_wgrad_wrapper_checks_offsets_by_default():
    # The high-level wrapper validates offsets unless told not to (the cuDNN wrapper rejects
    # malformed offsets); the raw kgw_wgrad_* bindings stay asynchronous and do not.
    import inspect
    assert inspect.signature(kgw.wgrad).parameters["check"].default is True
    for fn in (kgw.kgw_wgrad_bf16, kgw.kgw_wgrad_fp8, kgw.kgw_wgrad_fp8_native, kgw.kgw_wgrad_bf16_ex,
               kgw.kgw_wgrad_fp8_ex, kgw.kgw_wgrad_fp4):
        assert inspect.signature(fn).parameters["validate"].default is False, fn.__name__


def test_noalloc_entry_point_argument_errors(lib):
    # the no-alloc variant shares kgw_wgrad_bf16's host checks (no device touched)
    f = lib.kgw_wgrad_bf16_noalloc
    assert f(FAKE, FAKE, FAKE, 0, 256, 512, 1024, FAKE, 0, 0, None) == kgw.KGW_ERROR_INVALID_VALUE
    assert f(FAKE, FAKE, FAKE, 4, 256, 512, 1024, None, 0, 0, None) == kgw.KGW_ERROR_INVALID_VALUE
    assert f(FAKE, FAKE, FAKE, 4, 256, 512, 1000, FAKE, 0, 0, None) == kgw.KGW_ERROR_BAD_OFFSETS
    assert f(FAKE, FAKE, FAKE, 4, 256, 516, 1024, FAKE, 0, 0, None) == kgw.KGW_ERROR_MISALIGNED
    assert f(FAKE, FAKE, FAKE, 4, 256, 512, 1024, FAKE, 3, 0, None) == kgw.KGW_ERROR_INVALID_VALUE
    assert f(None, None, FAKE, 4, 0, 512, 1024, None, 0, 0, None) == kgw.KGW_SUCCESS      # no output elements


def test_mfma_ceiling_argument_errors(lib):
    f = lib.kgw_mfma_ceiling
    bad = kgw.KGW_ERROR_INVALID_VALUE
    assert f(None, 1 << 20, 0, 100, 256, FAKE, None) == bad
    assert f(FAKE, 1 << 20, 0, 100, 256, None, None) == bad
    assert f(FAKE, 1024, 0, 100, 256, FAKE, None) == bad            # fewer than 4096 bytes
    assert f(FAKE, 1 << 20, 4, 100, 256, FAKE, None) == bad         # unknown kind
    assert f(FAKE, 1 << 20, -1, 100, 256, FAKE, None) == bad
    assert f(FAKE, 1 << 20, 0, 0, 256, FAKE, None) == bad
    assert f(FAKE, 1 << 20, 0, 100, 0, FAKE, None) == bad
    assert f(FAKE + 2, 1 << 20, 0, 100, 256, FAKE, None) == kgw.KGW_ERROR_MISALIGNED
    assert f(FAKE, 1 << 20, 0, 100, 256, FAKE + 4, None) == kgw.KGW_ERROR_MISALIGNED
