"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something other than itself: a worked
example, a library decoder, a closed form, an invariant the operation must
satisfy, or a brute-force product computed independently with numpy.  They
are chosen so that a dropped term, a wrong sign, an off-by-one token range
or a transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float values that are exact in bf16 -> uint16 bit patterns (test-side, independent of the oracle)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def brute_force(A64, B64, counts):
    """Independent per-expert product with numpy float64 matmul."""
    out = []
    start = 0
    for c in counts:
        out.append(A64[:, start:start + c] @ B64[start:start + c, :])
        start += c
    return np.stack(out)


# ----------------------------------------------------------------------------
# worked example and offsets decode
# ----------------------------------------------------------------------------
def test_hand_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    A = bf16_bits(np.array(g["A"], dtype=np.float32))
    B = bf16_bits(np.array(g["B"], dtype=np.float32))
    off = np.array(g["offsets"], dtype=np.int32)
    W = oracle.wgrad_bf16(A, B, off)
    np.testing.assert_array_equal(W, np.array(g["wgrad"], dtype=np.float64))
    acc = oracle.apply_output_mode(W, True, np.ones_like(W))
    np.testing.assert_array_equal(acc, np.array(g["accumulate_onto_ones"], dtype=np.float64))


def test_expert_range_inclusive_cumsum(oracle_lib):
    off = np.array([256, 256, 768, 1024], dtype=np.int32)
    assert [oracle.expert_range(off, e) for e in range(4)] == [(0, 256), (256, 256), (256, 768), (768, 1024)]


# ----------------------------------------------------------------------------
# format decoders against library decoders and printed spec values
# ----------------------------------------------------------------------------
def test_bf16_decoder_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3fn_decoder_all_patterns(oracle_lib):
    bits = np.arange(256, dtype=np.int32).astype(np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3fn_value(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # spec values: largest finite, smallest subnormal, smallest normal, NaN, signed zero
    assert oracle.e4m3fn_value(0x7E) == 448.0
    assert oracle.e4m3fn_value(0x01) == 2.0 ** -9
    assert oracle.e4m3fn_value(0x08) == 2.0 ** -6
    assert np.isnan(oracle.e4m3fn_value(0x7F)) and np.isnan(oracle.e4m3fn_value(0xFF))
    assert np.signbit(oracle.e4m3fn_value(0x80))


def test_e8m0_decoder(oracle_lib):
    bits = np.arange(256, dtype=np.int32).astype(np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_value(int(b)) for b in bits])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(128) == 2.0 and oracle.e8m0_value(126) == 0.5


# ----------------------------------------------------------------------------
# the product: brute force, special cases, invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bf16_matches_numpy_brute_force(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 7))
    counts = [int(x) for x in rng.integers(0, 5, size=E) * 8]
    counts[int(rng.integers(0, E))] = 0
    H, N = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    T = sum(counts)
    A = bf16_bits(rng.standard_normal((H, T)))
    B = bf16_bits(rng.standard_normal((T, N)))
    off = workloads.offsets_from_counts(counts)
    W = oracle.wgrad_bf16(A, B, off)
    ref = brute_force(bf16_to_f64(A), bf16_to_f64(B), counts)
    assert W.shape == (E, H, N)
    np.testing.assert_allclose(W, ref, rtol=1e-12, atol=1e-12)


def test_single_expert_is_plain_gemm(oracle_lib):
    rng = np.random.default_rng(7)
    H, T, N = 17, 64, 23
    A = bf16_bits(rng.standard_normal((H, T)))
    B = bf16_bits(rng.standard_normal((T, N)))
    W = oracle.wgrad_bf16(A, B, np.array([T], dtype=np.int32))
    ref = torch.from_numpy(bf16_to_f64(A)) @ torch.from_numpy(bf16_to_f64(B))
    np.testing.assert_allclose(W[0], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sum_over_experts_is_full_product(oracle_lib):
    rng = np.random.default_rng(8)
    counts = [32, 0, 96, 64, 0, 32]
    H, N = 24, 40
    T = sum(counts)
    A = bf16_bits(rng.standard_normal((H, T)))
    B = bf16_bits(rng.standard_normal((T, N)))
    W = oracle.wgrad_bf16(A, B, workloads.offsets_from_counts(counts))
    full = bf16_to_f64(A) @ bf16_to_f64(B)
    np.testing.assert_allclose(W.sum(axis=0), full, rtol=1e-11, atol=1e-11)


def test_integer_inputs_are_exact(oracle_lib):
    rng = np.random.default_rng(9)
    counts = [256, 0, 512, 256]
    H, N = 20, 33
    T = sum(counts)
    Ai = rng.integers(-4, 5, size=(H, T))
    Bi = rng.integers(-4, 5, size=(T, N))
    W = oracle.wgrad_bf16(bf16_bits(Ai), bf16_bits(Bi), workloads.offsets_from_counts(counts))
    start = 0
    for e, c in enumerate(counts):
        exact = Ai[:, start:start + c].astype(np.int64) @ Bi[start:start + c].astype(np.int64)
        assert np.array_equal(W[e], exact.astype(np.float64))
        start += c


def test_empty_experts_are_zero(oracle_lib):
    rng = np.random.default_rng(10)
    H, N = 8, 8
    A = bf16_bits(rng.standard_normal((H, 0)))
    B = bf16_bits(rng.standard_normal((0, N)))
    W = oracle.wgrad_bf16(A, B, np.array([0, 0, 0], dtype=np.int32))
    assert W.shape == (3, H, N) and np.all(W == 0.0)
    counts = [0, 16, 0]
    A = bf16_bits(rng.standard_normal((H, 16)))
    B = bf16_bits(rng.standard_normal((16, N)))
    W = oracle.wgrad_bf16(A, B, workloads.offsets_from_counts(counts))
    assert np.all(W[0] == 0.0) and np.all(W[2] == 0.0) and np.any(W[1] != 0.0)


def test_power_of_two_scaling_is_exact(oracle_lib):
    rng = np.random.default_rng(11)
    counts = [48, 80]
    H, N = 12, 20
    A = rng.standard_normal((H, 128)).astype(np.float32)
    B = bf16_bits(rng.standard_normal((128, N)))
    off = workloads.offsets_from_counts(counts)
    W1 = oracle.wgrad_bf16(bf16_bits(A), B, off)
    W2 = oracle.wgrad_bf16(bf16_bits(bf16_to_f64(bf16_bits(A)) * 2.0), B, off)
    assert np.array_equal(W2, 2.0 * W1)


def test_token_permutation_within_expert(oracle_lib):
    rng = np.random.default_rng(12)
    counts = [64, 96]
    H, N = 10, 14
    A = bf16_bits(rng.standard_normal((H, 160)))
    B = bf16_bits(rng.standard_normal((160, N)))
    off = workloads.offsets_from_counts(counts)
    W = oracle.wgrad_bf16(A, B, off)
    perm = np.concatenate([rng.permutation(64), 64 + rng.permutation(96)])
    Wp = oracle.wgrad_bf16(np.ascontiguousarray(A[:, perm]), np.ascontiguousarray(B[perm]), off)
    np.testing.assert_allclose(Wp, W, rtol=1e-12, atol=1e-12)
    # moving a token across the expert boundary must change both experts
    swap = np.arange(160)
    swap[63], swap[64] = 64, 63
    Ws = oracle.wgrad_bf16(np.ascontiguousarray(A[:, swap]), np.ascontiguousarray(B[swap]), off)
    assert not np.allclose(Ws[0], W[0]) and not np.allclose(Ws[1], W[1])


def test_rows_agree_with_dense(oracle_lib):
    wl = workloads.make_workload("tiny", seed=3)
    W = oracle.wgrad_bf16(wl.A, wl.B, wl.offsets)
    for e in range(wl.num_experts):
        rows = [0, 17, 255]
        np.testing.assert_array_equal(oracle.wgrad_rows_bf16(wl.A, wl.B, wl.offsets, e, rows), W[e][rows])


def test_tiny_config_against_brute_force(oracle_lib):
    wl = workloads.make_workload("tiny", seed=1)
    W = oracle.wgrad_bf16(wl.A, wl.B, wl.offsets)
    ref = brute_force(wl.A.double().numpy(), wl.B.double().numpy(), wl.counts)
    np.testing.assert_allclose(W, ref, rtol=1e-12, atol=1e-10)
    assert np.all(W[1] == 0.0)


# ----------------------------------------------------------------------------
# fp8 block-scaled product
# ----------------------------------------------------------------------------
def dequant(q: torch.Tensor, s: torch.Tensor, token_axis: int, block: int = 128) -> np.ndarray:
    """Library-side dequantisation: torch float8 decode times 2^(s-127) per `block` tokens."""
    v = q.view(torch.float8_e4m3fn).double()
    sc = torch.exp2(s.double() - 127.0).repeat_interleave(block, dim=0)  # (T, other)
    if token_axis == 1:
        sc = sc.t()
    return (v * sc).numpy()


@pytest.mark.parametrize("block", [128, 32])
def test_fp8_matches_dequantised_brute_force(oracle_lib, block):
    counts = [128, 0, 256, 384]
    wl = workloads.make_operands(counts, 24, 40, "fp8", torch.bfloat16, False, seed=5, scale_block=block)
    assert wl.sfa.shape == (768 // block, 24)
    W = oracle.wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, block=block)
    ref = brute_force(dequant(wl.A, wl.sfa, 1, block), dequant(wl.B, wl.sfb, 0, block), counts)
    np.testing.assert_allclose(W, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("block", [128, 32])
def test_fp8_block_scale_byte_doubles_its_block(oracle_lib, block):
    counts = [256, 128]
    wl = workloads.make_operands(counts, 8, 16, "fp8", torch.bfloat16, False, seed=6, scale_block=block)
    W = oracle.wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, block=block)
    # contribution of token block 1 (tokens block..2*block-1, inside expert 0) to row 3
    A1 = wl.A.clone()
    A1[:, :block] = 0  # zero e4m3 byte is +0
    A1[:, 2 * block:] = 0
    part = oracle.wgrad_fp8(A1, wl.sfa, wl.B, wl.sfb, wl.offsets, block=block)
    sfa2 = wl.sfa.clone()
    sfa2[1, 3] += 1
    W2 = oracle.wgrad_fp8(wl.A, sfa2, wl.B, wl.sfb, wl.offsets, block=block)
    np.testing.assert_allclose(W2[0, 3] - W[0, 3], part[0, 3], rtol=1e-12, atol=1e-12)
    mask = np.ones_like(W, dtype=bool)
    mask[0, 3] = False
    assert np.array_equal(W2[mask], W[mask])
    # the same through B: doubling block 1's scale of column 5 adds its contribution once more
    B1 = wl.B.clone()
    B1[:block] = 0
    B1[2 * block:] = 0
    partb = oracle.wgrad_fp8(wl.A, wl.sfa, B1, wl.sfb, wl.offsets, block=block)
    sfb2 = wl.sfb.clone()
    sfb2[1, 5] += 1
    W3 = oracle.wgrad_fp8(wl.A, wl.sfa, wl.B, sfb2, wl.offsets, block=block)
    np.testing.assert_allclose(W3[0, :, 5] - W[0, :, 5], partb[0, :, 5], rtol=1e-12, atol=1e-12)


def test_fp8_block_size_matters(oracle_lib):
    # reading 32-token scales as 128-token ones (or the reverse) must change the result
    counts = [256]
    wl = workloads.make_operands(counts, 8, 16, "fp8", torch.bfloat16, False, seed=9, scale_block=32)
    W = oracle.wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, block=32)
    ref = brute_force(dequant(wl.A, wl.sfa, 1, 32), dequant(wl.B, wl.sfb, 0, 32), counts)
    np.testing.assert_allclose(W, ref, rtol=1e-12, atol=1e-12)
    wrong = brute_force(dequant(wl.A, wl.sfa[::4].contiguous(), 1, 128),
                        dequant(wl.B, wl.sfb[::4].contiguous(), 0, 128), counts)
    assert not np.allclose(W, wrong, rtol=1e-3)


# ----------------------------------------------------------------------------
# packed scale words (reading: four consecutive blocks per little-endian int32,
# block 4w + j in byte j of word (w, m), zero bytes past the last block)
# ----------------------------------------------------------------------------
def test_pack_scales_hand_example(oracle_lib):
    # five blocks of two columns: column 0 holds 1, 3, 5, 7, 9 and column 1 holds 2, 4, ..., 10
    s = np.arange(1, 11, dtype=np.uint8).reshape(5, 2)
    w = oracle.pack_scales(s).view(np.uint32)
    assert w.shape == (2, 2)
    assert w.tolist() == [[0x07050301, 0x08060402], [0x00000009, 0x0000000A]]
    assert np.array_equal(oracle.unpack_scales(w.view(np.int32), 5), s)
    # the same words read as bytes in memory order: byte j of a word is its bits 8j..8j+7
    assert w.view(np.uint8)[0].tolist() == [1, 3, 5, 7, 2, 4, 6, 8]


@pytest.mark.parametrize("nblocks", [1, 4, 6, 13])
def test_pack_scales_round_trip_and_generator(oracle_lib, nblocks):
    g = torch.Generator().manual_seed(nblocks)
    s = torch.randint(0, 256, (nblocks, 7), generator=g, dtype=torch.int32).to(torch.uint8)
    w = oracle.pack_scales(s.numpy())
    assert w.shape == ((nblocks + 3) // 4, 7) and w.dtype == np.int32
    assert np.array_equal(oracle.unpack_scales(w, nblocks), s.numpy())
    assert np.array_equal(workloads.pack_scale_words(s).numpy(), w)
    # padding bytes past the last block are zero
    pad = 4 * w.shape[0] - nblocks
    if pad:
        last = w[-1].view(np.uint32)
        assert np.all(last >> np.uint32(8 * (4 - pad)) == 0)


def test_fp8_integer_inputs_are_exact(oracle_lib):
    counts = [128, 256]
    wl = workloads.make_operands(counts, 6, 10, "fp8", torch.bfloat16, False, seed=7, integer_range=8)
    W = oracle.wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets)
    Ai = wl.A.view(torch.float8_e4m3fn).double().numpy().astype(np.int64)
    Bi = wl.B.view(torch.float8_e4m3fn).double().numpy().astype(np.int64)
    assert np.array_equal(W[0], (Ai[:, :128] @ Bi[:128]).astype(np.float64))
    assert np.array_equal(W[1], (Ai[:, 128:] @ Bi[128:]).astype(np.float64))


# ----------------------------------------------------------------------------
# rounding helpers used by the exactness comparisons
# ----------------------------------------------------------------------------
def test_round_to_bf16_matches_library(oracle_lib):
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875])])  # two exact ties
    got = oracle.round_to_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, ref)


def test_bf16_ulp_is_spacing(oracle_lib):
    rng = np.random.default_rng(14)
    x = oracle.round_to_bf16(rng.standard_normal(5000) * 100.0)
    x = x[x > 0]
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    nxt = (bits + 1).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(nxt - x, oracle.bf16_ulp(x))


# ----------------------------------------------------------------------------
# token-axis fp8 quantiser (llm-infra-atlas "05 Grouped GEMM", section 3: 1x128
# blocks, UE8M0 scales; reading: smallest 2^k with amax <= 448 * 2^k, RNE)
# ----------------------------------------------------------------------------
def _e4m3_codes_positive():
    """(code, value) of every finite non-negative e4m3fn code, increasing."""
    out = []
    for b in range(0x7F):               # 0x7F is NaN
        out.append((b, oracle.e4m3fn_value(b)))
    return out


def test_e4m3fn_encode_inverts_the_decoder():
    for b in range(256):
        if b & 0x7F == 0x7F:
            continue
        v = oracle.e4m3fn_value(b)
        assert oracle.e4m3fn_encode(v) == b, hex(b)


def test_e4m3fn_encode_rounds_to_nearest_ties_to_even():
    codes = _e4m3_codes_positive()
    for (b0, v0), (b1, v1) in zip(codes, codes[1:]):
        mid = (v0 + v1) / 2.0
        even = b0 if (b0 & 1) == 0 else b1          # the code with the even last mantissa bit
        assert oracle.e4m3fn_encode(mid) == even, (hex(b0), hex(b1))
        assert oracle.e4m3fn_encode(-mid) == even | 0x80
        eps = (v1 - v0) / 64.0
        assert oracle.e4m3fn_encode(mid - eps) == b0
        assert oracle.e4m3fn_encode(mid + eps) == b1
    assert oracle.e4m3fn_encode(448.0) == 0x7E
    assert oracle.e4m3fn_encode(float("nan")) == 0x7F
    assert oracle.e4m3fn_encode(-0.0) == 0x80


def test_e4m3fn_encode_matches_torch_float8_conversion():
    # a library routine with the same rounding: torch's float32 -> float8_e4m3fn cast
    g = torch.Generator().manual_seed(5)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-12, 9, (20000,), generator=g).float())
    x = x.clamp(-448.0, 448.0)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3fn_encode(float(v)) for v in x.numpy()], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e8m0_for_amax_is_the_smallest_sufficient_power_of_two():
    rng = np.random.default_rng(6)
    amax = np.exp2(rng.uniform(-120, 120, 2000)) * rng.uniform(1, 2, 2000)
    for a in amax:
        e = oracle.e8m0_for_amax(float(a))
        k = e - 127
        assert a <= 448.0 * 2.0 ** k
        if e > 1:                                      # minimal unless clamped at the bottom
            assert a > 448.0 * 2.0 ** (k - 1)
    assert oracle.e8m0_for_amax(448.0) == 127
    assert oracle.e8m0_for_amax(np.nextafter(448.0, 1e9)) == 128
    assert oracle.e8m0_for_amax(1.0) == 119            # 1 <= 448 * 2^-8 = 1.75
    assert oracle.e8m0_for_amax(0.0) == 127
    assert oracle.e8m0_for_amax(1e-45) == 1            # clamped
    assert oracle.e8m0_for_amax(float("inf")) == 255
    assert oracle.e8m0_for_amax(float("nan")) == 255


@pytest.mark.parametrize("block", [128, 32])
@pytest.mark.parametrize("token_axis", [0, 1])
def test_quantizer_matches_the_independent_generator_implementation(token_axis, block):
    # workloads.quantize_token_blocks (torch float8 cast, float64 log2) is written separately
    g = torch.Generator().manual_seed(7)
    shape = (200, 384) if token_axis else (384, 200)
    x = (torch.randn(shape, generator=g) * torch.exp2(torch.randint(-20, 20, (1, shape[1]), generator=g).float())
         ).to(torch.bfloat16)
    q_ref, s_ref = workloads.quantize_token_blocks(x, token_axis=token_axis, block=block)
    q, s = oracle.quantize_fp8_tokens(x, token_axis, block=block)
    assert s.shape == (384 // block, 200)
    assert np.array_equal(s, s_ref.numpy())
    assert np.array_equal(q, q_ref.numpy())


@pytest.mark.parametrize("block", [128, 32])
@pytest.mark.parametrize("token_axis", [0, 1])
def test_quantizer_dequantised_values_are_within_half_an_e4m3_step(token_axis, block):
    g = torch.Generator().manual_seed(8)
    shape = (64, 256) if token_axis else (256, 64)
    x = torch.randn(shape, generator=g).to(torch.bfloat16)
    q, s = oracle.quantize_fp8_tokens(x, token_axis, block=block)
    xs = x.float().numpy().astype(np.float64)
    deq = np.vectorize(oracle.e4m3fn_value)(q)
    scale = np.exp2(s.astype(np.float64) - 127)
    scale_full = np.repeat(scale, block, axis=0)          # (tokens, other)
    if token_axis:
        scale_full = scale_full.T
    v = deq * scale_full
    # within half a step of e4m3 at the element's own binade (3 mantissa bits), or of the
    # subnormal step 2^-9 * scale
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(xs), 1e-300))) - 3), np.exp2(-9) * scale_full)
    assert np.all(np.abs(v - xs) <= step / 2 + 1e-300)
    # every block's largest element, scaled, lies in (224, 448], so after rounding in [224, 448]
    tok_major = deq if not token_axis else deq.T                    # (tokens, other)
    bmax = np.abs(tok_major).reshape(-1, block, tok_major.shape[1]).max(axis=1)
    assert np.all(bmax >= 224) and np.all(bmax <= 448)


def test_quantizer_special_blocks():
    x = torch.randn(256, 4).to(torch.bfloat16)
    x[:128, 0] = 0.0                                      # all-zero block
    x[130, 1] = float("nan")                              # NaN block
    x[5, 2] = float("inf")                                # inf block
    q, s = oracle.quantize_fp8_tokens(x, 0)
    assert s[0, 0] == 127 and np.all(q[:128, 0] == 0)
    assert s[1, 1] == 255 and np.all(q[128:, 1] == 0x7F)
    assert s[0, 2] == 255 and np.all(q[:128, 2] == 0x7F)
    assert s[1, 0] != 255 and s[0, 3] != 255
    with pytest.raises(ValueError):
        oracle.quantize_fp8_tokens(x[:200], 0)
    # 32-token blocks: the NaN at token 130 poisons only block 4 of column 1
    q32, s32 = oracle.quantize_fp8_tokens(x, 0, block=32)
    assert s32[4, 1] == 255 and np.all(q32[128:160, 1] == 0x7F)
    assert np.all(s32[[0, 1, 2, 3, 5, 6, 7], 1] != 255) and np.all(q32[160:, 1] != 0x7F)
    assert s32[0, 2] == 255 and s32[1, 2] != 255
    assert np.all(s32[:4, 0] == 127)
    with pytest.raises(ValueError):
        oracle.quantize_fp8_tokens(x[:240], 0, block=32)


def test_round_to_fp16_ties_overflow_and_ulp():
    # binary16: 10 fraction bits; ties to even; the largest finite is 65504
    assert oracle.round_to_fp16(np.array([1 + 2.0 ** -11]))[0] == 1.0
    assert oracle.round_to_fp16(np.array([1 + 3 * 2.0 ** -11]))[0] == 1 + 2.0 ** -9
    assert oracle.round_to_fp16(np.array([65504.0]))[0] == 65504.0
    assert np.isinf(oracle.round_to_fp16(np.array([65520.0]))[0])
    assert oracle.round_to_fp16(np.array([2.0 ** -25]))[0] == 0.0          # half the smallest subnormal
    assert oracle.fp16_ulp(np.array([1.0]))[0] == 2.0 ** -10
    assert oracle.fp16_ulp(np.array([3000.0]))[0] == 2.0
    assert oracle.fp16_ulp(np.array([2.0 ** -20]))[0] == 2.0 ** -24


# ----------------------------------------------------------------------------
# m-grouped product (forward "nt" and dgrad "nn" of the same experts)
# ----------------------------------------------------------------------------
def test_mgrouped_hand_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "mgrouped_example.json")))
    A = bf16_bits(np.array(g["A"], dtype=np.float64))
    W = bf16_bits(np.array(g["W"], dtype=np.float64))
    off = np.array(g["offsets"], dtype=np.int32)
    assert np.array_equal(oracle.mgrouped_bf16(A, W, offsets=off, layout="nn"), np.array(g["nn_out"], dtype=np.float64))
    assert np.array_equal(oracle.mgrouped_bf16(A, W, offsets=off, layout="nt"), np.array(g["nt_out"], dtype=np.float64))


def _mgrouped_case(counts, K, N, seed, pad_rows=0):
    rng = np.random.default_rng(seed)
    M = sum(counts) + pad_rows
    A = bf16_bits(rng.standard_normal((M, K)))
    W = bf16_bits(rng.standard_normal((len(counts), N, K)))
    return A, W, np.cumsum(counts).astype(np.int32), M


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_mgrouped_matches_numpy_brute_force(oracle_lib, layout):
    counts = [3, 0, 5, 2]
    A, W, off, M = _mgrouped_case(counts, 7, 6, seed=31, pad_rows=2)
    if layout == "nn":
        W = np.ascontiguousarray(W.transpose(0, 2, 1))       # (E, K, N)
    got = oracle.mgrouped_bf16(A, W, offsets=off, layout=layout)
    A64, W64 = bf16_to_f64(A), bf16_to_f64(W)
    start = 0
    for e, c in enumerate(counts):
        Wg = W64[e].T if layout == "nt" else W64[e]
        np.testing.assert_allclose(got[start:start + c], A64[start:start + c] @ Wg, rtol=1e-12, atol=1e-12)
        start += c
    assert np.all(np.isnan(got[start:]))                       # rows past the last offset: no group


def test_mgrouped_nt_equals_nn_on_transposed_weights(oracle_lib):
    A, W, off, M = _mgrouped_case([4, 4, 8], 5, 9, seed=32)
    Wt = np.ascontiguousarray(W.transpose(0, 2, 1))
    assert np.array_equal(oracle.mgrouped_bf16(A, W, offsets=off, layout="nt"),
                          oracle.mgrouped_bf16(A, Wt, offsets=off, layout="nn"))


def test_mgrouped_m_indices_match_offsets_and_mark_padding(oracle_lib):
    counts = [2, 0, 3, 1]
    A, W, off, M = _mgrouped_case(counts, 4, 3, seed=33, pad_rows=2)
    idx = np.concatenate([np.repeat(np.arange(4), counts), [-1, -1]]).astype(np.int32)
    a = oracle.mgrouped_bf16(A, W, offsets=off)
    b = oracle.mgrouped_bf16(A, W, m_indices=idx)
    assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[:6], b[:6])
    # one row moved to another group changes exactly that row
    idx2 = idx.copy()
    idx2[0] = 3
    c = oracle.mgrouped_bf16(A, W, m_indices=idx2)
    assert not np.allclose(c[0], b[0]) and np.array_equal(c[1:6], b[1:6])
    # ids outside [0, E) -- negative or too large -- mark rows of no group
    d = oracle.mgrouped_bf16(A, W, m_indices=np.where(idx == 2, 4, idx).astype(np.int32))
    assert np.all(np.isnan(d[2:5])) and np.array_equal(d[:2], b[:2]) and np.array_equal(d[5:6], b[5:6])


def test_mgrouped_single_group_is_plain_gemm_and_integers_exact(oracle_lib):
    rng = np.random.default_rng(34)
    A = rng.integers(-4, 5, (9, 11)).astype(np.float64)
    W = rng.integers(-4, 5, (1, 6, 11)).astype(np.float64)
    got = oracle.mgrouped_bf16(bf16_bits(A), bf16_bits(W), offsets=np.array([9], dtype=np.int32))
    assert np.array_equal(got, A @ W[0].T)


def test_mgrouped_forward_dgrad_wgrad_trace_identity(oracle_lib):
    # With Y = X W^T per expert (forward), dX = dY W (dgrad) and dW = dY^T X (wgrad, the
    # k-grouped oracle): <Y, dY> = <dX, X> = sum_e <W_e, dW_e>.
    counts = [256, 0, 512, 256]
    T, K, N = sum(counts), 24, 40
    rng = np.random.default_rng(35)
    X = bf16_bits(rng.standard_normal((T, K)))
    dY = bf16_bits(rng.standard_normal((T, N)))
    W = bf16_bits(rng.standard_normal((4, N, K)))
    off = np.cumsum(counts).astype(np.int32)
    Y = oracle.mgrouped_bf16(X, W, offsets=off, layout="nt")                 # (T, N)
    dX = oracle.mgrouped_bf16(dY, W, offsets=off, layout="nn")               # W_e read as (N, K): (T, K)
    dW = oracle.wgrad_bf16(np.ascontiguousarray(dY.T), X, off)               # (E, N, K)
    X64, dY64, W64 = bf16_to_f64(X), bf16_to_f64(dY), bf16_to_f64(W)
    a = float(np.sum(Y * dY64))
    b = float(np.sum(dX * X64))
    c = float(np.sum(W64 * dW))
    assert abs(a - b) <= 1e-9 * max(1.0, abs(a)) and abs(a - c) <= 1e-9 * max(1.0, abs(a))


# ----------------------------------------------------------------------------
# FP4 (e2m1) operands with 32-token UE8M0 scales
# ----------------------------------------------------------------------------
def test_e2m1_decoder_matches_the_format_table(oracle_lib):
    # OCP e2m1: exponent field 0 is subnormal (0, 0.5); 1..3 give 1, 1.5, 2, 3, 4, 6
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == (-1 if c & 8 else 1) * table[c & 7] and (np.signbit(v) == bool(c & 8))


def test_e2m1_encode_round_trip_ties_and_generator():
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for i in range(7):
        mid = (mags[i] + mags[i + 1]) / 2
        assert oracle.e2m1_encode(mid) == (i if i % 2 == 0 else i + 1)           # ties to the even code
        assert oracle.e2m1_encode(mid - 1e-9) == i and oracle.e2m1_encode(mid + 1e-9) == i + 1
    assert oracle.e2m1_encode(100.0) == 7 and oracle.e2m1_encode(-100.0) == 15
    rng = np.random.default_rng(15)
    v = rng.standard_normal(4000) * 3
    v = np.concatenate([v, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.0]])
    assert np.array_equal(workloads.e2m1_codes(v), [oracle.e2m1_encode(x) for x in v])


def test_fp4_quantizer_matches_generator_and_bounds():
    g = torch.Generator().manual_seed(16)
    x = (torch.randn(40, 256, generator=g) * torch.exp2(torch.randint(-10, 10, (40, 1), generator=g).float())
         ).to(torch.bfloat16)
    x[3, 32:64] = 0
    q, s = oracle.quantize_fp4_tokens(x)
    q_ref, s_ref = workloads.quantize_fp4_token_blocks(x)
    assert np.array_equal(q, q_ref.numpy()) and np.array_equal(s, s_ref.numpy())
    assert s[1, 3] == 127 and np.all(q[3, 16:32] == 0)
    # dequantised: every block's largest magnitude lands in [3, 6] (the top binade of e2m1)
    codes = np.stack([q & 15, q >> 4], axis=2).reshape(40, 256)
    vals = np.vectorize(oracle.e2m1_value)(codes) * np.repeat(np.exp2(s.T.astype(np.float64) - 127), 32, axis=1)
    blk = np.abs(vals / np.repeat(np.exp2(s.T.astype(np.float64) - 127), 32, axis=1)).reshape(40, 8, 32).max(axis=2)
    nz = blk > 0
    assert np.all(blk[nz] >= 3) and np.all(blk[nz] <= 6)


def test_fp4_quantizer_special_blocks():
    # closed-form cases of the stated rule: all-zero block -> scale 127 and zero codes; a NaN
    # or an infinity -> scale 0xFF and zero codes; -0 keeps its sign (code 8); amax exactly
    # 6 * 2^k -> byte 127 + k, one bf16 step above -> 128 + k; an amax below 6 * 2^-126 clamps the
    # byte to 1
    def col(vals):
        v = np.zeros(32)
        v[:len(vals)] = vals
        return v
    blocks = [col([]), col([1.0, np.nan]), col([np.inf, 2.0]), col([-0.0, 6.0]),
              col([6.0 * 8, 3.0 * 8]), col([6.0 * 8 * (1 + 2.0 ** -7)]), col([2.0 ** -130])]
    x = torch.tensor(np.concatenate(blocks)[None, :], dtype=torch.float32).to(torch.bfloat16)
    q, s = oracle.quantize_fp4_tokens(x)
    assert s[:, 0].tolist() == [127, 255, 255, 127, 130, 131, 1]
    codes = np.stack([q[0] & 15, q[0] >> 4], axis=1).reshape(-1)
    assert np.all(codes[0:32] == 0) and np.all(codes[32:64] == 0) and np.all(codes[64:96] == 0)
    assert codes[96] == 8 and codes[97] == 7                         # -0 and 6 at scale 2^0
    assert codes[128] == 7 and codes[129] == 5                      # 48 and 24 at scale 2^3: 6 and 3
    assert codes[160] == 5                                          # bf16(48.375) = 48.5 at 2^4: 3.03 -> 3
    assert codes[192] == 0                                          # 2^-130 (a bf16 subnormal) at 2^-126: 1/16


def _dequant_fp4(q, s):
    codes = np.stack([q & 15, q >> 4], axis=2).reshape(q.shape[0], -1)
    return np.vectorize(oracle.e2m1_value)(codes) * np.repeat(np.exp2(s.T.astype(np.float64) - 127), 32, axis=1)


def test_fp4_product_matches_dequantised_brute_force():
    counts = [64, 0, 128, 96]
    wl = workloads.make_fp4_operands(counts, 12, 20, seed=17)
    W = oracle.wgrad_fp4(wl["A"], wl["sfa"], wl["B"], wl["sfb"], wl["offsets"])
    A = _dequant_fp4(wl["A"].numpy(), wl["sfa"].numpy())          # (hidden, T)
    B = _dequant_fp4(wl["B"].numpy(), wl["sfb"].numpy())          # (n, T)
    start = 0
    for e, c in enumerate(counts):
        np.testing.assert_allclose(W[e], A[:, start:start + c] @ B[:, start:start + c].T, rtol=1e-12, atol=1e-12)
        start += c


def test_fp4_nibble_order_hand_example():
    # one expert of 32 tokens, hidden = n = 1: A tokens 0, 1 are 1 and 2 (byte 0x42: 2 is code 4 in
    # the high nibble), B tokens 0, 1 are 3 and 0.5 (byte 0x15); every other code 0; scales 1
    A = np.zeros((1, 16), dtype=np.uint8)
    B = np.zeros((1, 16), dtype=np.uint8)
    A[0, 0], B[0, 0] = 0x42, 0x15
    s = np.full((1, 1), 127, dtype=np.uint8)
    W = oracle.wgrad_fp4(A, s, B, s, np.array([32], dtype=np.int32))
    assert W[0, 0, 0] == 1.0 * 3.0 + 2.0 * 0.5
    s2 = s.copy()
    s2[0, 0] = 129                                                  # A's block scaled by 4
    assert oracle.wgrad_fp4(A, s2, B, s, np.array([32], dtype=np.int32))[0, 0, 0] == 4 * (1.0 * 3.0 + 2.0 * 0.5)


def test_fp4_integer_operands_exact():
    counts = [96, 160]
    wl = workloads.make_fp4_operands(counts, 7, 9, seed=18, integer_range=6)
    W = oracle.wgrad_fp4(wl["A"], wl["sfa"], wl["B"], wl["sfb"], wl["offsets"])
    A = _dequant_fp4(wl["A"].numpy(), wl["sfa"].numpy())
    B = _dequant_fp4(wl["B"].numpy(), wl["sfb"].numpy())
    assert np.all(A == np.round(A))
    assert np.array_equal(W[0], (A[:, :96].astype(np.int64) @ B[:, :96].astype(np.int64).T).astype(np.float64))
    assert np.array_equal(W[1], (A[:, 96:].astype(np.int64) @ B[:, 96:].astype(np.int64).T).astype(np.float64))


def test_thread_count_does_not_change_results():
    # every output row is summed in the same token order whatever the OpenMP thread count
    g = torch.Generator().manual_seed(7)
    A = torch.randn((64, 512), generator=g).to(torch.bfloat16)
    B = torch.randn((512, 96), generator=g).to(torch.bfloat16)
    off = torch.tensor([256, 512], dtype=torch.int32)
    threads = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        one = oracle.wgrad_bf16(A, B, off)
        oracle.set_num_threads(max(2, threads))
        many = oracle.wgrad_bf16(A, B, off)
    finally:
        oracle.set_num_threads(threads)
    assert np.array_equal(one, many)


# ----------------------------------------------------------------------------
# fp8 m-grouped forward product (llm-infra-atlas section 2.1 / section 3)
# ----------------------------------------------------------------------------
FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _e4m3_f64(codes):
    # torch's own e4m3fn decoder: independent of the oracle's
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _fp8_mgrouped_case(counts, K, N, seed, pad_rows=0):
    rng = np.random.default_rng(seed)
    M, E = sum(counts) + pad_rows, len(counts)
    A = rng.choice(FINITE_E4M3, (M, K))
    W = rng.choice(FINITE_E4M3, (E, N, K))
    sa = rng.integers(118, 137, (K // 128, M)).astype(np.uint8)
    sw = rng.integers(118, 137, (E, K // 128, N)).astype(np.uint8)
    return A, sa, W, sw, np.cumsum(counts).astype(np.int32), M


def _dequant_rows(codes, scales_kb_by_row):
    # codes (R, K); scales (K/128, R) -> values (R, K), each scale repeated over its 128 values
    return _e4m3_f64(codes) * np.exp2(np.repeat(scales_kb_by_row.T.astype(np.float64) - 127.0, 128, axis=1))


def test_mgrouped_fp8_matches_brute_force(oracle_lib):
    counts = [3, 0, 5, 2]
    A, sa, W, sw, off, M = _fp8_mgrouped_case(counts, 256, 6, seed=41, pad_rows=2)
    got = oracle.mgrouped_fp8(A, sa, W, sw, offsets=off)
    a = _dequant_rows(A, sa)
    start = 0
    for e, c in enumerate(counts):
        w = _dequant_rows(W[e], sw[e])                           # (N, K)
        want = a[start:start + c] @ w.T
        np.testing.assert_allclose(got[start:start + c], want, rtol=1e-12, atol=1e-12 * np.abs(want).max(initial=1))
        start += c
    assert np.all(np.isnan(got[start:]))                         # rows past the last offset: no group


def test_mgrouped_fp8_integers_unit_scales_exact_single_group(oracle_lib):
    rng = np.random.default_rng(42)
    Ai = rng.integers(-8, 9, (5, 256)).astype(np.float64)
    Wi = rng.integers(-8, 9, (1, 7, 256)).astype(np.float64)
    A = torch.from_numpy(Ai).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    W = torch.from_numpy(Wi).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sa = np.full((2, 5), 127, np.uint8)
    sw = np.full((1, 2, 7), 127, np.uint8)
    got = oracle.mgrouped_fp8(A, sa, W, sw, offsets=np.array([5], dtype=np.int32))
    assert np.array_equal(got, Ai @ Wi[0].T)


def test_mgrouped_fp8_scale_byte_doubles_its_block(oracle_lib):
    # only K block 1 of A is nonzero; raising sw[g=0, kb=1, j=2] by one doubles column 2 of
    # group 0's rows, exactly, and changes nothing else
    A, sa, W, sw, off, M = _fp8_mgrouped_case([4, 3], 384, 5, seed=43)
    A[:, :128] = 0
    A[:, 256:] = 0
    base = oracle.mgrouped_fp8(A, sa, W, sw, offsets=off)
    sw2 = sw.copy()
    sw2[0, 1, 2] += 1
    got = oracle.mgrouped_fp8(A, sa, W, sw2, offsets=off)
    assert np.array_equal(got[:4, 2], 2 * base[:4, 2])
    keep = np.ones_like(got, dtype=bool)
    keep[:4, 2] = False
    assert np.array_equal(got[keep], base[keep])
    # and a scale of A's row 5 in block 1 doubles that row (group 1) only
    sa2 = sa.copy()
    sa2[1, 5] += 1
    got2 = oracle.mgrouped_fp8(A, sa2, W, sw, offsets=off)
    assert np.array_equal(got2[5], 2 * base[5]) and np.array_equal(np.delete(got2, 5, 0), np.delete(base, 5, 0))


def test_mgrouped_fp8_m_indices_match_offsets(oracle_lib):
    counts = [2, 0, 3]
    A, sa, W, sw, off, M = _fp8_mgrouped_case(counts, 128, 4, seed=44, pad_rows=1)
    idx = np.concatenate([np.repeat(np.arange(3), counts), [-1]]).astype(np.int32)
    a = oracle.mgrouped_fp8(A, sa, W, sw, offsets=off)
    b = oracle.mgrouped_fp8(A, sa, W, sw, m_indices=idx)
    assert np.array_equal(a[:5], b[:5]) and np.all(np.isnan(a[5])) and np.all(np.isnan(b[5]))
