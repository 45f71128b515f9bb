/*
 * kgw.h -- K-grouped MoE weight-gradient GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation (cuDNN "Grouped GEMM + WGrad (Unified)", section "Operation";
 * llm-infra-atlas "05 Grouped GEMM", section 5.2 "wgrad: k-grouped GEMM"):
 * for expert e, with begin = 0 for e == 0 and offsets[e-1] otherwise and
 * end = offsets[e],
 *
 *     Wgrad[e] = A[:, begin:end] @ B[begin:end, :]
 *
 * The contracted axis is the token axis; each expert's token count is only
 * known on the device.  One call computes every expert in one persistent
 * kernel launch on `stream`.
 *
 * Conventions shared by every entry point
 *  - Pointers named A, B, sfa, sfb, offsets, out and workspace are DEVICE
 *    pointers on the current HIP device.  The caller owns every buffer and
 *    keeps it alive until the work queued on `stream` has finished (same
 *    page, section "Output modes": caller-owned allocations).
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *  - Calls are asynchronous and stream-ordered: no device-to-host transfer,
 *    no synchronisation, no allocation (except kgw_validate_offsets, which is
 *    documented as synchronous).  The library keeps no mutable global state
 *    other than a per-device property cache; it is thread-safe.
 *  - Errors are returned as kgw_status_t; nothing is thrown across the ABI.
 *    Every argument check happens on the host before anything is enqueued, so
 *    a failed call leaves the output untouched.
 *  - Offsets are NOT read on the host by kgw_wgrad_*.  Malformed offsets
 *    (decreasing, unaligned counts, last value != tokens_sum) are the caller's
 *    to rule out, e.g. with kgw_validate_offsets.  The kernels clamp every
 *    token range into [0, tokens_sum) and round it down to the kernel's K
 *    step, so malformed offsets can give wrong values for the experts they
 *    touch but never an out-of-bounds access.
 */
#ifndef KGW_H
#define KGW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  The cuDNN page (section "Scheduling, cache, and errors")
 * splits its errors into ValueError (contract violations) and RuntimeError
 * (device trouble); the Python binding maps codes 1-4 to ValueError and 5 to
 * RuntimeError. */
typedef enum {
    KGW_SUCCESS = 0,
    KGW_ERROR_INVALID_VALUE = 1, /* NULL pointer where data is needed, num_experts < 1,
                                    negative size, unknown out_dtype, accumulate not 0/1   */
    KGW_ERROR_MISALIGNED = 2,    /* a pointer not 16-byte aligned, or n not a multiple of
                                    8 (bf16) / 16 (fp8) elements                           */
    KGW_ERROR_BAD_OFFSETS = 3,   /* decreasing offsets, a count not a multiple of the
                                    alignment or offsets[E-1] != tokens_sum (from the
                                    kgw_validate_offsets* calls); tokens_sum not a multiple
                                    of the alignment (from every call)                     */
    KGW_ERROR_UNSUPPORTED = 4,   /* a size beyond what the kernels index (see below)       */
    KGW_ERROR_DEVICE = 5         /* no HIP device, device is not gfx950, or a HIP call or
                                    kernel launch failed                                   */
} kgw_status_t;

/* Output element type of the dense (num_experts, hidden, n) result.  The fp32
 * accumulators are rounded once, to nearest even, into a 16-bit type (fp16
 * overflows to infinity); the cuDNN page, "BF16 contract" table, lists fp32,
 * bf16 and fp16 outputs. */
typedef enum {
    KGW_OUT_FP32 = 0,
    KGW_OUT_BF16 = 1,
    KGW_OUT_FP16 = 2
} kgw_out_dtype_t;

/* Layout of the UE8M0 scales of an fp8 operand (mn = hidden for sfa, n for sfb).
 * The llm-infra-atlas page, section 3, keeps the scales mn-major with packed
 * 8-bit exponents, and the DeepGEMM k-grouped page casts with gran_k = 32 and
 * use_packed_ue8m0; neither prints the packed layout.  Reading taken here: four
 * consecutive token blocks share one little-endian 32-bit word, block 4w + j in
 * byte j of word (w, m); bytes past the last block are zero (written so by
 * kgw_quantize_fp8, ignored by the GEMMs).
 *   KGW_SCALES_U8         one byte per 128 tokens: uint8 (tokens_sum/128, mn).
 *   KGW_SCALES_PACKED     one byte per 128 tokens, packed: int32
 *                         (ceil(tokens_sum/512), mn).
 *   KGW_SCALES_PACKED_32  one byte per 32 tokens (MX-style blocks), packed: int32
 *                         (tokens_sum/128, mn) -- word (w, m) holds the scales of
 *                         tokens 128w + 32j .. 128w + 32j + 31 in byte j; 4-byte
 *                         aligned (16-byte for kgw_quantize_fp8's output). */
typedef enum {
    KGW_SCALES_U8 = 0,
    KGW_SCALES_PACKED = 1,
    KGW_SCALES_PACKED_32 = 2
} kgw_scale_format_t;

/* Token-count alignment each entry point requires (cuDNN page, section "BF16
 * contract": every count a multiple of 256 for BF16; for fp8 one UE8M0 scale
 * block, llm-infra-atlas section 3, is 128 tokens). */
#define KGW_BF16_TOKEN_ALIGN 256
#define KGW_FP8_TOKEN_ALIGN 128
/* FP4 stages hold 256 tokens (one 128-byte line per operand row). */
#define KGW_FP4_TOKEN_ALIGN 256

/*
 * kgw_wgrad_bf16 -- bf16 operands, fp32 accumulation (cuDNN page, "BF16 contract":
 * FP32 accumulation for BF16 inputs).
 *
 *   A        bf16 (hidden, tokens_sum), row-major: the token axis is contiguous
 *            (the page's K-major A, stride (tokens_sum, 1)).
 *   B        bf16 (tokens_sum, n), row-major (the page's N-major B, stride (n, 1)).
 *   offsets  int32 (num_experts,), inclusive cumulative token counts.
 *            Contract: non-decreasing, every count a multiple of 256,
 *            offsets[num_experts-1] == tokens_sum.
 *   out      dense (num_experts, hidden, n), row-major, element type out_dtype.
 *   accumulate  1: out[e] += Wgrad[e] (out must be initialised; an empty expert is
 *                  left untouched, bit for bit);
 *               0: out[e]  = Wgrad[e] (an empty expert is written with +0.0).
 *            Section "Operation" of the cuDNN page defines both modes.
 *   workspace, workspace_bytes  device scratch owned by the caller: at least
 *            kgw_workspace_bytes(...) bytes, 16-byte aligned, not used by
 *            another call at the same time; it needs no initial contents.  When
 *            that size is 0 or the workspace is NULL or smaller, the call runs
 *            in one pass on the static schedule.  Otherwise it holds either
 *            (few output tiles) split-K partials: each expert's token range is
 *            cut into chunks whose fp32 partials land in the workspace and a
 *            second pass sums them in chunk order before applying the output
 *            mode once -- the result differs from the one-pass result only by
 *            the order of the fp32 additions -- or (many rounds of output tiles,
 *            at most 64 experts averaging 1024+ tokens) the 256-byte claim
 *            counters of the dynamic schedule, which the call zeroes itself (a
 *            kernel queued before the product) -- the result is bit for bit the
 *            static schedule's, since every tile is still computed whole by one
 *            workgroup (cuDNN page, section "Scheduling, cache, and errors":
 *            dynamic persistent scheduling for the BF16 kernel).
 *
 * Sizes: 1 <= num_experts <= 65536; 0 <= hidden, n < 2^28; tokens_sum >= 0 and a
 * multiple of 256; n a multiple of 8; tokens_sum < 2^31 (int32 offsets).
 * tokens_sum == 0 (or hidden == 0, or n == 0) is valid: overwrite writes zeros,
 * accumulate does nothing; A and B may then be NULL.  A, B and out must be
 * 16-byte aligned.
 */
kgw_status_t kgw_wgrad_bf16(const void* A, const void* B, const int32_t* offsets,
                            int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                            void* out, int32_t out_dtype, int32_t accumulate,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * kgw_wgrad_bf16_noalloc -- kgw_wgrad_bf16 for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, contract, errors and kernels as kgw_wgrad_bf16, minus
 * the workspace: where kgw_wgrad_bf16 would use one (split-K partials, or the dynamic
 * schedule's claim counters), the call uses a fixed 64 MiB scratch array the library
 * holds on every device it runs on (until the process ends), so the result is bit for
 * bit that of kgw_wgrad_bf16 given a workspace of kgw_workspace_bytes(...) bytes.  The
 * split plan keeps chunks x tiles within the compute units and a 256 x 256 fp32 tile
 * takes 256 KiB, so on MI355X's 256 compute units every planned split fits those
 * 64 MiB; on a device with more compute units a plan that would not fit runs in one
 * pass instead (no error: one pass needs no scratch; the result then differs only by
 * the order of the fp32 additions).  The call allocates and frees nothing.
 * All calls on one device share that device's scratch, which keeps the last call's
 * contents (no call needs it to start at zero): two calls that overlap in time on the
 * same device -- on different streams, or from different threads -- race on it and may
 * give wrong results.  Order such calls on one stream or synchronise between them.
 */
kgw_status_t kgw_wgrad_bf16_noalloc(const void* A, const void* B, const int32_t* offsets,
                                    int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                                    void* out, int32_t out_dtype, int32_t accumulate, void* stream);

/* Operand layouts of kgw_wgrad_bf16_ex (cuDNN page, "BF16 contract" table and
 * its input_order), combined as bit flags; 0 is kgw_wgrad_bf16's layout
 * (A K-major: (hidden, tokens_sum) row-major; B N-major: (tokens_sum, n)
 * row-major).  Element (m, t) of A and (t, j) of B then live at:
 *   KGW_A_M_MAJOR  A stored as (tokens_sum, hidden) row-major: A[t * hidden + m]
 *                  (stride (1, hidden)); hidden must be a multiple of 8.
 *   KGW_B_K_MAJOR  B stored as (n, tokens_sum) row-major: B[j * tokens_sum + t]
 *                  (stride (1, tokens_sum)).
 *   KGW_RAGGED     with KGW_B_K_MAJOR and without KGW_A_M_MAJOR only ("tensor_ragged":
 *                  per-expert K-contiguous blocks back to back): expert e's A block
 *                  is (hidden, n_e) row-major from element begin*hidden, its B block
 *                  (n, n_e) row-major from element begin*n, where n_e = end - begin:
 *                  A[begin*hidden + m*n_e + (t - begin)], B[begin*n + j*n_e + (t - begin)]. */
#define KGW_A_M_MAJOR 1
#define KGW_B_K_MAJOR 2
#define KGW_RAGGED 4

/*
 * kgw_wgrad_bf16_ex -- kgw_wgrad_bf16 with a choice of operand layout (`layout`,
 * KGW_A_M_MAJOR | KGW_B_K_MAJOR | KGW_RAGGED flags as above; any other bit, or
 * KGW_RAGGED with another combination, is KGW_ERROR_INVALID_VALUE) and of
 * output form (cuDNN page, section "Output modes": one dense tensor, or discrete
 * per-expert outputs through an array of pointers, wgrad_ptrs).  Exactly one of
 * `out` and `out_ptrs` is non-NULL:
 *   out       the dense (num_experts, hidden, n) output, as for kgw_wgrad_bf16;
 *   out_ptrs  DEVICE array of num_experts pointers, 8-byte aligned; entry e
 *             points to expert e's own (hidden, n) row-major matrix of
 *             out_dtype, 16-byte aligned, not overlapping another entry's (the
 *             pointers are read on the device only; like the offsets, they are
 *             the caller's to get right).  A NULL entry skips its expert:
 *             nothing is computed or written for it.
 * Everything else (modes, workspace, sizes, errors) as for kgw_wgrad_bf16.
 */
kgw_status_t kgw_wgrad_bf16_ex(const void* A, const void* B, int32_t layout, const int32_t* offsets,
                               int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                               void* out, void* const* out_ptrs, int32_t out_dtype, int32_t accumulate,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * kgw_wgrad_fp8 -- OCP e4m3 ("fn") operands with one power-of-two (UE8M0) scale per
 * 128 tokens, applied inside the K loop, fp32 accumulation (llm-infra-atlas
 * "05 Grouped GEMM", section 3: per-block 1x128 scaling, UE8M0 scales, fp8
 * consumed directly without a separate dequantisation pass; for the weight
 * gradient the blocks run along the contracted token axis, section 5.2).
 * Operands stay fp8 in memory; inside the K loop each fragment is converted
 * exactly to bf16 with its scale folded in and multiplied on the bf16 MFMA, so
 * the only rounding is the fp32 accumulation (see kgw_wgrad_fp8_native for the
 * native fp8 MFMA variant).
 *
 *   A    e4m3 bytes (hidden, tokens_sum), token axis contiguous.
 *   sfa  uint8 (tokens_sum/128, hidden): sfa[b][m] is the biased exponent of the
 *        scale of A[m, 128b : 128b+128]; value 2^(byte-127).
 *   B    e4m3 bytes (tokens_sum, n), row-major.
 *   sfb  uint8 (tokens_sum/128, n): scale exponent of B[128b : 128b+128, j].
 *   The real operand value is e4m3(q) * 2^(s - 127); a scale byte of 0xFF encodes
 *   NaN and, like a NaN operand, makes the affected outputs NaN.
 *   Counts must be multiples of 128; n a multiple of 16.  Everything else as for
 *   kgw_wgrad_bf16 (out_dtype, accumulate, workspace, sizes, alignment).
 */
kgw_status_t kgw_wgrad_fp8(const void* A, const uint8_t* sfa, const void* B, const uint8_t* sfb,
                           const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                           int64_t tokens_sum, void* out, int32_t out_dtype, int32_t accumulate,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kgw_wgrad_fp8_native -- same arguments, contract and results' definition as
 * kgw_wgrad_fp8, computed with the native scaled fp8 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4: the UE8M0 bytes go straight into the
 * instruction, as the scaled-MFMA reading of llm-infra-atlas section 3 suggests).
 * Faster, but less accurate: inside one instruction the hardware aligns the
 * products of a K group to the group's largest one and keeps only about 13 bits
 * below it, so a result can differ from the exactly rounded sum by up to about
 * 2^-13 of the largest product in each 32-token group (relative Frobenius error
 * about 1.5e-5 on block-quantised Gaussian data, versus about 1e-7 for
 * kgw_wgrad_fp8).  Integer-valued operands whose products share a binade range
 * of less than 2^13 are exact.
 */
kgw_status_t kgw_wgrad_fp8_native(const void* A, const uint8_t* sfa, const void* B, const uint8_t* sfb,
                                  const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                                  int64_t tokens_sum, void* out, int32_t out_dtype, int32_t accumulate,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kgw_wgrad_fp8_ex -- the fp8 product with a choice of scale layout and output
 * form.  scale_format is a kgw_scale_format_t: with KGW_SCALES_PACKED_32 every
 * operand element is scaled by the UE8M0 byte of its own 32-token block (the
 * DeepGEMM k-grouped page's gran_k = 32); otherwise by that of its 128-token
 * block.  native 0 computes as kgw_wgrad_fp8 (exact bf16 conversion, bf16
 * MFMA), 1 as kgw_wgrad_fp8_native (the scaled fp8 MFMA, whose hardware scale
 * blocks are exactly 32 tokens: each lane hands the instruction the byte of
 * its half of the 64-token step).  out / out_ptrs as for kgw_wgrad_bf16_ex.
 * layout: 0 (A (hidden, tokens_sum), B (tokens_sum, n), as for kgw_wgrad_fp8) or
 * the KGW_A_M_MAJOR / KGW_B_K_MAJOR / KGW_RAGGED combinations kgw_wgrad_bf16_ex
 * takes, with the same meaning: A stored (tokens_sum, hidden), element (m, t) at
 * A[t * hidden + m]; B stored (n, tokens_sum), element (t, j) at
 * B[j * tokens_sum + t] (with the default A: both operands token-contiguous, the
 * pair a (M, K), b (N, K) of the DeepGEMM k-grouped page); ragged per-expert
 * K-contiguous blocks (KGW_RAGGED | KGW_B_K_MAJOR).  The scales keep their
 * (tokens_sum/128, hidden) and (tokens_sum/128, n) layouts in every case.  These
 * layouts are taken with native 0 and KGW_SCALES_U8 only (else
 * KGW_ERROR_UNSUPPORTED); KGW_A_M_MAJOR needs hidden a multiple of 16
 * (KGW_ERROR_MISALIGNED) and below 2^25 (KGW_ERROR_UNSUPPORTED); other
 * combinations and bits are rejected as by kgw_wgrad_bf16_ex.  Every layout gives
 * the default layout's result bit for bit.
 * Counts stay multiples of 128 for every format.  Everything else as for
 * kgw_wgrad_fp8; an unknown scale_format or native value is
 * KGW_ERROR_INVALID_VALUE, a misaligned KGW_SCALES_PACKED_32 pointer
 * KGW_ERROR_MISALIGNED.
 */
kgw_status_t kgw_wgrad_fp8_ex(const void* A, const void* sfa, const void* B, const void* sfb,
                              int32_t scale_format, int32_t native, int32_t layout, const int32_t* offsets,
                              int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                              void* out, void* const* out_ptrs, int32_t out_dtype, int32_t accumulate,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * kgw_wgrad_fp4 -- FP4 operands: OCP e2m1 values with one UE8M0 scale per 32
 * tokens (the DeepGEMM k-grouped page casts a and b to FP4 with gran_k = 32; the
 * MX block), on the native scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
 * both formats e2m1), fp32 accumulation.  e2m1: 1 sign, 2 exponent bits (bias 1),
 * 1 mantissa bit -- magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Every product times
 * its scales is exact and each 32-token block's sum is exact inside the
 * instruction, so the result differs from the exact sum only by fp32
 * accumulation rounding.
 *
 *   A    e2m1 (hidden, tokens_sum) stored two tokens per byte along the token axis:
 *        (hidden, tokens_sum/2) bytes, token t of row m in byte m*tokens_sum/2 + t/2,
 *        low nibble for even t.  Token-contiguous (the page's a (M, K)).
 *   B    e2m1 (tokens_sum, n) stored token-contiguous the same way: (n, tokens_sum/2)
 *        bytes, token t of column j in byte j*tokens_sum/2 + t/2 (the page's b (N, K)).
 *   sfa, sfb  UE8M0 per 32 tokens in the KGW_SCALES_PACKED_32 layout: int32
 *        (tokens_sum/128, hidden) and (tokens_sum/128, n), 4-byte aligned.
 *   out, out_ptrs, out_dtype, accumulate, workspace  as for kgw_wgrad_bf16_ex.
 *   Counts multiples of 256 (KGW_FP4_TOKEN_ALIGN), n a multiple of 8.
 */
kgw_status_t kgw_wgrad_fp4(const void* A, const void* sfa, const void* B, const void* sfb, const int32_t* offsets,
                           int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, void* out,
                           void* const* out_ptrs, int32_t out_dtype, int32_t accumulate, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * kgw_quantize_fp8 -- produce the fp8 operands of kgw_wgrad_fp8 from bf16 on the
 * device: OCP e4m3fn bytes plus one UE8M0 scale byte per 128 tokens, the
 * blocks running along the token axis (llm-infra-atlas "05 Grouped GEMM",
 * section 3: 1x128 blocks with power-of-two UE8M0 scales, fp8 consumed
 * directly; section 5.2: the weight gradient contracts over tokens).  The pages
 * do not fix how the scale is chosen; here, per block, the scale is the
 * smallest power of two 2^k with amax <= 448 * 2^k (amax = largest |x| of the
 * block, 448 = largest e4m3fn), its byte k + 127 clamped to [1, 254] (127 for
 * an all-zero block), and every element is e4m3fn(x / 2^k) rounded to
 * nearest, ties to even.  A block holding a NaN or an infinity gets scale byte
 * 0xFF (NaN) and NaN elements (0x7F).  With scale_format KGW_SCALES_PACKED_32
 * the blocks are 32 tokens long (the DeepGEMM k-grouped page's gran_k = 32).
 *
 *   x       bf16 (rows, cols), row-major, device, 16-byte aligned.
 *   token_axis  1: tokens along the columns -- A of the weight gradient,
 *           (hidden, tokens_sum); scales with mn = rows.
 *           0: tokens along the rows -- B, (tokens_sum, n); scales with
 *           mn = cols.
 *   scale_format  a kgw_scale_format_t: the layout of `scales`, the one the
 *           GEMM entry points take with the same code.
 *   q       uint8 (rows, cols), same layout as x, device, 16-byte aligned.
 *   scales  device; KGW_SCALES_U8 8-byte aligned when token_axis == 0,
 *           KGW_SCALES_PACKED_32 16-byte aligned.
 *   stream  hipStream_t (NULL = default stream); asynchronous.
 *
 * The token length (cols for token_axis 1, rows for 0) must be a multiple of
 * 128 for every format (else KGW_ERROR_INVALID_VALUE) and cols a multiple of 8
 * (KGW_ERROR_MISALIGNED); an unknown token_axis or scale_format is
 * KGW_ERROR_INVALID_VALUE.  rows or cols == 0 does nothing.  Every output byte
 * is a function of x alone: results are bit-for-bit reproducible.
 */
kgw_status_t kgw_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis,
                              int32_t scale_format, void* q, void* scales, void* stream);

/*
 * kgw_quantize_fp4 -- produce the FP4 operands of kgw_wgrad_fp4 from bf16 on the
 * device: OCP e2m1 codes with one UE8M0 scale per 32 tokens (the DeepGEMM
 * k-grouped page casts a and b to FP4 with gran_k = 32).  The page does not fix
 * how the scale is chosen; here, per block, the scale is the smallest power of
 * two 2^k with amax <= 6 * 2^k (amax = largest |x| of the block, 6 = largest
 * e2m1), its byte k + 127 clamped to [1, 254] (127 for an all-zero block), and
 * every element is the e2m1 value nearest to x / 2^k, ties to the even code
 * (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 have codes 0..7, sign in bit 3).  A
 * block holding a NaN or an infinity gets scale byte 0xFF and zero codes (e2m1
 * has no NaN).  Codes are stored token-contiguous, two per byte, the even token
 * in the low nibble -- the layout kgw_wgrad_fp4 takes for both operands.
 *
 *   x       bf16 (rows, cols), row-major, device, 16-byte aligned.
 *   token_axis  1: tokens along the columns -- A of the weight gradient,
 *           (hidden, tokens_sum): q is (rows, cols/2) bytes, scales with mn = rows.
 *           0: tokens along the rows -- B, (tokens_sum, n): q is (cols, rows/2)
 *           bytes (the token axis made contiguous), scales with mn = cols.
 *   scale_format  KGW_SCALES_U8: uint8 (tokens/32, mn), one byte per 32 tokens
 *           (8-byte aligned when token_axis == 0); KGW_SCALES_PACKED_32: int32
 *           (tokens/128, mn), the layout kgw_wgrad_fp4 takes (16-byte aligned).
 *   q       uint8, shape as above, device, 16-byte aligned.
 *   stream  hipStream_t (NULL = default stream); asynchronous.
 *
 * The token length (cols for token_axis 1, rows for 0) must be a multiple of
 * 128 (else KGW_ERROR_INVALID_VALUE) and cols a multiple of 8
 * (KGW_ERROR_MISALIGNED); an unknown token_axis or scale_format (KGW_SCALES_PACKED
 * included) is KGW_ERROR_INVALID_VALUE.  rows or cols == 0 does nothing.  Every
 * output byte is a function of x alone: results are bit-for-bit reproducible.
 */
kgw_status_t kgw_quantize_fp4(const void* x, int64_t rows, int64_t cols, int32_t token_axis,
                              int32_t scale_format, void* q, void* scales, void* stream);

/* Weight layout of the m-grouped product (DeepGEMM's "nt" / "nn" naming). */
typedef enum {
    KGW_LAYOUT_NT = 0,   /* forward: W (num_groups, n, k), k contiguous; out = A @ W[g]^T */
    KGW_LAYOUT_NN = 1    /* dgrad:   W (num_groups, k, n), n contiguous; out = A @ W[g]   */
} kgw_layout_t;

/*
 * kgw_mgrouped_bf16 -- the m-grouped GEMM of the same MoE layer: its forward and
 * dgrad (llm-infra-atlas "05 Grouped GEMM": section 1, grouping along M only,
 * N and K fixed; section 2.1, the contiguous layout; section 5.1, dgrad is
 * m-grouped too).  Row r of A belongs to group g(r) and
 *
 *     layout KGW_LAYOUT_NT:  out[r, :] = A[r, :] @ W[g(r)]^T
 *     layout KGW_LAYOUT_NN:  out[r, :] = A[r, :] @ W[g(r)]
 *
 * bf16 operands, fp32 accumulation, output rounded once to out_dtype.
 *
 *   A          bf16 (m, k), row-major (k contiguous), device.
 *   W          bf16, (num_groups, n, k) for NT or (num_groups, k, n) for NN, device.
 *   offsets    int32 (num_groups,) inclusive cumulative row counts: row r is in
 *              group e when offsets[e-1] <= r < offsets[e]; rows at or past
 *              offsets[num_groups-1] are in no group.  Or NULL, with:
 *   m_indices  int32 (m,) group id of every row (any id outside
 *              [0, num_groups) marks a row of no group).  Exactly one of
 *              offsets / m_indices is given.
 *              Contract (not checked on the host): every group starts on a
 *              multiple of 128 rows and holds a multiple of 128 rows, i.e. every
 *              aligned 128-row block lies in one group (or in none).
 *   out        (m, n) row-major, out_dtype, device.  accumulate 0: out = product;
 *              1: out += product.  Rows of no group are left untouched.
 *   stream     hipStream_t (NULL = default stream); asynchronous, allocates nothing.
 *
 * Sizes: 1 <= num_groups <= 65536, 0 <= m < 2^31, 0 <= k < 2^22 and a multiple of
 * 64, 0 <= n < 2^24 and a multiple of 8 (KGW_ERROR_MISALIGNED otherwise);
 * A, W, out 16-byte aligned.  m == 0 or n == 0 does nothing; k == 0 writes zeros
 * (overwrite) into the rows of a group.  Errors as for kgw_wgrad_bf16.
 */
kgw_status_t kgw_mgrouped_bf16(const void* A, const void* W, int32_t layout, const int32_t* offsets,
                               const int32_t* m_indices, int32_t num_groups, int64_t m, int64_t k, int64_t n,
                               void* out, int32_t out_dtype, int32_t accumulate, void* stream);

/*
 * kgw_mgrouped_fp8 -- the m-grouped product with fp8 operands, forward or dgrad
 * (llm-infra-atlas "05 Grouped GEMM": section 2.1, m_grouped_fp8_gemm_nt_contiguous,
 * the contiguous layout; section 3, every fp8 input carries one power-of-two
 * (UE8M0) scale per 1x128 block along K, the scale tensor mn-major; section 5.1,
 * dgrad is m-grouped too).  Row r of A belongs to group g(r) and
 *
 *     out[r, j] = sum_t  a(r, t) * w(g(r), j, t),        t = 0 .. k-1
 *     a(r, t)    = e4m3(A[r, t])                  * 2^(sa[t/128, r] - 127),
 *     w(g, j, t) = e4m3(W element (g, j, t))      * 2^(sw[g, t/128, j] - 127),
 *
 * computed as kgw_wgrad_fp8 does: each operand fragment converted exactly to bf16
 * with its scale folded in, products summed in fp32 on the bf16 MFMA, the output
 * rounded once to out_dtype.
 *
 *   A          e4m3 bytes (m, k), row-major (k contiguous), device, 16-byte aligned.
 *   sa         uint8 (k/128, m): sa[b][r] is the biased exponent of the scale of
 *              A[r, 128b : 128b+128].
 *   W          e4m3 bytes, device, 16-byte aligned, laid out by `layout`:
 *              KGW_LAYOUT_NT (forward, out = A @ W[g]^T): (num_groups, n, k), element
 *              (g, j, t) at W[(g*n + j)*k + t]; KGW_LAYOUT_NN (dgrad, out = A @ W[g]):
 *              (num_groups, k, n), element (g, j, t) at W[(g*k + t)*n + j].
 *   sw         uint8 (num_groups, k/128, n): scale exponent of the 128 values
 *              (g, j, 128b .. 128b+127) of W, in either layout.
 *   offsets / m_indices, out, out_dtype, accumulate, stream  as for kgw_mgrouped_bf16,
 *              with the same 128-row group contract (not checked on the host).
 *   A scale byte of 0xFF encodes NaN and, like a NaN operand, makes the affected
 *   outputs NaN.
 *
 * Sizes: 1 <= num_groups <= 65536, 0 <= m < 2^31, 0 <= k < 2^22 and a multiple of
 * 128, 0 <= n < 2^24 and a multiple of 8 (NT) or 16 (NN) (KGW_ERROR_MISALIGNED
 * otherwise); an unknown layout is KGW_ERROR_INVALID_VALUE.  m == 0 or n == 0 does
 * nothing; k == 0 writes zeros (overwrite) into the rows of a group.  Errors as for
 * kgw_wgrad_bf16.
 */
kgw_status_t kgw_mgrouped_fp8(const void* A, const uint8_t* sa, const void* W, const uint8_t* sw,
                              int32_t layout, const int32_t* offsets, const int32_t* m_indices,
                              int32_t num_groups, int64_t m, int64_t k, int64_t n, void* out,
                              int32_t out_dtype, int32_t accumulate, void* stream);

/*
 * kgw_workspace_bytes -- device workspace the kgw_wgrad_* call uses for this shape
 * on the current device (fp8 != 0 selects the fp8 entry points; 256 compute
 * units are assumed when no device is visible).  Nonzero in two cases:
 *  - the output tiles alone would leave more than half of the compute units idle
 *    and the experts average at least 2048 tokens: the call splits each expert's
 *    token range into 2..16 chunks (split-K) and needs
 *    chunks * num_experts * hidden * n * 4 bytes, at most 1 GiB;
 *  - (bf16) the output tiles fill the compute units at least 8 times over, with at
 *    most 64 experts averaging 1024 or more tokens: 256 bytes of claim counters
 *    for the dynamic schedule.
 * 0 means one pass on the static schedule.
 */
size_t kgw_workspace_bytes(int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                           int32_t fp8);

/*
 * kgw_validate_offsets_host -- check HOST offsets against the contract of the
 * cuDNN page, section "BF16 contract": non-decreasing, every count
 * (offsets[e] - offsets[e-1], offsets[0] for e == 0) a non-negative multiple of
 * `alignment`, and offsets[num_experts-1] == tokens_sum.
 * Returns KGW_SUCCESS or KGW_ERROR_BAD_OFFSETS (KGW_ERROR_INVALID_VALUE for
 * NULL / num_experts < 1 / alignment < 1).  If bad_expert is not NULL it receives
 * the first offending expert index (-1 on success).  Pure host code.
 */
kgw_status_t kgw_validate_offsets_host(const int32_t* offsets, int32_t num_experts,
                                       int64_t tokens_sum, int32_t alignment,
                                       int32_t* bad_expert);

/*
 * kgw_validate_offsets -- the same check on DEVICE offsets.  SYNCHRONOUS: copies the
 * num_experts int32 values to the host after the work already queued on `stream`.
 */
kgw_status_t kgw_validate_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                                  int32_t alignment, int32_t* bad_expert, void* stream);

/*
 * kgw_check_offsets -- the same check on DEVICE offsets, kept on the device: a
 * kernel queued on `stream` writes to result[0] (a device int32) the first
 * offending expert, or -1 when the offsets meet the contract.  Asynchronous and
 * stream-ordered like the products (no copy to the host, no synchronisation, no
 * allocation), so a caller can queue it next to a kgw_wgrad_* call and read the
 * flag whenever it next synchronises.  The products clamp malformed ranges into
 * [0, tokens_sum) by themselves (see the conventions above); this is how a caller
 * that cannot afford kgw_validate_offsets' synchronisation learns that they did.
 * KGW_ERROR_INVALID_VALUE for NULL pointers, num_experts < 1, alignment < 1 or
 * tokens_sum < 0; KGW_ERROR_MISALIGNED for pointers not 4-byte aligned.
 */
kgw_status_t kgw_check_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                               int32_t alignment, int32_t* result, void* stream);

/*
 * kgw_mfma_ceiling -- measurement helper, not part of the product: the MFMA rate this
 * board sustains on given operand data.  MFMA power depends on the operand values and the
 * chip lowers its clock past its power limit, so realistic data runs below the nominal
 * peak; the product kernels are judged against both.  Launches `workgroups` workgroups
 * of four waves (one wave per SIMD); every lane loads 32 operand dwords once from `src`
 * (`src_bytes` bytes, at least 4096, 4-byte aligned) and runs `iters` rounds of 16
 * independent MFMAs on them:
 *   kind 0: v_mfma_f32_32x32x16_bf16 on the words of `src` read as bf16 pairs;
 *   kind 1: the same MFMA on e4m3 bytes of `src` converted exactly to bf16 (the operand
 *           values the exact fp8 entry point feeds its MFMAs);
 *   kind 2: v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 bytes of `src`, unit scales;
 *   kind 3: the same instruction with both operands e2m1 (two FP4 codes per byte of
 *           `src`), unit scales (the FP4 entry point's MFMA).
 * Per workgroup w it writes cycles[2w] = shader-clock cycles and cycles[2w+1] = 100 MHz
 * real-time ticks of the loop (8-byte aligned device array of 2 * workgroups values), so
 * cycles / ticks * 1e8 is the clock the loop ran at.  The FLOP count is 16 * iters MFMAs
 * per wave (32768 FLOP each for kinds 0-1, 131072 for kinds 2-3).  Asynchronous on `stream`.
 */
kgw_status_t kgw_mfma_ceiling(const void* src, int64_t src_bytes, int32_t kind, int32_t iters,
                              int32_t workgroups, uint64_t* cycles, void* stream);

/*
 * kgw_status_string -- static description of a status code; never NULL.
 */
const char* kgw_status_string(kgw_status_t status);

/*
 * kgw_device_info -- properties of the current device as the library sees them:
 * compute units, whether it is gfx950 (1/0), and the number of XCDs the
 * workgroup remapping assumes.  Any output pointer may be NULL.
 */
kgw_status_t kgw_device_info(int32_t* num_cus, int32_t* is_gfx950, int32_t* num_xcds);

#ifdef __cplusplus
}
#endif

#endif /* KGW_H */
