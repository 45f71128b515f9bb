/*
 * CPU oracle for the K-grouped MoE weight-gradient GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test-suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library and depends on nothing but libc, libm and OpenMP.
 *
 * What it computes (cuDNN "Grouped GEMM + WGrad (Unified)", section
 * "Operation"): for expert e, begin = 0 when e == 0 and offsets[e-1]
 * otherwise, end = offsets[e], and
 *
 *     Wgrad[e] = A[:, begin:end] @ B[begin:end, :]
 *
 * with A of shape (hidden, tokens_sum) stored token-contiguous and B of shape
 * (tokens_sum, n) stored row-major (same page, "BF16 contract" table).  Each
 * output element is one sum over the expert's tokens, taken in increasing
 * token order in IEEE double precision.  Nothing is blocked or reordered.
 *
 * For the fp8 path (llm-infra-atlas "05 Grouped GEMM", section 3, FP8 data
 * layout: one power-of-two scale per 1x128 block, here along the token axis
 * as the k-grouped weight gradient needs; the DeepGEMM k-grouped page's
 * casting step also quantises with gran_k = 32, one scale per 32 elements)
 * each operand element is first decoded to its real value
 * e4m3(q) * 2^(scale_byte - 127), the scale byte being that of the element's
 * block of `block` tokens (128 or 32), and the same sum is taken over those
 * values.
 *
 * Format decoders are written from the format definitions:
 *   bf16      : the upper 16 bits of an IEEE-754 binary32 word;
 *   e4m3 "fn" : OCP 8-bit float, 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *               subnormals when the exponent field is 0, no infinities, and
 *               S.1111.111 is NaN (largest finite 448);
 *   E8M0      : OCP MX scale byte, value 2^(b - 127), 0xFF is NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double oracle_bf16_value(uint16_t bits) {
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

double oracle_e4m3fn_value(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 3) & 0xF;
    int mant = bits & 0x7;
    double mag;
    if (expo == 0xF && mant == 0x7) return NAN;
    if (expo == 0)
        mag = ldexp((double)mant / 8.0, 1 - 7);          /* subnormal: 0.m * 2^(1-bias) */
    else
        mag = ldexp(1.0 + (double)mant / 8.0, expo - 7); /* normal: 1.m * 2^(e-bias) */
    return sign ? -mag : mag;
}

double oracle_e8m0_value(uint8_t bits) {
    if (bits == 0xFF) return NAN;
    return ldexp(1.0, (int)bits - 127);
}

/* Token range of expert e from the inclusive cumulative offsets. */
void oracle_expert_range(const int32_t* offsets, int32_t e, int64_t* begin, int64_t* end) {
    *begin = (e == 0) ? 0 : (int64_t)offsets[e - 1];
    *end = (int64_t)offsets[e];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following parallel loops (timing only: every row is summed in
   the same order whatever the count, so results do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Rows rows[0..nrows) of Wgrad for the token range [begin, end), bf16 operands.
 * A: uint16 bf16 bits (hidden, tokens_sum); B: uint16 bf16 bits (tokens_sum, n).
 * out: double (nrows, n).  Returns 0, or -1 on a bad range.
 */
int oracle_wgrad_rows_bf16(const uint16_t* A, const uint16_t* B, int64_t tokens_sum, int64_t n,
                           int64_t begin, int64_t end, const int64_t* rows, int64_t nrows,
                           double* out) {
    if (begin < 0 || end < begin || end > tokens_sum) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        double* w = out + r * n;
        for (int64_t j = 0; j < n; ++j) w[j] = 0.0;
        for (int64_t k = begin; k < end; ++k) {
            const double a = oracle_bf16_value(A[m * tokens_sum + k]);
            const uint16_t* brow = B + k * n;
            for (int64_t j = 0; j < n; ++j) w[j] += a * oracle_bf16_value(brow[j]);
        }
    }
    return 0;
}

/*
 * Same for fp8 operands with one UE8M0 scale per `block` tokens:
 * A: e4m3 bytes (hidden, tokens_sum); sfa: bytes (tokens_sum/block, hidden);
 * B: e4m3 bytes (tokens_sum, n);      sfb: bytes (tokens_sum/block, n).
 */
int oracle_wgrad_rows_fp8(const uint8_t* A, const uint8_t* sfa, int64_t hidden, const uint8_t* B,
                          const uint8_t* sfb, int64_t tokens_sum, int64_t n, int64_t begin,
                          int64_t end, const int64_t* rows, int64_t nrows, double* out, int64_t block) {
    if (begin < 0 || end < begin || end > tokens_sum) return -1;
    if (block < 1 || tokens_sum % block != 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        double* w = out + r * n;
        for (int64_t j = 0; j < n; ++j) w[j] = 0.0;
        for (int64_t k = begin; k < end; ++k) {
            const int64_t blk = k / block;
            const double a = oracle_e4m3fn_value(A[m * tokens_sum + k]) *
                             oracle_e8m0_value(sfa[blk * hidden + m]);
            const uint8_t* brow = B + k * n;
            const uint8_t* srow = sfb + blk * n;
            for (int64_t j = 0; j < n; ++j)
                w[j] += a * (oracle_e4m3fn_value(brow[j]) * oracle_e8m0_value(srow[j]));
        }
    }
    return 0;
}

/* Dense Wgrad (num_experts, hidden, n) for every expert, bf16 operands. */
int oracle_wgrad_bf16(const uint16_t* A, const uint16_t* B, const int32_t* offsets,
                      int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum,
                      double* out) {
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(hidden > 0 ? hidden : 1));
    if (!rows) return -2;
    for (int64_t m = 0; m < hidden; ++m) rows[m] = m;
    int rc = 0;
    for (int32_t e = 0; e < num_experts && rc == 0; ++e) {
        int64_t begin, end;
        oracle_expert_range(offsets, e, &begin, &end);
        rc = oracle_wgrad_rows_bf16(A, B, tokens_sum, n, begin, end, rows, hidden,
                                    out + (int64_t)e * hidden * n);
    }
    free(rows);
    return rc;
}

/* Dense Wgrad (num_experts, hidden, n) for every expert, fp8 block-scaled operands. */
int oracle_wgrad_fp8(const uint8_t* A, const uint8_t* sfa, const uint8_t* B, const uint8_t* sfb,
                     const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                     int64_t tokens_sum, double* out, int64_t block) {
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(hidden > 0 ? hidden : 1));
    if (!rows) return -2;
    for (int64_t m = 0; m < hidden; ++m) rows[m] = m;
    int rc = 0;
    for (int32_t e = 0; e < num_experts && rc == 0; ++e) {
        int64_t begin, end;
        oracle_expert_range(offsets, e, &begin, &end);
        rc = oracle_wgrad_rows_fp8(A, sfa, hidden, B, sfb, tokens_sum, n, begin, end, rows, hidden,
                                   out + (int64_t)e * hidden * n, block);
    }
    free(rows);
    return rc;
}

/*
 * Token-axis fp8 quantiser (llm-infra-atlas "05 Grouped GEMM", section 3: one
 * power-of-two UE8M0 scale per 1x128 block; for the k-grouped weight gradient
 * the blocks run along the token axis, section 5.2; the DeepGEMM k-grouped
 * page's casting step uses blocks of gran_k = 32 elements instead).  The pages leave the
 * choice of the scale open; the reading used here takes, per block, the
 * smallest power of two 2^k with amax <= 448 * 2^k (448 = largest e4m3fn),
 * stores the biased exponent k + 127 clamped to [1, 254] (127 for an all-zero
 * block, 255 = the E8M0 NaN code for a block holding a NaN or an infinity),
 * and encodes every element as e4m3fn(x / 2^k), rounded to nearest, ties to
 * even.  In a NaN/infinity block every element is the e4m3fn NaN 0x7F.
 */

/* e4m3fn encoding of v, round to nearest with ties to even, sign kept (also
 * for zero); NaN and magnitudes that round above 448 give 0x7F. */
uint8_t oracle_e4m3fn_encode(double v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double mag = fabs(v);
    if (mag == 0.0) return sign;
    if (mag < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; a result of 8 quanta is the
         * smallest normal 2^-6, whose code 0x08 continues the count */
        double n = mag * 512.0;              /* exact: power-of-two scaling */
        double m = nearbyint(n);             /* default rounding: nearest, ties to even */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int ex;
    frexp(mag, &ex);                         /* mag = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                          /* mag in [2^E, 2^(E+1)) */
    double n = ldexp(mag, 3 - E);            /* in [8, 16), exact */
    double m = nearbyint(n);
    if (m == 16.0) {
        m = 8.0;
        E += 1;
    }
    const int field = E + 7;
    if (field > 15 || (field == 15 && (int)m - 8 == 7)) return 0x7F;  /* beyond 448 */
    return (uint8_t)(sign | (uint8_t)(field << 3) | (uint8_t)((int)m - 8));
}

/* Biased UE8M0 exponent for a block whose largest magnitude is amax. */
uint8_t oracle_e8m0_for_amax(double amax) {
    if (isnan(amax) || isinf(amax)) return 0xFF;
    if (amax == 0.0) return 127;
    int k = (int)ceil(log2(amax / 448.0));
    while (amax > ldexp(448.0, k)) ++k;          /* exact comparisons settle log2's rounding */
    while (amax <= ldexp(448.0, k - 1)) --k;
    int e = k + 127;
    if (e < 1) e = 1;
    if (e > 254) e = 254;
    return (uint8_t)e;
}

/* x: bf16 bits, (rows, cols) row-major.  token_axis 1: tokens run along the
 * columns (A of the weight gradient, (hidden, tokens)), scales s are
 * (cols/block, rows); token_axis 0: tokens run along the rows (B, (tokens, n)),
 * scales (rows/block, cols).  q: e4m3fn bytes in x's layout.  Returns 0, or -1
 * when the token length is not a multiple of the block (block >= 1). */
int oracle_quantize_fp8_tokens(const uint16_t* x, int64_t rows, int64_t cols, int token_axis, uint8_t* q,
                               uint8_t* s, int64_t block) {
    const int64_t tokens = token_axis ? cols : rows;
    const int64_t other = token_axis ? rows : cols;
    if (block < 1 || tokens % block != 0) return -1;
    const int64_t nblocks = tokens / block;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < other; ++o) {
        for (int64_t b = 0; b < nblocks; ++b) {
            double amax = 0.0;
            int bad = 0;
            for (int64_t t = block * b; t < block * b + block; ++t) {
                const int64_t idx = token_axis ? o * cols + t : t * cols + o;
                const double v = oracle_bf16_value(x[idx]);
                if (isnan(v) || isinf(v)) bad = 1;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            const uint8_t e = bad ? 0xFF : oracle_e8m0_for_amax(amax);
            s[b * other + o] = e;
            for (int64_t t = block * b; t < block * b + block; ++t) {
                const int64_t idx = token_axis ? o * cols + t : t * cols + o;
                q[idx] = bad ? 0x7F : oracle_e4m3fn_encode(ldexp(oracle_bf16_value(x[idx]), 127 - (int)e));
            }
        }
    }
    return 0;
}

/*
 * M-grouped GEMM (llm-infra-atlas "05 Grouped GEMM", section 1 "grouping only
 * along M" and section 2.1 "contiguous layout"; section 5.1 for the dgrad
 * form).  The rows of A (M, K) are the concatenated tokens of the experts;
 * row m belongs to group g(m) and
 *
 *     forward ("nt"): out[m, :] = A[m, :] @ W[g(m)]^T    W (E, N, K)
 *     dgrad   ("nn"): out[m, :] = A[m, :] @ W[g(m)]      W (E, K, N)
 *
 * bf16 operands, each output element one fp64 sum over k in increasing order.
 * A group id outside [0, num_groups) marks a row that belongs to no group (the
 * pages use -1 for padding rows; larger ids are read the same way): it is not
 * computed (out row left as NaN for the caller to recognise).  Returns 0.
 */
int oracle_mgrouped_bf16(const uint16_t* A, const uint16_t* W, const int32_t* group, int64_t M, int64_t K,
                         int64_t N, int32_t num_groups, int nt, double* out) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = 0; m < M; ++m) {
        double* o = out + m * N;
        const int32_t g = group[m];
        if (g < 0 || g >= num_groups) {
            for (int64_t j = 0; j < N; ++j) o[j] = NAN;
            continue;
        }
        const uint16_t* Wg = W + (int64_t)g * K * N;
        for (int64_t j = 0; j < N; ++j) o[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = oracle_bf16_value(A[m * K + k]);
            if (nt) {
                for (int64_t j = 0; j < N; ++j) o[j] += a * oracle_bf16_value(Wg[j * K + k]);
            } else {
                const uint16_t* wrow = Wg + k * N;
                for (int64_t j = 0; j < N; ++j) o[j] += a * oracle_bf16_value(wrow[j]);
            }
        }
    }
    return 0;
}

/*
 * m-grouped forward product with fp8 operands (llm-infra-atlas "05 Grouped GEMM":
 * section 2.1 names m_grouped_fp8_gemm_nt_contiguous, section 3 gives its inputs as
 * (values, scales) pairs with one power-of-two scale per 1x128 block along K, the
 * scale tensor mn-major).  Row m of group g = group[m]:
 *
 *     out[m][j] = sum_k a(m, k) * w(g, j, k)
 *     a(m, k)    = e4m3(A[m*K + k])       * 2^(sa[(k/128)*M + m] - 127)
 *     w(g, j, k) = e4m3(W[(g*N + j)*K + k]) * 2^(sw[(g*(K/128) + k/128)*N + j] - 127)
 *
 * A (M, K) and W (E, N, K) are K-contiguous e4m3 bytes; sa (K/128, M) and sw
 * (E, K/128, N) hold UE8M0 bytes with the row / column index contiguous.  Each sum
 * in fp64 over k in increasing order; a row of no group is NaN.  Returns 0.
 */
int oracle_mgrouped_fp8(const uint8_t* A, const uint8_t* sa, const uint8_t* W, const uint8_t* sw,
                        const int32_t* group, int64_t M, int64_t K, int64_t N, int32_t num_groups, double* out) {
    const int64_t kb = K / 128;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = 0; m < M; ++m) {
        double* o = out + m * N;
        const int32_t g = group[m];
        if (g < 0 || g >= num_groups) {
            for (int64_t j = 0; j < N; ++j) o[j] = NAN;
            continue;
        }
        const uint8_t* Wg = W + (int64_t)g * N * K;
        const uint8_t* swg = sw + (int64_t)g * kb * N;
        for (int64_t j = 0; j < N; ++j) o[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = oracle_e4m3fn_value(A[m * K + k]) * oracle_e8m0_value(sa[(k / 128) * M + m]);
            const uint8_t* srow = swg + (k / 128) * N;
            for (int64_t j = 0; j < N; ++j)
                o[j] += a * (oracle_e4m3fn_value(Wg[j * K + k]) * oracle_e8m0_value(srow[j]));
        }
    }
    return 0;
}

/*
 * FP4 (OCP e2m1) operands with one UE8M0 scale per 32 tokens (the DeepGEMM
 * k-grouped page's per_token_cast_to_fp4 with gran_k = 32; the MX block of the
 * OCP formats).  e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent
 * field 0 is subnormal (0 or 0.5); no infinities or NaN; largest 6.
 * Both operands keep the token axis contiguous, two tokens per byte, the
 * even token in the low nibble:
 *   A  (hidden, tokens_sum/2) bytes, A[m][t] = nibble t%2 of byte m*T/2 + t/2;
 *   B  (n, tokens_sum/2) bytes,      B[t][j] = nibble t%2 of byte j*T/2 + t/2;
 *   sfa (tokens_sum/32, hidden), sfb (tokens_sum/32, n) UE8M0 bytes.
 */
double oracle_e2m1_value(uint8_t code) {
    const int sign = (code >> 3) & 1;
    const int expo = (code >> 1) & 3;
    const int mant = code & 1;
    const double mag = expo == 0 ? 0.5 * mant : ldexp(1.0 + 0.5 * mant, expo - 1);
    return sign ? -mag : mag;
}

static double fp4_at(const uint8_t* rowbytes, int64_t t) {
    const uint8_t b = rowbytes[t >> 1];
    return oracle_e2m1_value((t & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15));
}

int oracle_wgrad_rows_fp4(const uint8_t* A, const uint8_t* sfa, int64_t hidden, const uint8_t* B,
                          const uint8_t* sfb, int64_t tokens_sum, int64_t n, int64_t begin, int64_t end,
                          const int64_t* rows, int64_t nrows, double* out) {
    if (begin < 0 || end < begin || end > tokens_sum || tokens_sum % 32 != 0) return -1;
    const int64_t half = tokens_sum / 2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        double* w = out + r * n;
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = begin; t < end; ++t) {
                const int64_t blk = t / 32;
                const double a = fp4_at(A + m * half, t) * oracle_e8m0_value(sfa[blk * hidden + m]);
                const double b = fp4_at(B + j * half, t) * oracle_e8m0_value(sfb[blk * n + j]);
                acc += a * b;
            }
            w[j] = acc;
        }
    }
    return 0;
}

int oracle_wgrad_fp4(const uint8_t* A, const uint8_t* sfa, const uint8_t* B, const uint8_t* sfb,
                     const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                     int64_t tokens_sum, double* out) {
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(hidden > 0 ? hidden : 1));
    if (!rows) return -2;
    for (int64_t m = 0; m < hidden; ++m) rows[m] = m;
    int rc = 0;
    for (int32_t e = 0; e < num_experts && rc == 0; ++e) {
        int64_t begin, end;
        oracle_expert_range(offsets, e, &begin, &end);
        rc = oracle_wgrad_rows_fp4(A, sfa, hidden, B, sfb, tokens_sum, n, begin, end, rows, hidden,
                                   out + (int64_t)e * hidden * n);
    }
    free(rows);
    return rc;
}

/* e2m1 code of v (round to nearest, ties to the even code, sign kept); magnitudes
 * that round above 6 saturate to 6 (e2m1 has no infinity or NaN; NaN -> +6 here,
 * a case the quantiser below never produces for a finite block). */
uint8_t oracle_e2m1_encode(double v) {
    const uint8_t sign = signbit(v) ? 8 : 0;
    double mag = fabs(v);
    if (isnan(v)) return 7;
    uint8_t best = 0;
    for (uint8_t c = 1; c < 8; ++c) {
        const double lo = oracle_e2m1_value((uint8_t)(c - 1)), hi = oracle_e2m1_value(c);
        if (mag > hi) { best = c; continue; }
        const double mid = 0.5 * (lo + hi);
        if (mag < mid) best = (uint8_t)(c - 1);
        else if (mag > mid) best = c;
        else best = ((c - 1) & 1) ? c : (uint8_t)(c - 1);   /* tie: the even code */
        break;
    }
    return (uint8_t)(sign | best);
}

/* Biased UE8M0 exponent of the smallest 2^k with amax <= 6 * 2^k, clamped to
 * [1, 254]; 127 for zero, 255 for NaN/inf. */
uint8_t oracle_e8m0_for_amax_fp4(double amax) {
    if (isnan(amax) || isinf(amax)) return 0xFF;
    if (amax == 0.0) return 127;
    int k = (int)ceil(log2(amax / 6.0));
    while (amax > ldexp(6.0, k)) ++k;
    while (amax <= ldexp(6.0, k - 1)) --k;
    int e = k + 127;
    if (e < 1) e = 1;
    if (e > 254) e = 254;
    return (uint8_t)e;
}

/* Quantise bf16 x (rows, cols), the token axis along the columns (cols % 32 == 0),
 * to e2m1 with one UE8M0 scale per 32 tokens: q (rows, cols/2) packed bytes,
 * s (cols/32, rows).  A block holding a NaN or an infinity gets scale 0xFF and
 * zero codes (e2m1 has no NaN code; the scale carries it). */
int oracle_quantize_fp4_tokens(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s) {
    if (cols % 32 != 0) return -1;
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            double amax = 0.0;
            int bad = 0;
            for (int64_t t = 32 * b; t < 32 * b + 32; ++t) {
                const double v = oracle_bf16_value(x[r * cols + t]);
                if (isnan(v) || isinf(v)) bad = 1;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            const uint8_t e = bad ? 0xFF : oracle_e8m0_for_amax_fp4(amax);
            s[b * rows + r] = e;
            for (int64_t t = 32 * b; t < 32 * b + 32; t += 2) {
                uint8_t lo = 0, hi = 0;
                if (!bad) {
                    lo = oracle_e2m1_encode(ldexp(oracle_bf16_value(x[r * cols + t]), 127 - (int)e));
                    hi = oracle_e2m1_encode(ldexp(oracle_bf16_value(x[r * cols + t + 1]), 127 - (int)e));
                }
                q[r * (cols / 2) + t / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}
