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
 * as the k-grouped weight gradient needs) each operand element is first
 * decoded to its real value e4m3(q) * 2^(scale_byte - 127) and the same sum
 * is taken over those values.
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
 * Same for fp8 operands with one UE8M0 scale per 128 tokens:
 * A: e4m3 bytes (hidden, tokens_sum); sfa: bytes (tokens_sum/128, hidden);
 * B: e4m3 bytes (tokens_sum, n);      sfb: bytes (tokens_sum/128, n).
 */
int oracle_wgrad_rows_fp8(const uint8_t* A, const uint8_t* sfa, int64_t hidden, const uint8_t* B,
                          const uint8_t* sfb, int64_t tokens_sum, int64_t n, int64_t begin,
                          int64_t end, const int64_t* rows, int64_t nrows, double* out) {
    if (begin < 0 || end < begin || end > tokens_sum) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        double* w = out + r * n;
        for (int64_t j = 0; j < n; ++j) w[j] = 0.0;
        for (int64_t k = begin; k < end; ++k) {
            const int64_t blk = k / 128;
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
                     int64_t tokens_sum, double* out) {
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(hidden > 0 ? hidden : 1));
    if (!rows) return -2;
    for (int64_t m = 0; m < hidden; ++m) rows[m] = m;
    int rc = 0;
    for (int32_t e = 0; e < num_experts && rc == 0; ++e) {
        int64_t begin, end;
        oracle_expert_range(offsets, e, &begin, &end);
        rc = oracle_wgrad_rows_fp8(A, sfa, hidden, B, sfb, tokens_sum, n, begin, end, rows, hidden,
                                   out + (int64_t)e * hidden * n);
    }
    free(rows);
    return rc;
}
