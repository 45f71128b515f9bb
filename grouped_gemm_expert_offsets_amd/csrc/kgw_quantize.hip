// Token-axis fp8 quantiser (gfx950): bf16 -> OCP e4m3fn bytes plus one UE8M0
// scale byte per 128 tokens, the operand format the fp8 weight-gradient
// kernels consume (llm-infra-atlas "05 Grouped GEMM", section 3: 1x128
// blocks, power-of-two UE8M0 scales; for the k-grouped weight gradient the
// blocks run along the contracted token axis, section 5.2).  The scales come
// out as bytes (mn-major), packed four consecutive blocks to a little-endian
// word, or -- with one scale per 32 tokens, the DeepGEMM k-grouped page's
// gran_k = 32 -- as one packed word per 128 tokens.
//
// Per block: amax = the largest |x|; the scale is the smallest power of two
// 2^k with amax <= 448 * 2^k (448 = largest e4m3fn), stored as the biased
// exponent k + 127 clamped to [1, 254] (127 for an all-zero block); every
// element becomes e4m3fn(x * 2^-k), rounded to nearest, ties to even
// (v_cvt_pk_fp8_f32; x * 2^-k is exact in fp32).  A block holding a NaN or an
// infinity gets scale byte 0xFF (the E8M0 NaN) and NaN bytes 0x7F.
//
// Roofline: HBM.  Per element 2 bytes read and 1 written, plus one scale byte
// per 128 elements; both layouts read every input byte once:
//   - tokens contiguous (A of the weight gradient, (hidden, tokens)): a lane
//     holds 16 tokens (two 16-byte loads), 8 lanes one 128-token block; the
//     block maximum is reduced across the 8 lanes; 16-byte stores;
//   - tokens along the rows (B, (tokens, n)): a wave holds a 128-row x 64-column
//     block in registers (lane: 8 columns of 16 rows, each load 8 rows x 128
//     bytes), reduces each column over its 16 rows (four 32-row sub-blocks
//     of 4 rows each for 32-token scales) and then across the 8 lanes that
//     share the column, and stores from registers.
#include "kgw_device.h"
#include "kgw_internal.h"

namespace kgw {
namespace {

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;

// Biased UE8M0 exponent of the smallest 2^k with amax <= 448 * 2^k, from the
// fp32 bits of amax (amax = 1.f * 2^E; 448 = 1.75 * 2^8: k = E - 8 when
// 1.f <= 1.75, else E - 7), clamped to [1, 254]; 127 for zero.
__device__ __forceinline__ uint32_t e8m0_for_amax(float amax) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
    if (bits == 0u) return 127u;
    const int E = (int)(bits >> 23) - 127;               // subnormal amax gives -127: clamps to 1
    const int k = E - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    const int e = k + 127;
    return (uint32_t)(e < 1 ? 1 : (e > 254 ? 254 : e));
}

// 2^(127 - e) as an fp32, for e in [1, 254] (normal for every e a finite bf16
// block can produce; e = 254 would need amax above the bf16 range).
__device__ __forceinline__ float inv_scale(uint32_t e) {
    const uint32_t field = 254u - e;
    return __builtin_bit_cast(float, field == 0u ? 0x00400000u : (field << 23));
}

__device__ __forceinline__ bool not_finite(float v) {
    return (__builtin_bit_cast(uint32_t, v) & 0x7F800000u) == 0x7F800000u;
}

// Four fp32 -> four e4m3fn bytes (little-endian order).
__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// Store the scale of 128-token block b (of nb) for mn index o (of mn) in layout FMT
// (kScalesU8 or kScalesPacked); the lane that stores a packed word's last block
// also zeroes the word's unused bytes.
template <int FMT>
__device__ __forceinline__ void store_scale_byte(uint8_t* s, int64_t b, int64_t nb, int64_t o, int64_t mn,
                                                 uint32_t e) {
    if constexpr (FMT == kScalesU8) {
        s[b * mn + o] = (uint8_t)e;
    } else {
        uint8_t* w = s + (b >> 2) * 4 * mn + 4 * o;
        w[b & 3] = (uint8_t)e;
        if (b == nb - 1)
            for (int64_t j = (b & 3) + 1; j < 4; ++j) w[j] = 0;
    }
}

// tokens along the columns: x (rows, cols), q same layout, scales in layout FMT
// with mn = rows.  Lane l: tokens 16l .. 16l+15 of the wave's 1024 (two 16-byte
// loads, one 16-byte store); 8 lanes make one 128-token block, 2 lanes one
// 32-token block (kScalesPacked32, whose word for a 128-token group is
// assembled from the four pairs and stored by the group's first lane).
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_tokens_cols(const uint16_t* x, int64_t rows, int64_t cols,
                                                          uint8_t* q, uint8_t* s) {
    constexpr int RED = FMT == kScalesPacked32 ? 2 : 8;   // lanes per scale block
    const int lane = threadIdx.x & 63;
    const int64_t chunks = (cols + 1023) / 1024;         // 1024 tokens (eight blocks) per wave step
    const int64_t units = rows * chunks;
    const int64_t nb = cols / 128;
    const int64_t wave0 = (int64_t)blockIdx.x * NWAVE + (threadIdx.x >> 6);
    for (int64_t u = wave0; u < units; u += (int64_t)gridDim.x * NWAVE) {
        const int64_t r = u / chunks;
        const int64_t c = u - r * chunks;
        const int64_t t0 = c * 1024 + 16 * lane;        // this lane's first token
        const bool active = t0 < cols;                   // cols is a multiple of 128: whole 8-lane groups
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        if (active) {
            const i32x4 r0 = *(const i32x4*)(x + r * cols + t0);
            const i32x4 r1 = *(const i32x4*)(x + r * cols + t0 + 8);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_lo((uint32_t)r0[h]);
                v[2 * h + 1] = bf16_hi((uint32_t)r0[h]);
                v[8 + 2 * h] = bf16_lo((uint32_t)r1[h]);
                v[8 + 2 * h + 1] = bf16_hi((uint32_t)r1[h]);
            }
        }
        float amax = 0.0f;
        int bad = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            amax = fmaxf(amax, fabsf(v[i]));
            bad |= not_finite(v[i]) ? 1 : 0;
        }
        // reduce over the lanes of the block (xor 1, 2, 4 stays in the 8-lane group)
#pragma unroll
        for (int m = 1; m < RED; m <<= 1) {
            amax = fmaxf(amax, __shfl_xor(amax, m, 64));
            bad |= __shfl_xor(bad, m, 64);
        }
        const uint32_t e = bad ? 255u : e8m0_for_amax(amax);
        uint32_t word = 0;
        if constexpr (FMT == kScalesPacked32) {
            const int g0 = lane & ~7;                     // the 128-token group's first lane
#pragma unroll
            for (int j = 0; j < 4; ++j) word |= (uint32_t)__shfl((int)e, g0 + 2 * j, 64) << (8 * j);
        }
        if (!active) continue;
        i32x4 out;
        if (bad) {
            out = i32x4{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
        } else {
            const float f = inv_scale(e);
#pragma unroll
            for (int h = 0; h < 4; ++h) out[h] = cvt4(v[4 * h] * f, v[4 * h + 1] * f, v[4 * h + 2] * f, v[4 * h + 3] * f);
        }
        *(i32x4*)(q + r * cols + t0) = out;
        if ((lane & 7) == 0) {
            if constexpr (FMT == kScalesPacked32) ((uint32_t*)s)[(t0 / 128) * rows + r] = word;
            else store_scale_byte<FMT>(s, t0 / 128, nb, r, rows, e);
        }
    }
}

// tokens along the rows: x (rows, cols), q same layout, scales in layout FMT
// with mn = cols.  Lane l: columns 8*(l & 7) .. +7 of the wave's 64, rows
// (l >> 3) + 8*i, i < 16, of one 128-row block; with 32-token blocks
// (kScalesPacked32) rows i = 4k .. 4k+3 of every lane form sub-block k.
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_tokens_rows(const uint16_t* x, int64_t rows, int64_t cols,
                                                          uint8_t* q, uint8_t* s) {
    constexpr int NSUB = FMT == kScalesPacked32 ? 4 : 1;  // scale blocks per 128 rows
    const int lane = threadIdx.x & 63;
    const int64_t cchunks = (cols + 63) / 64;
    const int64_t nb = rows / 128;
    const int64_t units = nb * cchunks;
    const int64_t wave0 = (int64_t)blockIdx.x * NWAVE + (threadIdx.x >> 6);
    const int rsub = lane >> 3;
    for (int64_t u = wave0; u < units; u += (int64_t)gridDim.x * NWAVE) {
        const int64_t b = u / cchunks;
        const int64_t n0 = (u - b * cchunks) * 64 + 8 * (lane & 7);
        const bool active = n0 < cols;                   // cols is a multiple of 8
        i32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t row = 128 * b + rsub + 8 * i;
            if (active) v[i] = *(const i32x4*)(x + row * cols + n0);
            else v[i] = i32x4{0, 0, 0, 0};
        }
        // per column (8 per lane) and sub-block: max over this lane's rows of
        // the sub-block, then over the 8 lanes with the same column group (xor
        // 8, 16, 32); bit 8k + j of `bad` flags column j of sub-block k
        float amax[NSUB][8];
        int bad = 0;
#pragma unroll
        for (int k = 0; k < NSUB; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) amax[k][j] = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = i / (16 / NSUB);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float a = bf16_lo((uint32_t)v[i][h]), c = bf16_hi((uint32_t)v[i][h]);
                amax[k][2 * h] = fmaxf(amax[k][2 * h], fabsf(a));
                amax[k][2 * h + 1] = fmaxf(amax[k][2 * h + 1], fabsf(c));
                bad |= (not_finite(a) ? 1 : 0) << (8 * k + 2 * h);
                bad |= (not_finite(c) ? 1 : 0) << (8 * k + 2 * h + 1);
            }
        }
#pragma unroll
        for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
            for (int k = 0; k < NSUB; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) amax[k][j] = fmaxf(amax[k][j], __shfl_xor(amax[k][j], m, 64));
            bad |= __shfl_xor(bad, m, 64);
        }
        if (!active) continue;
        uint32_t e[NSUB][8];
        float f[NSUB][8];
#pragma unroll
        for (int k = 0; k < NSUB; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                e[k][j] = ((bad >> (8 * k + j)) & 1) ? 255u : e8m0_for_amax(amax[k][j]);
                f[k][j] = inv_scale(e[k][j] == 255u ? 127u : e[k][j]);
            }
        if (rsub == 0) {
            if constexpr (FMT == kScalesU8) {
                const i32x2 sw = {(int)(e[0][0] | (e[0][1] << 8) | (e[0][2] << 16) | (e[0][3] << 24)),
                                  (int)(e[0][4] | (e[0][5] << 8) | (e[0][6] << 16) | (e[0][7] << 24))};
                *(i32x2*)(s + b * cols + n0) = sw;
            } else if constexpr (FMT == kScalesPacked) {
#pragma unroll
                for (int j = 0; j < 8; ++j) store_scale_byte<FMT>(s, b, nb, n0 + j, cols, e[0][j]);
            } else {
                uint32_t w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) w[j] = e[0][j] | (e[1][j] << 8) | (e[2][j] << 16) | (e[3][j] << 24);
                i32x4* dst = (i32x4*)(s + (b * cols + n0) * 4);
                dst[0] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                dst[1] = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = i / (16 / NSUB);
            float val[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                val[2 * h] = bf16_lo((uint32_t)v[i][h]) * f[k][2 * h];
                val[2 * h + 1] = bf16_hi((uint32_t)v[i][h]) * f[k][2 * h + 1];
            }
            i32x2 out = {cvt4(val[0], val[1], val[2], val[3]), cvt4(val[4], val[5], val[6], val[7])};
            // NaN/infinity columns of the sub-block: every byte of the block is NaN
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((bad >> (8 * k + j)) & 1) out[j >> 2] = (out[j >> 2] & ~(0xFF << (8 * (j & 3)))) | (0x7F << (8 * (j & 3)));
            const int64_t row = 128 * b + rsub + 8 * i;
            *(i32x2*)(q + row * cols + n0) = out;
        }
    }
}

}  // namespace

template <int FMT>
static void launch_fmt(const void* x, int64_t rows, int64_t cols, int32_t token_axis, void* q, void* s,
                       int64_t blocks, hipStream_t stream) {
    if (token_axis)
        hipLaunchKernelGGL(quantize_tokens_cols<FMT>, dim3((unsigned)blocks), dim3(NT), 0, stream,
                           (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
    else
        hipLaunchKernelGGL(quantize_tokens_rows<FMT>, dim3((unsigned)blocks), dim3(NT), 0, stream,
                           (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
}

hipError_t launch_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                               void* q, void* s, int num_cus, hipStream_t stream) {
    const int64_t units = token_axis ? rows * ((cols + 1023) / 1024) : (rows / 128) * ((cols + 63) / 64);
    int64_t blocks = (units + NWAVE - 1) / NWAVE;
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (scale_format == kScalesPacked32) launch_fmt<kScalesPacked32>(x, rows, cols, token_axis, q, s, blocks, stream);
    else if (scale_format == kScalesPacked) launch_fmt<kScalesPacked>(x, rows, cols, token_axis, q, s, blocks, stream);
    else launch_fmt<kScalesU8>(x, rows, cols, token_axis, q, s, blocks, stream);
    return hipGetLastError();
}

}  // namespace kgw
