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
// element becomes e4m3fn(x * 2^-k), rounded to nearest, ties to even (tokens
// along the columns: v_cvt_scalef32_pk_fp8_bf16 on bf16 pairs with the block's
// scale; along the rows, where a lane's pairs span two columns' scales:
// v_cvt_pk_fp8_f32 after the exact multiply by 2^-k).  A block holding a NaN or an
// infinity gets scale byte 0xFF (the E8M0 NaN) and NaN bytes 0x7F.
//
// Roofline: HBM.  Per element 2 bytes read and 1 written, plus one scale byte
// per 128 elements; both layouts read every input byte once:
//   - tokens contiguous (A of the weight gradient, (hidden, tokens)): a wave
//     reads 2048 tokens of a row as four contiguous 1 KiB loads, 16 lanes make
//     one 128-token block (its maximum reduced across them), stores of 512 B;
//     a workgroup's 64 rows of scales leave through LDS as whole runs;
//   - tokens along the rows (B, (tokens, n)): a workgroup holds a 128-row x
//     128-column block in registers (each load 4 rows x 256 bytes, each store
//     4 rows x 128 bytes), reduces each column over a lane's 8 rows, the 4
//     lanes that share the column (a 32-token block) and, for 128-token
//     blocks, the 4 waves through LDS, and stores from registers.
#include <type_traits>

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

// Reductions over an aligned group of G lanes (4, 8 or 16) inside one 16-lane
// row, on the DPP data paths (no LDS round trip): swaps within quads (lanes
// xor 1, xor 2), then the half-row mirror (lane i <-> 7 - i of each 8) and the
// row mirror (i <-> 15 - i); after each step every lane holds the combination
// over its group so far, so the mirrors join whole sub-groups.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int G>
__device__ __forceinline__ int group_or(int v) {
    static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
    v |= dpp_mov<kDppXor1>(v);
    v |= dpp_mov<kDppXor2>(v);
    if constexpr (G >= 8) v |= dpp_mov<kDppHalfMirror>(v);
    if constexpr (G >= 16) v |= dpp_mov<kDppMirror>(v);
    return v;
}

// 2^(e - 127) as an fp32, for e in [1, 254] (always normal).
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return __builtin_bit_cast(float, e << 23); }

// Magnitude bit patterns of the two bf16 of a word (sign bits cleared).  Their
// integer order is the order of the magnitudes for finite values; +inf is
// 0x7F80 and every NaN lies above it, so the largest pattern of a block gives
// both its amax and whether it holds a NaN or an infinity.
constexpr uint32_t kBf16MagMask = 0x7FFF7FFFu;
constexpr uint32_t kBf16Inf = 0x7F80u;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Unsigned maximum over an aligned group of G lanes (as group_or).
template <int G>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
    static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
    v = max(v, (uint32_t)dpp_mov<kDppXor1>((int)v));
    v = max(v, (uint32_t)dpp_mov<kDppXor2>((int)v));
    if constexpr (G >= 8) v = max(v, (uint32_t)dpp_mov<kDppHalfMirror>((int)v));
    if constexpr (G >= 16) v = max(v, (uint32_t)dpp_mov<kDppMirror>((int)v));
    return v;
}

// UE8M0 byte of a 448-range (e4m3fn) block from its largest magnitude pattern
// (255 for NaN / inf).
__device__ __forceinline__ uint32_t fp8_block_exponent(uint32_t mag_bits) {
    return mag_bits >= kBf16Inf ? 255u : e8m0_for_amax(__builtin_bit_cast(float, mag_bits << 16));
}

// Four bf16 (two words, low halves first) / scale -> four e4m3fn bytes in that
// order: v_cvt_scalef32_pk_fp8_bf16 writes a word's two values into the low or
// high half of the result.  For a power-of-two scale the division is exact and
// the conversion rounds to nearest even wherever |value / scale| <= 448, which
// the quantiser's scale guarantees (tests/test_quantize_gpu.py pushes every
// finite bf16 value through it at block scales 2^-40 .. 2^30, subnormals and ties
// included, and compares with the oracle bit for bit).
typedef __attribute__((ext_vector_type(2))) short s16x2;
__device__ __forceinline__ int e4m3_quad(int w0, int w1, float scale) {
    s16x2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w1), scale, true);
    return __builtin_bit_cast(int, r);
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
// with mn = rows.  A workgroup takes 64 rows x 2048 tokens; wave w rows 16w ..
// 16w+15, one after the other (the next row's loads issued before the current
// row is converted).  A row's 2048 tokens are four 512-token chunks; in chunk k
// lane l holds tokens 512k + 8l .. +7 (each load instruction reads 1 KiB
// contiguous, each store writes 512 B), so 16 lanes make a 128-token block and
// 4 lanes a 32-token block (kScalesPacked32: the 128-token group's word is
// assembled over its 16 lanes).  The scales (mn-major: consecutive rows are
// consecutive bytes or words) collect in LDS and leave as whole runs of 64 rows
// once the workgroup is done, instead of one scattered byte per block.  Input
// and codes move with non-temporal hints (each byte is touched once; measured
// 4% faster on a 7168 x 264320 input).
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_tokens_cols(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
    constexpr bool MX = FMT == kScalesPacked32;
    constexpr int RED = MX ? 4 : 16;                     // lanes per scale block
    __shared__ uint32_t sc[16][64];   // [block or group j of the chunk][row]: scale byte (MX: the word)
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunks = (cols + 2047) / 2048;
    const int64_t rb = blockIdx.x / chunks;
    const int64_t c = blockIdx.x - rb * chunks;
    const int64_t r0 = rb * 64;
    const int64_t nb = cols / 128;
    const int64_t tl = c * 2048 + 8 * lane;              // this lane's first token in chunk 0
    const int64_t rw = r0 + 16 * wave;                   // the wave's first row
    const int nrow = (int)max<int64_t>(0, min<int64_t>(16, rows - rw));

    auto load_row = [&](int64_t r, i32x4 (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // cols is a multiple of 128: whole 16-lane groups are in or out
            if (tl + 512 * k < cols) raw[k] = __builtin_nontemporal_load((const i32x4*)(x + r * cols + tl + 512 * k));
            else raw[k] = i32x4{0, 0, 0, 0};
        }
    };
    i32x4 cur[4], nxt[4];
    if (nrow > 0) load_row(rw, cur);
    for (int i = 0; i < nrow; ++i) {
        if (i + 1 < nrow) load_row(rw + i + 1, nxt);
        const int64_t r = rw + i;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t m2 = max_u16x2(max_u16x2((uint32_t)cur[k][0] & kBf16MagMask, (uint32_t)cur[k][1] & kBf16MagMask),
                                          max_u16x2((uint32_t)cur[k][2] & kBf16MagMask, (uint32_t)cur[k][3] & kBf16MagMask));
            const uint32_t e = fp8_block_exponent(group_umax<RED>(max(m2 & 0xFFFFu, m2 >> 16)));
            uint32_t word = 0;
            if constexpr (MX) {
                // byte j of the 128-token group's word: the scale of its lanes 4j .. 4j+3
                word = (uint32_t)group_or<16>((int)(e << (8 * ((lane >> 2) & 3))));
            }
            const int64_t t = tl + 512 * k;
            if (t >= cols) continue;
            i32x2 out;
            if (e == 255u) {
                out = i32x2{0x7F7F7F7F, 0x7F7F7F7F};
            } else {
                const float sc = e8m0_scale(e);
                out[0] = e4m3_quad(cur[k][0], cur[k][1], sc);
                out[1] = e4m3_quad(cur[k][2], cur[k][3], sc);
            }
            __builtin_nontemporal_store(out, (i32x2*)(q + r * cols + t));
            if ((lane & 15) == 0) sc[4 * k + (lane >> 4)][16 * wave + i] = MX ? word : e;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
    }
    __syncthreads();

    // the chunk's scales of rows r0 .. r0+63, four rows (16 bytes for U8) per lane and store
    const int64_t vrows = min<int64_t>(64, rows - r0);
    if constexpr (FMT == kScalesU8) {
        // block j = lane >> 2 of the chunk, rows 16*(lane & 3) .. +15
        const int j = wave == 0 ? lane >> 2 : 16;
        const int64_t b = c * 16 + j;
        const int i0 = 16 * (lane & 3);
        if (j < 16 && b < nb && i0 < vrows) {
            uint8_t* dst = s + b * rows + r0 + i0;
            if (i0 + 16 <= vrows && ((uintptr_t)dst & 15u) == 0) {
                i32x4 v;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    v[m] = (int)((sc[j][i0 + 4 * m] & 0xFF) | ((sc[j][i0 + 4 * m + 1] & 0xFF) << 8) |
                                 ((sc[j][i0 + 4 * m + 2] & 0xFF) << 16) | ((sc[j][i0 + 4 * m + 3] & 0xFF) << 24));
                *(i32x4*)dst = v;
            } else {
                for (int ii = 0; ii < 16 && i0 + ii < vrows; ++ii) dst[ii] = (uint8_t)sc[j][i0 + ii];
            }
        }
    } else if constexpr (FMT == kScalesPacked) {
        // word row wq = lane >> 4 of the chunk (blocks 4wq .. 4wq+3), rows 4*(lane & 15) .. +3;
        // bytes of blocks past the last are zero
        const int wq = wave == 0 ? lane >> 4 : 4;
        const int64_t wi = c * 4 + wq;
        const int i0 = 4 * (lane & 15);
        if (wq < 4 && 4 * wi < nb && i0 < vrows) {
            uint32_t wv[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                uint32_t w = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    if (4 * wi + bb < nb) w |= (sc[4 * wq + bb][i0 + rr] & 0xFF) << (8 * bb);
                wv[rr] = w;
            }
            uint32_t* dst = (uint32_t*)s + wi * rows + r0 + i0;
            if (i0 + 4 <= vrows && ((uintptr_t)dst & 15u) == 0)
                *(i32x4*)dst = i32x4{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
            else
                for (int rr = 0; rr < 4 && i0 + rr < vrows; ++rr) dst[rr] = wv[rr];
        }
    } else {
        // groups j = 4*wave + (lane >> 4) of the chunk, rows 4*(lane & 15) .. +3
        const int j = 4 * wave + (lane >> 4);
        const int64_t g = c * 16 + j;
        const int i0 = 4 * (lane & 15);
        if (g < nb && i0 < vrows) {
            uint32_t* dst = (uint32_t*)s + g * rows + r0 + i0;
            if (i0 + 4 <= vrows && ((uintptr_t)dst & 15u) == 0)
                *(i32x4*)dst = i32x4{(int)sc[j][i0], (int)sc[j][i0 + 1], (int)sc[j][i0 + 2], (int)sc[j][i0 + 3]};
            else
                for (int rr = 0; rr < 4 && i0 + rr < vrows; ++rr) dst[rr] = sc[j][i0 + rr];
        }
    }
}

// tokens along the rows: x (rows, cols), q same layout, scales in layout FMT
// with mn = cols.  A workgroup takes 128 rows x 128 columns: wave w rows
// 32w .. 32w+31; lane l columns 8*(l & 15) .. +7 and rows (l >> 4) + 4i, i < 8
// (each load 4 rows x 256 bytes, each store 4 rows x 128 bytes: whole lines).
// Each column's maximum runs over the lane's 8 rows, then the 4 lanes sharing
// the column (xor 16, 32): that is a 32-token block (kScalesPacked32); for
// 128-token blocks the four waves' maxima meet in LDS.  LDS buffers alternate
// between units, so one barrier per unit suffices.  Input and codes move with
// non-temporal hints (measured 5% faster on a 264320 x 4096 input).
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_tokens_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s) {
    constexpr bool MX = FMT == kScalesPacked32;
    __shared__ float red_amax[2][NWAVE][128];
    __shared__ int red_bad[2][NWAVE][16];
    __shared__ uint8_t red_e[2][NWAVE][128];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cg = lane & 15, rsub = lane >> 4;
    const int64_t cchunks = (cols + 127) / 128;
    const int64_t nb = rows / 128;
    const int64_t units = nb * cchunks;
    int par = 0;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x, par ^= 1) {
        const int64_t b = u / cchunks;
        const int64_t n0 = (u - b * cchunks) * 128 + 8 * cg;
        const bool active = n0 < cols;                   // cols is a multiple of 8
        const int64_t row0 = 128 * b + 32 * wave + rsub;
        i32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (active) v[i] = __builtin_nontemporal_load((const i32x4*)(x + (row0 + 4 * i) * cols + n0));
            else v[i] = i32x4{0, 0, 0, 0};
        }
        // bit j of `bad` flags column j
        float amax[8];
        int bad = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float a = bf16_lo((uint32_t)v[i][h]), c = bf16_hi((uint32_t)v[i][h]);
                amax[2 * h] = fmaxf(amax[2 * h], fabsf(a));
                amax[2 * h + 1] = fmaxf(amax[2 * h + 1], fabsf(c));
                bad |= (not_finite(a) ? 1 : 0) << (2 * h);
                bad |= (not_finite(c) ? 1 : 0) << (2 * h + 1);
            }
#pragma unroll
        for (int m = 16; m < 64; m <<= 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], m, 64));
            bad |= __shfl_xor(bad, m, 64);
        }
        if constexpr (!MX) {
            // the four waves' 32-row maxima -> the 128-row block's
            if (rsub == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) red_amax[par][wave][8 * cg + j] = amax[j];
                red_bad[par][wave][cg] = bad;
            }
            __syncthreads();
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
#pragma unroll
                for (int j = 0; j < 8; ++j) amax[j] = fmaxf(amax[j], red_amax[par][w][8 * cg + j]);
                bad |= red_bad[par][w][cg];
            }
        }
        uint32_t e[8];
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            e[j] = ((bad >> j) & 1) ? 255u : e8m0_for_amax(amax[j]);
            f[j] = inv_scale(e[j] == 255u ? 127u : e[j]);
        }
        if (active) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float val[8];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    val[2 * h] = bf16_lo((uint32_t)v[i][h]) * f[2 * h];
                    val[2 * h + 1] = bf16_hi((uint32_t)v[i][h]) * f[2 * h + 1];
                }
                i32x2 out = {cvt4(val[0], val[1], val[2], val[3]), cvt4(val[4], val[5], val[6], val[7])};
                // NaN/infinity columns of the block: every byte of the block is NaN
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if ((bad >> j) & 1) out[j >> 2] = (out[j >> 2] & ~(0xFF << (8 * (j & 3)))) | (0x7F << (8 * (j & 3)));
                __builtin_nontemporal_store(out, (i32x2*)(q + (row0 + 4 * i) * cols + n0));
            }
        }
        if constexpr (FMT == kScalesU8) {
            if (wave == 0 && rsub == 0 && active) {
                const i32x2 sw = {(int)(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24)),
                                  (int)(e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24))};
                *(i32x2*)(s + b * cols + n0) = sw;
            }
        } else if constexpr (FMT == kScalesPacked) {
            if (wave == 0 && rsub == 0 && active) {
#pragma unroll
                for (int j = 0; j < 8; ++j) store_scale_byte<FMT>(s, b, nb, n0 + j, cols, e[j]);
            }
        } else {
            // the four waves' 32-token scales of each column -> one word
            if (rsub == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) red_e[par][wave][8 * cg + j] = (uint8_t)e[j];
            }
            __syncthreads();
            if (wave == 0 && rsub == 0 && active) {
                uint32_t w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    w[j] = (uint32_t)red_e[par][0][8 * cg + j] | ((uint32_t)red_e[par][1][8 * cg + j] << 8) |
                           ((uint32_t)red_e[par][2][8 * cg + j] << 16) | ((uint32_t)red_e[par][3][8 * cg + j] << 24);
                i32x4* dst = (i32x4*)(s + (b * cols + n0) * 4);
                dst[0] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                dst[1] = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// FP4 (OCP e2m1) quantiser: one UE8M0 scale per 32 tokens (the DeepGEMM
// k-grouped page casts a and b to FP4 with gran_k = 32).  Per block: amax = the
// largest |x|; the scale is the smallest power of two 2^k with amax <= 6 * 2^k
// (6 = largest e2m1), stored as k + 127 clamped to [1, 254] (127 for an all-zero
// block); every element becomes the nearest e2m1 of x * 2^-k (exact in fp32),
// ties to the even code.  A block holding a NaN or an infinity gets scale byte
// 0xFF and zero codes (e2m1 has no NaN).  Output codes are token-contiguous, two
// per byte, the even token in the low nibble: the operand layout of the FP4
// weight gradient (A (hidden, T/2), B (n, T/2)).
// ---------------------------------------------------------------------------

// Biased UE8M0 exponent of the smallest 2^k with amax <= 6 * 2^k, from the fp32
// bits of amax = 1.f * 2^E: 6 * 2^(E-2) = 1.5 * 2^E covers amax when 1.f <= 1.5,
// else 2^(E-1) is needed; clamped to [1, 254], 127 for zero.
__device__ __forceinline__ uint32_t e8m0_for_amax_fp4(float amax) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
    if (bits == 0u) return 127u;
    const int E = (int)(bits >> 23) - 127;               // subnormal amax gives -127: clamps to 1
    const int k = E - 2 + ((bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    const int e = k + 127;
    return (uint32_t)(e < 1 ? 1 : (e > 254 ? 254 : e));
}

// UE8M0 byte of a block from its largest magnitude pattern (255 for NaN / inf).
__device__ __forceinline__ uint32_t fp4_block_exponent(uint32_t mag_bits) {
    return mag_bits >= kBf16Inf ? 255u : e8m0_for_amax_fp4(__builtin_bit_cast(float, mag_bits << 16));
}

// Two bf16 (a word, the low half first) -> two e2m1 codes of value / scale in byte
// SEL of `acc`, the first value in the low nibble: v_cvt_scalef32_pk_fp4_bf16.
// For a power-of-two scale the division is exact, and the conversion rounds to
// the nearest e2m1 value, ties to the even code, and saturates at 6: the
// encoding the format defines (tests/test_quantize_fp4_gpu.py pushes every finite
// bf16 value through it at block scales 2^-40 .. 2^30, plus every tie point's
// neighbours and signed zeros, and compares with the oracle bit for bit).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t acc, uint32_t word, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, __builtin_bit_cast(bf16x2, word), scale, SEL);
}

// Eight bf16 values (four words) / scale -> eight e2m1 codes, value i in nibble i.
__device__ __forceinline__ uint32_t e2m1_pack8(const i32x4& w, float scale) {
    uint32_t out = e2m1_pair<0>(0u, (uint32_t)w[0], scale);
    out = e2m1_pair<1>(out, (uint32_t)w[1], scale);
    out = e2m1_pair<2>(out, (uint32_t)w[2], scale);
    return e2m1_pair<3>(out, (uint32_t)w[3], scale);
}

// tokens along the columns: x (rows, cols) -> q (rows, cols/2), scales with mn =
// rows.  The fp8 kernel's tiling: a workgroup takes 64 rows x 2048 tokens, wave w
// rows 16w .. 16w+15; in chunk k of a row lane l holds tokens 512k + 8l .. +7, so
// a quad of lanes is one 32-token block; each lane writes 4 code bytes (a wave
// 256 B contiguous).  Scales collect in LDS and leave as runs of 64 rows:
// bytes (KGW_SCALES_U8, (cols/32, rows)) or the 128-token groups' words
// (kScalesPacked32, (cols/128, rows)).
template <int FMT>
__global__ __launch_bounds__(NT) void quantize_fp4_cols(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ s) {
    constexpr bool MX = FMT == kScalesPacked32;
    __shared__ uint32_t sc[64][64];   // [32-token block (U8) or 128-token group (MX) of the chunk][row]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunks = (cols + 2047) / 2048;
    const int64_t rb = blockIdx.x / chunks;
    const int64_t c = blockIdx.x - rb * chunks;
    const int64_t r0 = rb * 64;
    const int64_t nb32 = cols / 32;
    const int64_t tl = c * 2048 + 8 * lane;
    const int64_t rw = r0 + 16 * wave;
    const int nrow = (int)max<int64_t>(0, min<int64_t>(16, rows - rw));

    auto load_row = [&](int64_t r, i32x4 (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // cols is a multiple of 128: whole 16-lane groups are in or out
            if (tl + 512 * k < cols) raw[k] = __builtin_nontemporal_load((const i32x4*)(x + r * cols + tl + 512 * k));
            else raw[k] = i32x4{0, 0, 0, 0};
        }
    };
    i32x4 cur[4], nxt[4];
    if (nrow > 0) load_row(rw, cur);
    for (int i = 0; i < nrow; ++i) {
        if (i + 1 < nrow) load_row(rw + i + 1, nxt);
        const int64_t r = rw + i;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t m2 = max_u16x2(max_u16x2((uint32_t)cur[k][0] & kBf16MagMask, (uint32_t)cur[k][1] & kBf16MagMask),
                                          max_u16x2((uint32_t)cur[k][2] & kBf16MagMask, (uint32_t)cur[k][3] & kBf16MagMask));
            const uint32_t e = fp4_block_exponent(group_umax<4>(max(m2 & 0xFFFFu, m2 >> 16)));
            uint32_t word = 0;
            if constexpr (MX) word = (uint32_t)group_or<16>((int)(e << (8 * ((lane >> 2) & 3))));
            const int64_t t = tl + 512 * k;
            if (t >= cols) continue;
            const uint32_t codes = e == 255u ? 0u : e2m1_pack8(cur[k], e8m0_scale(e));
            __builtin_nontemporal_store(codes, (uint32_t*)(q + r * (cols / 2) + t / 2));
            if constexpr (MX) {
                if ((lane & 15) == 0) sc[4 * k + (lane >> 4)][16 * wave + i] = word;
            } else {
                if ((lane & 3) == 0) sc[16 * k + (lane >> 2)][16 * wave + i] = e;
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
    }
    __syncthreads();

    const int64_t vrows = min<int64_t>(64, rows - r0);
    if constexpr (FMT == kScalesU8) {
        // block j = tid >> 2 (0..63) of the chunk, rows 16*(tid & 3) .. +15
        const int tid = threadIdx.x;
        const int j = tid >> 2;
        const int64_t b = c * 64 + j;
        const int i0 = 16 * (tid & 3);
        if (b < nb32 && i0 < vrows) {
            uint8_t* dst = s + b * rows + r0 + i0;
            if (i0 + 16 <= vrows && ((uintptr_t)dst & 15u) == 0) {
                i32x4 v;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    v[m] = (int)((sc[j][i0 + 4 * m] & 0xFF) | ((sc[j][i0 + 4 * m + 1] & 0xFF) << 8) |
                                 ((sc[j][i0 + 4 * m + 2] & 0xFF) << 16) | ((sc[j][i0 + 4 * m + 3] & 0xFF) << 24));
                *(i32x4*)dst = v;
            } else {
                for (int ii = 0; ii < 16 && i0 + ii < vrows; ++ii) dst[ii] = (uint8_t)sc[j][i0 + ii];
            }
        }
    } else {
        // group j = 4*wave + (lane >> 4) of the chunk, rows 4*(lane & 15) .. +3
        const int j = 4 * wave + (lane >> 4);
        const int64_t g = c * 16 + j;
        const int i0 = 4 * (lane & 15);
        if (g < cols / 128 && i0 < vrows) {
            uint32_t* dst = (uint32_t*)s + g * rows + r0 + i0;
            if (i0 + 4 <= vrows && ((uintptr_t)dst & 15u) == 0)
                *(i32x4*)dst = i32x4{(int)sc[j][i0], (int)sc[j][i0 + 1], (int)sc[j][i0 + 2], (int)sc[j][i0 + 3]};
            else
                for (int rr = 0; rr < 4 && i0 + rr < vrows; ++rr) dst[rr] = sc[j][i0 + rr];
        }
    }
}

// tokens along the rows: x (rows, cols) -> q (cols, rows/2), the token axis made
// contiguous (the FP4 weight gradient's B layout), scales with mn = cols.  A
// workgroup of 512 threads takes runs of FP4_ROWS_SPAN units of 256 tokens x 128
// columns that share their columns (1024 consecutive tokens): in a unit, wave w
// (0..7) takes tokens 32w .. 32w+31 -- one 32-token block -- and lane l columns
// 8*(l & 15) .. +7 and tokens 8*(l >> 4) .. +7 of the wave's 32 (each load 4 rows
// x 256 bytes; eight consecutive tokens make one 4-byte code word per column).
// The code words of the whole run collect in LDS, and each column's 512 bytes
// leave as four consecutive lines, eight lanes per column, so every store
// instruction writes whole lines (the output is transposed: stores that each
// wrote half of every line they touched ran at about 2 TB/s and took 40% of the
// kernel's time).  Scales as bytes ((rows/32, cols), stored per unit) or as the
// 128-token groups' words (assembled in LDS, stored per run).
// Units past the last 256-token chunk are skipped; a trailing 128-token half unit
// is skipped by waves 4-7.
constexpr int NT_FP4_ROWS = 512;
constexpr int FP4_ROWS_SPAN = 4;
template <int FMT>
__global__ __launch_bounds__(NT_FP4_ROWS) void quantize_fp4_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s) {
    constexpr bool MX = FMT == kScalesPacked32;
    constexpr int S = FP4_ROWS_SPAN;
    __shared__ uint32_t codes_lds[128][32 * S + 1];   // [column][token group of 8] (+1: bank spread)
    __shared__ uint8_t red_e[8 * S][128];             // [32-token block of the run][column]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = lane & 15, tg = lane >> 4;
    const int64_t cchunks = (cols + 127) / 128;
    const int64_t tchunks = (rows + 255) / 256;
    const int64_t runs = ((tchunks + S - 1) / S) * cchunks;
    // unit i of run r: its input block for this lane (zeros for lanes outside the tensor)
    auto load_unit = [&](int64_t r, int i, i32x4 (&v)[8]) __attribute__((always_inline)) {
        const int64_t g = r / cchunks;
        const int64_t n0 = (r - g * cchunks) * 128 + 8 * cg;
        const int64_t tw = 256 * (g * S + i) + 32 * wave;
        const bool active = tw < rows && n0 < cols;
        const int64_t t0 = tw + 8 * tg;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (active) v[k] = __builtin_nontemporal_load((const i32x4*)(x + (t0 + k) * cols + n0));
            else v[k] = i32x4{0, 0, 0, 0};
        }
    };
    i32x4 v[8], vn[8];
    if (blockIdx.x < runs) load_unit(blockIdx.x, 0, v);
    for (int64_t r = blockIdx.x; r < runs; r += gridDim.x) {
        const int64_t g = r / cchunks;
        const int64_t c0 = (r - g * cchunks) * 128;
        const int64_t n0 = c0 + 8 * cg;
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int64_t b = g * S + i;                     // the unit's 256-token chunk
            const int64_t tw = 256 * b + 32 * wave;          // the wave's first token
            const bool active = tw < rows && n0 < cols;      // rows: a multiple of 128; cols: of 8
            // largest magnitude pattern of columns 2h (low half) and 2h+1 (high half)
            // over the lane's 8 tokens, then over the 4 lanes of the 32-token block
            uint32_t mag[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int h = 0; h < 4; ++h) mag[h] = max_u16x2(mag[h], (uint32_t)v[k][h] & kBf16MagMask);
#pragma unroll
            for (int m = 16; m < 64; m <<= 1)
#pragma unroll
                for (int h = 0; h < 4; ++h) mag[h] = max_u16x2(mag[h], (uint32_t)__shfl_xor((int)mag[h], m, 64));
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = fp4_block_exponent((j & 1) ? mag[j >> 1] >> 16 : mag[j >> 1] & 0xFFFFu);
            // column j's eight tokens: value k of the word is token t0 + k; tokens 2p and
            // 2p+1 of the column are joined into one bf16 pair (v_perm_b32) and converted
            // together into byte p
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float sc_j = e8m0_scale(e[j] == 255u ? 127u : e[j]);
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                uint32_t codes = e2m1_pair<0>(0u, __builtin_amdgcn_perm((uint32_t)v[1][j >> 1], (uint32_t)v[0][j >> 1], sel), sc_j);
                codes = e2m1_pair<1>(codes, __builtin_amdgcn_perm((uint32_t)v[3][j >> 1], (uint32_t)v[2][j >> 1], sel), sc_j);
                codes = e2m1_pair<2>(codes, __builtin_amdgcn_perm((uint32_t)v[5][j >> 1], (uint32_t)v[4][j >> 1], sel), sc_j);
                codes = e2m1_pair<3>(codes, __builtin_amdgcn_perm((uint32_t)v[7][j >> 1], (uint32_t)v[6][j >> 1], sel), sc_j);
                if (e[j] == 255u) codes = 0;
                codes_lds[8 * cg + j][32 * i + 4 * wave + tg] = codes;
            }
            if constexpr (!MX) {
                if (tg == 0 && active) {
                    const i32x2 sw = {(int)(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24)),
                                      (int)(e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24))};
                    *(i32x2*)(s + (8 * b + wave) * cols + n0) = sw;
                }
            } else {
                if (tg == 0) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) red_e[8 * i + wave][8 * cg + j] = (uint8_t)e[j];
                }
            }
            // the next unit's loads go out before this unit's conversions finish
            if (i + 1 < S) load_unit(r, i + 1, vn);
            else if (r + gridDim.x < runs) load_unit(r + gridDim.x, 0, vn);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = vn[k];
        }
        __syncthreads();
        // codes: in pass p, thread -> column 64p + (tid >> 3); store m writes bytes
        // 16*(tid & 7) .. +15 of the column's line m (unit m: 256 tokens, 128 bytes), so every
        // store instruction writes eight whole lines and each column's run leaves in order
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int col = 64 * pass + (tid >> 3), l8 = tid & 7;
            if (c0 + col < cols) {
                uint8_t* dst_col = q + (c0 + col) * (rows / 2) + 128 * g * S + 16 * l8;
#pragma unroll
                for (int m = 0; m < S; ++m) {
                    const int64_t tchunk = 256 * (g * S + m) + 32 * l8;   // the chunk's first token
                    if (tchunk < rows) {
                        const uint32_t* src = &codes_lds[col][32 * m + 4 * l8];
                        __builtin_nontemporal_store(i32x4{(int)src[0], (int)src[1], (int)src[2], (int)src[3]},
                                                    (i32x4*)(dst_col + 128 * m));
                    }
                }
            }
        }
        if constexpr (MX) {
            // the run's 2S 128-token groups: word (group, column) from blocks 4*group .. +3
            const int col = tid & 127;
#pragma unroll
            for (int k = 0; k < (2 * S + 3) / 4; ++k) {
                const int grp = (tid >> 7) + 4 * k;
                const int64_t gg = 2 * g * S + grp;
                if (grp < 2 * S && c0 + col < cols && 128 * gg < rows) {
                    const uint32_t w = (uint32_t)red_e[4 * grp][col] | ((uint32_t)red_e[4 * grp + 1][col] << 8) |
                                       ((uint32_t)red_e[4 * grp + 2][col] << 16) |
                                       ((uint32_t)red_e[4 * grp + 3][col] << 24);
                    ((uint32_t*)s)[gg * cols + c0 + col] = w;
                }
            }
        }
        __syncthreads();                                  // the LDS is refilled by the next run
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

hipError_t launch_quantize_fp4(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                               void* q, void* s, int num_cus, hipStream_t stream) {
    const bool mx = scale_format == kScalesPacked32;
    if (token_axis) {
        const int64_t blocks = ((rows + 63) / 64) * ((cols + 2047) / 2048);
        if (blocks < 1 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        if (mx)
            hipLaunchKernelGGL(quantize_fp4_cols<kScalesPacked32>, dim3((unsigned)blocks), dim3(NT), 0, stream,
                               (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
        else
            hipLaunchKernelGGL(quantize_fp4_cols<kScalesU8>, dim3((unsigned)blocks), dim3(NT), 0, stream,
                               (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
    } else {
        int64_t blocks = ((rows + 256 * FP4_ROWS_SPAN - 1) / (256 * FP4_ROWS_SPAN)) * ((cols + 127) / 128);
        const int64_t cap = (int64_t)num_cus * 8;
        if (blocks > cap) blocks = cap;
        if (blocks < 1) blocks = 1;
        if (mx)
            hipLaunchKernelGGL(quantize_fp4_rows<kScalesPacked32>, dim3((unsigned)blocks), dim3(NT_FP4_ROWS), 0,
                               stream, (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
        else
            hipLaunchKernelGGL(quantize_fp4_rows<kScalesU8>, dim3((unsigned)blocks), dim3(NT_FP4_ROWS), 0, stream,
                               (const uint16_t*)x, rows, cols, (uint8_t*)q, (uint8_t*)s);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                               void* q, void* s, int num_cus, hipStream_t stream) {
    // cols: one workgroup per 64 rows x 2048 tokens (no loop); rows: workgroups stride over
    // the 128 x 128 blocks
    int64_t blocks;
    if (token_axis) {
        blocks = ((rows + 63) / 64) * ((cols + 2047) / 2048);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    } else {
        blocks = (rows / 128) * ((cols + 127) / 128);
        const int64_t cap = (int64_t)num_cus * 16;
        if (blocks > cap) blocks = cap;
    }
    if (blocks < 1) blocks = 1;
    if (scale_format == kScalesPacked32) launch_fmt<kScalesPacked32>(x, rows, cols, token_axis, q, s, blocks, stream);
    else if (scale_format == kScalesPacked) launch_fmt<kScalesPacked>(x, rows, cols, token_axis, q, s, blocks, stream);
    else launch_fmt<kScalesU8>(x, rows, cols, token_axis, q, s, blocks, stream);
    return hipGetLastError();
}

}  // namespace kgw
