// Output side shared by the kernels: zero-filling a tile of an empty expert and
// writing a wave's accumulators (overwrite or accumulate; fp32, bf16 or fp16).
#pragma once

#include "kgw_device.h"
#include "kgw_internal.h"

namespace kgw {

// The output helpers take any parameter block with the fields `out`,
// `out_ptrs`, `hidden` (rows of one output matrix), `n` and `accumulate`.
//
// First byte of output matrix e (hidden x n, row-major): slab e of the dense
// output, or the caller's pointer for expert e (NULL: the expert is skipped).
template <int OUT, class P>
__device__ __forceinline__ char* expert_output(const P& p, int e) {
    constexpr int ESIZE = OUT == kOutF32 ? 4 : 2;
    if (p.out_ptrs) return (char*)p.out_ptrs[e];
    return (char*)p.out + (int64_t)e * p.hidden * p.n * ESIZE;
}

// Overwrite-mode output of an expert without tokens: +0.0 over the tile
// [m0, m0+BM) x [n0, n0+BN) of out[e], clipped to (hidden, n).
template <int OUT, int BM, int BN, int NT, class P>
__device__ __forceinline__ void zero_tile(const P& p, int e, int64_t m0, int64_t n0, int tid) {
    constexpr int ESIZE = OUT == kOutF32 ? 4 : 2;
    constexpr int PER_CHUNK = 16 / ESIZE;
    const int rows = (int)min<int64_t>(BM, p.hidden - m0);
    const int cols = (int)min<int64_t>(BN, p.n - n0);
    const int cpr = cols / PER_CHUNK;  // n is a multiple of 8: whole 16-byte chunks
    const int total = rows * cpr;
    char* base = expert_output<OUT>(p, e) + (m0 * p.n + n0) * ESIZE;
    const i32x4 z = {0, 0, 0, 0};
    for (int c = tid; c < total; c += NT) {
        const int r = c / cpr;
        const int q = c - r * cpr;
        *(i32x4*)(base + ((int64_t)r * p.n + q * PER_CHUNK) * ESIZE) = z;
    }
}

// A wave's 128x128 quarter of output matrix e's tile, held as 4 (N blocks j) x 4 (M blocks i)
// MFMA 32x32 accumulators of the transposed product: acc[j][i][4g + t] is
// out[m][n] with m = mb + 32i + (lane & 31) and n = nb + 32j + 8g + 4*(lane >> 5) + t,
// written (overwrite or accumulate, output kind OUT) through `stage`, a 32 KiB LDS region
// private to the calling wave (16-byte aligned, free of other traffic).  The
// MFMA layout gives each lane one row and four columns per register group, so
// direct stores scatter 16 bytes over 32 rows per instruction; after a
// transpose through LDS every store instruction writes whole row segments
// (fp32: 2 rows x 512 B; bf16/fp16: 8 values per lane, 4 rows x 256 B), and
// accumulate mode reads the old values the same way.  The accumulators go
// through LDS as fp32 in two passes of 64 rows (16-bit outputs are rounded
// once, after the optional add).  The LDS image holds rows of 32 16-byte chunks with
// chunk c of row r at slot c ^ (r & 31), so both the scattered writes and the
// row reads spread over all banks.  The caller must keep other waves' LDS
// traffic out of `stage` until this returns (its LDS reads are complete once
// its last store is issued).
template <int OUT, class P>
__device__ __forceinline__ void store_wave_tile_staged(const P& p, int e, int64_t mb, int64_t nb,
                                                       int lane, const f32x16 (&acc)[4][4], lds_char* stage) {
    const int64_t H = p.hidden, N = p.n;
    char* const obase = expert_output<OUT>(p, e);
    const int l32 = lane & 31, lhi = lane >> 5;
    const int c_read = lane & 31;
    const int64_t nn = nb + 4 * c_read;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * pass + ii;
            const int r = 32 * ii + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = 8 * j + 2 * g + lhi;   // columns 32j + 8g + 4lhi .. +3
                    const f32x4 w = {acc[j][i][4 * g + 0], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2],
                                     acc[j][i][4 * g + 3]};
                    lds_store_16B(stage, (uint32_t)(r * 512 + ((c ^ (r & 31)) << 4)), __builtin_bit_cast(i32x4, w));
                }
        }
        if constexpr (OUT != kOutF32) {
            // each lane: 8 consecutive columns (two chunks) -> one 16-byte store;
            // an instruction writes four rows of 256 B
            const int c2 = lane & 15;
            const int64_t nn8 = nb + 8 * c2;
#pragma unroll 4
            for (int q = 0; q < 16; ++q) {
                const int r = 4 * q + (lane >> 4);
                const f32x4 v0 = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + (((2 * c2) ^ (r & 31)) << 4))));
                const f32x4 v1 = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + (((2 * c2 + 1) ^ (r & 31)) << 4))));
                const int64_t m = mb + 64 * pass + r;
                if (m >= H || nn8 >= N) continue;
                float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                i32x4* dst = (i32x4*)(obase + (m * N + nn8) * 2);
                if (p.accumulate) {
                    const i32x4 old = *dst;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        v[2 * h] += half_lo<OUT>((uint32_t)old[h]);
                        v[2 * h + 1] += half_hi<OUT>((uint32_t)old[h]);
                    }
                }
                const i32x4 w = {(int)pack_half2<OUT>(v[0], v[1]), (int)pack_half2<OUT>(v[2], v[3]),
                                 (int)pack_half2<OUT>(v[4], v[5]), (int)pack_half2<OUT>(v[6], v[7])};
                *dst = w;
            }
        } else {
#pragma unroll 8
            for (int q = 0; q < 32; ++q) {
                const int r = 2 * q + (lane >> 5);
                f32x4 v = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + ((c_read ^ (r & 31)) << 4))));
                const int64_t m = mb + 64 * pass + r;
                if (m >= H || nn >= N) continue;
                f32x4* dst = (f32x4*)(obase + (m * N + nn) * 4);
                if (p.accumulate) v += *dst;
                *dst = v;
            }
        }
    }
}

}  // namespace kgw
