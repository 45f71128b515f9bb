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
    gbl_char* base = (gbl_char*)expert_output<OUT>(p, e) + (m0 * p.n + n0) * ESIZE;
    const i32x4 z = {0, 0, 0, 0};
    for (int c = tid; c < total; c += NT) {
        const int r = c / cpr;
        const int q = c - r * cpr;
        __builtin_nontemporal_store(z, (gbl_i32x4*)(base + ((int64_t)r * p.n + q * PER_CHUNK) * ESIZE));
    }
}

// Overwrite-mode output of an expert without tokens, written as contiguous parts:
// part `part` of `parts` equal runs of 16-byte chunks of output matrix e (the
// expert's whole hidden x n slab; n is a multiple of 8, so the slab is whole
// chunks).  The `parts` items of one expert together cover its slab once.
template <int OUT, int NT, class P>
__device__ __forceinline__ void zero_slab_part(const P& p, int e, int part, int parts, int tid) {
    constexpr int ESIZE = OUT == kOutF32 ? 4 : 2;
    const int64_t chunks = p.hidden * p.n * ESIZE / 16;
    const int64_t per = (chunks + parts - 1) / parts;
    const int64_t c0 = (int64_t)part * per;
    const int64_t c1 = min(chunks, c0 + per);
    gbl_i32x4* base = (gbl_i32x4*)expert_output<OUT>(p, e);
    const i32x4 z = {0, 0, 0, 0};
    for (int64_t c = c0 + tid; c < c1; c += NT) __builtin_nontemporal_store(z, base + c);
}

// Rows [m_pass, m_pass + 64) x columns [nb, nb + 128) of one output matrix (base
// `obase`, hidden x n) from their fp32 LDS image in `stage` (layout: see
// store_wave_tile_staged), overwriting or (ACC) adding the old values first.
// Accumulate mode loads the old values of eight row segments before storing any
// of them, so eight loads per lane are in flight at once (the compiler cannot
// tell the stores from later loads, so it would otherwise wait out one load per
// store); the two modes are separate code so that overwrite stores never wait
// on the accumulate loads' counter.  With FULL (all 64 x 128 inside the matrix)
// nothing is checked per lane; otherwise lanes outside the matrix load its first
// 16 bytes instead (no branch per load) and store nothing.  LDS reads run a few
// rows ahead of the stores.
template <int OUT, bool ACC, bool FULL>
__device__ __forceinline__ void store_rows_from_lds(gbl_char* obase, int64_t m_pass, int64_t nb, int64_t H,
                                                    int64_t N, int lane, lds_char* stage) {
    if constexpr (OUT != kOutF32) {
        // each lane: 8 consecutive columns (two chunks) -> one 16-byte store;
        // an instruction writes four rows of 256 B; two batches of eight row groups
        // (old values, then LDS reads and stores four at a time)
        const int c2 = lane & 15;
        const int64_t nn8 = nb + 8 * c2;
        const bool col_ok = FULL || nn8 < N;
#pragma unroll
        for (int q0 = 0; q0 < 16; q0 += 8) {
            i32x4 old[8];
            if constexpr (ACC) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t m = m_pass + 4 * (q0 + u) + (lane >> 4);
                    const int64_t off = FULL || (m < H && col_ok) ? (m * N + nn8) * 2 : 0;
                    old[u] = __builtin_nontemporal_load((const gbl_i32x4*)(obase + off));
                }
            }
#pragma unroll
            for (int q1 = 0; q1 < 8; q1 += 4) {
                f32x4 v0[4], v1[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = 4 * (q0 + q1 + u) + (lane >> 4);
                    v0[u] = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + (((2 * c2) ^ (r & 31)) << 4))));
                    v1[u] = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + (((2 * c2 + 1) ^ (r & 31)) << 4))));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t m = m_pass + 4 * (q0 + q1 + u) + (lane >> 4);
                    if (!FULL && (m >= H || !col_ok)) continue;
                    float v[8] = {v0[u][0], v0[u][1], v0[u][2], v0[u][3], v1[u][0], v1[u][1], v1[u][2], v1[u][3]};
                    if constexpr (ACC) {
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            v[2 * h] += half_lo<OUT>((uint32_t)old[q1 + u][h]);
                            v[2 * h + 1] += half_hi<OUT>((uint32_t)old[q1 + u][h]);
                        }
                    }
                    const i32x4 w = {(int)pack_half2<OUT>(v[0], v[1]), (int)pack_half2<OUT>(v[2], v[3]),
                                     (int)pack_half2<OUT>(v[4], v[5]), (int)pack_half2<OUT>(v[6], v[7])};
                    __builtin_nontemporal_store(w, (gbl_i32x4*)(obase + (m * N + nn8) * 2));
                }
            }
        }
    } else {
        // each lane: 4 consecutive columns; an instruction writes two rows of 512 B;
        // four batches of eight row pairs (old values, then LDS reads, then stores)
        const int l32 = lane & 31, lhi = lane >> 5;
        const int64_t nn = nb + 4 * l32;
        const bool col_ok = FULL || nn < N;
#pragma unroll
        for (int u0 = 0; u0 < 32; u0 += 8) {
            f32x4 old[8], v[8];
            if constexpr (ACC) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t m = m_pass + 2 * (u0 + u) + lhi;
                    const int64_t off = FULL || (m < H && col_ok) ? (m * N + nn) * 4 : 0;
                    old[u] = __builtin_nontemporal_load((const gbl_f32x4*)(obase + off));
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 2 * (u0 + u) + lhi;
                v[u] = __builtin_bit_cast(f32x4, lds_load_16B(stage, (uint32_t)(r * 512 + ((l32 ^ (r & 31)) << 4))));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t m = m_pass + 2 * (u0 + u) + lhi;
                if (!FULL && (m >= H || !col_ok)) continue;
                if constexpr (ACC) v[u] += old[u];
                __builtin_nontemporal_store(v[u], (gbl_f32x4*)(obase + (m * N + nn) * 4));
            }
        }
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
// row reads spread over all banks.  All output accesses go through global (not
// flat) pointers, so they never hold up the LDS reads' counter, and carry
// non-temporal hints: each output byte is read (accumulate) and written once
// per call (measured 6% faster on the E=256 fp32 workload, whose 15 GB output
// write dominates).  The caller
// must keep other waves' LDS traffic out of `stage` until this returns (its LDS
// reads are complete once its last store is issued).
template <int OUT, class P>
__device__ __forceinline__ void store_wave_tile_staged(const P& p, int e, int64_t mb, int64_t nb,
                                                       int lane, const f32x16 (&acc)[4][4], lds_char* stage) {
    // the matrix's base address is wave-uniform: keep it in scalar registers (a pointer
    // read from `out_ptrs` would otherwise stay a pending vector load for every access)
    const uint64_t ob = (uint64_t)expert_output<OUT>(p, e);
    gbl_char* const obase = (gbl_char*)(((uint64_t)__builtin_amdgcn_readfirstlane((int)(ob >> 32)) << 32) |
                                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ob));
    const int l32 = lane & 31, lhi = lane >> 5;
    const bool full = mb + 128 <= p.hidden && nb + 128 <= p.n;   // the wave's whole 128 x 128
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
        const int64_t m_pass = mb + 64 * pass;
        if (full) {
            if (p.accumulate)
                store_rows_from_lds<OUT, true, true>(obase, m_pass, nb, p.hidden, p.n, lane, stage);
            else
                store_rows_from_lds<OUT, false, true>(obase, m_pass, nb, p.hidden, p.n, lane, stage);
        } else {
            if (p.accumulate)
                store_rows_from_lds<OUT, true, false>(obase, m_pass, nb, p.hidden, p.n, lane, stage);
            else
                store_rows_from_lds<OUT, false, false>(obase, m_pass, nb, p.hidden, p.n, lane, stage);
        }
    }
}

}  // namespace kgw
