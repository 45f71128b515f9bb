// Persistent m-grouped GEMM, bf16 operands, fp32 accumulation (gfx950): the
// forward and dgrad products of the same MoE experts whose weight gradient the
// k-grouped kernels compute (llm-infra-atlas "05 Grouped GEMM": section 1,
// grouping only along M; section 2.1, the contiguous layout with per-row group
// ids or offsets; section 5.1, dgrad is m-grouped as well).
//
//     forward, "nt": out[m, :] = A[m, :] @ W[g(m)]^T     W (E, N, K)
//     dgrad,   "nn": out[m, :] = A[m, :] @ W[g(m)]       W (E, K, N)
//
// A (M, K) is K-contiguous.  Row m's group g(m) comes from per-row ids
// (m_indices) or from inclusive cumulative offsets (the first e with
// offsets[e] > m); a row of no group (id < 0 or >= E, or past the last offset)
// is neither computed nor written.  Groups start on multiples of 128 rows.
//
// Work decomposition: one item per 256x256 output tile (M-first columns of four
// tiles, persistent grid, XCD-aware slots as in the k-grouped kernels).  The
// two 128-row halves of a tile each lie in one group.  When they lie in two
// different groups the tile's item computes half 0 with its group and a second
// item, in a second list after all tiles, half 1 with the other: each loads only
// its half's A rows (the other half's rows read as zeros through the buffer
// range) and stores only its half, so only such boundary tiles do extra MFMA
// work, and every item of the first list costs one K loop.  A half of no group is
// not stored.
//
// K loop (K a multiple of 64): the k-grouped bf16 kernel's pipeline.  A moves
// in 64-token stages of full 128-byte rows through a 3-slot ring.  nn: W[g] is
// N-contiguous and moves like the k-grouped kernel's B (32-row stages, 4-slot
// ring, transposing ds_read_b64_tr_b16 fragments).  nt: W[g] is K-contiguous
// like A, so it moves like A (64-token stages of full 128-byte rows, plain
// 16-byte fragment reads) through a 2-slot ring (3 x 32 + 2 x 32 KiB = all of
// the LDS); a whole B stage is issued in the odd step two steps before its first
// use, since its slot only frees when the stage before the previous one has been
// read.
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NT = 256;
constexpr int NA = 3;                       // A ring: 3 stages of 2 K steps
constexpr int A_STAGE = BM * 2 * BK * 2;    // 32 KiB: 256 rows x 128 B
constexpr int B_RING = NA * A_STAGE;
constexpr int GROUP_M = 4;
constexpr int B_LOADS = 4;                  // nn: direct loads per wave per B step

// nn: B ring of 4 one-step stages (32 k-rows x 512 B); nt: 2 two-step stages
// (256 n-rows x 128 B).
template <bool BT>
struct BRing {
    static constexpr int slots = BT ? 2 : 4;
    static constexpr int stage = BT ? A_STAGE : BK * BN * 2;
};
static_assert(B_RING + 4 * BK * BN * 2 <= 160 * 1024 && B_RING + 2 * A_STAGE <= 160 * 1024, "LDS budget");

template <int OUT, bool BT>
__global__ __launch_bounds__(NT, 1) void mgrouped_bf16_kernel(MGroupedParams p) {
    constexpr int NB = BRing<BT>::slots;
    constexpr int B_STAGE = BRing<BT>::stage;
    __shared__ __attribute__((aligned(1024))) char smem[B_RING + NB * B_STAGE];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t M = p.hidden, N = p.n, K = p.k;

    // Direct-load slots.  A (and nt's B): wave instruction t (0..7) fills LDS
    // rows 64*wave + 8*t + (lane>>3), 16-byte slot lane&7 = logical chunk ^
    // ((row>>1)&7).  nn's B: instruction t (0..3) fills k-rows 8*wave + 2*t +
    // (lane>>5), slot lane&31 = logical chunk ^ 4*(k&3).
    int a_q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) a_q[t] = (lane & 7) ^ ((4 * t + (lane >> 4)) & 7);
    int b_q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b_q[t] = (lane & 31) ^ (((2 * t + (lane >> 5)) & 3) << 2);

    // Fragment read offsets (fixed per lane): A rows wm*128 + 32i + l32; nt's B
    // rows (n) wn*128 + 32j + l32 with the same chunk swizzle; nn's B as in the
    // k-grouped kernel.
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u;
    const uint32_t bt_frag_row = (uint32_t)(wn * 128 + l32) * 128u;
    const int a_sw = (l32 >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    uint32_t b_frag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 8 * (g16 >> 1) + (i16 >> 2);
        const int chunk = 16 * wn + 2 * (g16 & 1) + ((i16 & 3) >> 1) + 4 * (j ^ (i16 >> 2));
        b_frag[j] = (uint32_t)krow * 512u + (uint32_t)chunk * 16u + (uint32_t)(i16 & 1) * 8u;
    }

    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);
    const int kst = (int)(K / BK);          // K steps of one pass (even)

    for (int item = slot; item < p.num_items; item += G) {
        // Items num_tiles.. are the second halves of the tiles whose 128-row halves lie in
        // two groups: such a tile's first item computes half 0 with group g0, its second
        // item half 1 with g1, each a K loop with the other half's A rows read as zeros.
        // (As one item with two K loops it held up its workgroup a whole tile behind the
        // others of its XCD, which then stopped sharing operand panels in the XCD's L2.)
        const bool second = item >= p.num_tiles;
        int tm, tn;
        tile_coords(second ? item - p.num_tiles : item, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        // Groups of the two 128-row halves.
        const int g0 = group_of_row(p, m0);
        const int g1 = m0 + 128 < M ? group_of_row(p, m0 + 128) : -1;
        const bool v0 = g0 >= 0 && g0 < p.num_groups;
        const bool v1 = g1 >= 0 && g1 < p.num_groups;
        if (!v0 && !v1) continue;
        const bool split = v0 && v1 && g0 != g1;      // one item per half, A rows masked
        if (second && !split) continue;
        const int grp = second ? g1 : (v0 ? g0 : g1);
        const int live_half = split ? (second ? 1 : 0) : -1;   // -1: both halves' A rows
        const int ksteps = kst;
        const int rows_valid = (int)min<int64_t>(BM, M - m0);
        if (ksteps == 0) {                              // K == 0: the product is zero
            if (!p.accumulate && !second) {
                if (v0) zero_tile<OUT, 128, BN, NT>(p, 0, m0, n0, tid);
                if (v1) zero_tile<OUT, 128, BN, NT>(p, 0, m0 + 128, n0, tid);
            }
            continue;
        }

        const char* Abase = (const char*)p.A + m0 * K * 2;
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        uint32_t a_voff[8], bt_voff[8], b_voff[4];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = min(64 * wave + 8 * t + (lane >> 3), rows_valid - 1);
            a_voff[t] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)a_q[t] * 16u;
            const int nrow = min(64 * wave + 8 * t + (lane >> 3), cols_valid - 1);
            bt_voff[t] = (uint32_t)nrow * (uint32_t)(K * 2) + (uint32_t)a_q[t] * 16u;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int krow = 8 * wave + 2 * t + (lane >> 5);
            b_voff[t] = (uint32_t)krow * (uint32_t)(N * 2) + (uint32_t)min(8 * b_q[t], cols_valid - 8) * 2u;
        }
        // The item's group's weight; the A loads of waves 0-1 cover tile rows 0-127 and
        // those of waves 2-3 rows 128-255 (row = 64*wave + ...), so for one half of a split
        // tile the other half's waves load A from an empty range (zeros).
        const char* W0 = (const char*)p.W + (int64_t)grp * K * N * 2;
        const int my_half = wave >> 1;
        const bool a_live = live_half < 0 || my_half == live_half;

        // A stage a (steps 2a, 2a+1) to slot a % NA, load `t` of the wave's eight.
        auto dma_a = [&](int a, int t) __attribute__((always_inline)) {
            const uint32_t dst = tiles_addr + (uint32_t)((a % NA) * A_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
            const bool live = 2 * a < ksteps && a_live;
            const i32x4 r = rsrc_words(Abase + (int64_t)a * (4 * BK), live ? 0xFFFFFFFFu : 0u);
            dma_16B(r, a_voff[t], dst);
        };
        // nn: B step sb (k-rows 32*sb.. of the pass's group) to slot sb % 4.
        auto dma_b = [&](int sb, int t) __attribute__((always_inline)) {
            const uint32_t dst = tiles_addr + (uint32_t)(B_RING + (sb % NB) * B_STAGE) + (uint32_t)(4 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(W0 + ((int64_t)sb * BK * N + n0) * 2, sb < ksteps ? 0xFFFFFFFFu : 0u);
            dma_16B(r, b_voff[t], dst);
        };
        // nt: B stage b (steps 2b, 2b+1; n-rows n0.., 64 tokens) to slot b % 2.
        auto dma_bt = [&](int b, int t) __attribute__((always_inline)) {
            const uint32_t dst = tiles_addr + (uint32_t)(B_RING + (b % NB) * B_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(W0 + (n0 * K + (int64_t)b * 2 * BK) * 2, 2 * b < ksteps ? 0xFFFFFFFFu : 0u);
            dma_16B(r, bt_voff[t], dst);
        };
        // Loads of step s (also the prologue's virtual steps s < 0), in issue
        // order.  nn (8 per step): B step s+4, then half of an A stage -- the
        // first half of A stage (s+5)/2 for odd s, the second half of A stage
        // (s+4)/2 for even s.  nt: odd s: all of B stage (s+3)/2 (8), then the
        // first half of A stage (s+5)/2 (4); even s: the second half of A stage
        // (s+4)/2 (4).  Every slot written was last read during step s-1 or
        // earlier.
        constexpr int LOADS_ODD = BT ? 12 : 8;
        constexpr int LOADS_EVEN = BT ? 4 : 8;
        auto dma_step = [&](int s, int d) __attribute__((always_inline)) {
            if constexpr (BT) {
                if (s & 1) {
                    if (d < 8) {
                        if ((s + 3) / 2 >= 0) dma_bt((s + 3) / 2, d);
                    } else {
                        dma_a((s + 5) / 2, d - 8);
                    }
                } else {
                    dma_a((s + 4) / 2, d + 4);
                }
            } else {
                if (d < B_LOADS) {
                    if (s + NB >= 0) dma_b(s + NB, d);
                } else if (s & 1) {
                    dma_a((s + 5) / 2, d - B_LOADS);
                } else {
                    dma_a((s + 4) / 2, d);
                }
            }
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        // Fragments of one K step.  nn: B as transposed 4-token halves; nt: B as
        // 16-byte reads like A.
        struct Frags {
            i32x4 a[2][4];
            i16x4 blo[2][4];
            i16x4 bhi[2][4];
            i32x4 bt[2][4];
        };
        // Block read r (0..15) of step s: per ks the four A blocks, then the four
        // B blocks (nn: two transposed halves each).
        constexpr int READS = 16;
        auto read_one = [&](int s, int r, Frags& f) __attribute__((always_inline)) {
            const int ks = r >> 3, q = r & 7;
            if (q < 4) {
                const lds_char* As = tiles + ((s >> 1) % NA) * A_STAGE;
                const uint32_t a_chunk = (uint32_t)(((4 * (s & 1) + 2 * ks + lhi) ^ a_sw) << 4);
                f.a[ks][q] = lds_load_16B(As, a_frag_row + q * 4096u + a_chunk);
            } else if constexpr (BT) {
                const lds_char* Bs = tiles + B_RING + ((s >> 1) % NB) * B_STAGE;
                const uint32_t chunk = (uint32_t)(((4 * (s & 1) + 2 * ks + lhi) ^ a_sw) << 4);
                f.bt[ks][q - 4] = lds_load_16B(Bs, bt_frag_row + (q - 4) * 4096u + chunk);
            } else {
                const lds_char* Bs = tiles + B_RING + (s % NB) * B_STAGE;
                const int j = q - 4;
                f.blo[ks][j] = lds_read_tr16(Bs, b_frag[j] + ks * 8192u);
                f.bhi[ks][j] = lds_read_tr16(Bs, b_frag[j] + ks * 8192u + 2048u);
            }
        };
        auto read_all = [&](int s, Frags& f) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < READS; ++r) read_one(s, r, f);
        };
        auto mfma_one = [&](const Frags& f, int ks, int k) __attribute__((always_inline)) {
            const int j = k >> 2, i = k & 3;
            if constexpr (BT) {
                acc[j][i] = mfma_bf16_32x32x16(f.bt[ks][j], f.a[ks][i], acc[j][i]);
            } else {
                const i16x4 lo = f.blo[ks][j], hi = f.bhi[ks][j];
                const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[j][i] = mfma_bf16_32x32x16(__builtin_bit_cast(i32x4, v), f.a[ks][i], acc[j][i]);
            }
        };

        // The partial vmcnt waits count only this item's direct loads.
        wait_vmcnt<0>();
        // Prologue: virtual steps -5..-1.  nn: as the k-grouped kernel (24 loads
        // after the second half of A stage 0).  nt: A stage 0 (steps -5, -4), B
        // stage 0 with A stage 1's first half (-3), A stage 1's second half (-2),
        // B stage 1 with A stage 2's first half (-1): 20 loads after B stage 0.
        if constexpr (BT) {
#pragma unroll
            for (int v = -5; v < 0; ++v) {
                if (v & 1) {
#pragma unroll
                    for (int d = 0; d < LOADS_ODD; ++d) dma_step(v, d);
                } else {
#pragma unroll
                    for (int d = 0; d < LOADS_EVEN; ++d) dma_step(v, d);
                }
            }
            wait_vmcnt<20>();
        } else {
#pragma unroll
            for (int d = B_LOADS; d < 2 * B_LOADS; ++d) dma_step(-5, d);
#pragma unroll
            for (int v = -4; v < 0; ++v)
#pragma unroll
                for (int d = 0; d < 2 * B_LOADS; ++d) dma_step(v, d);
            wait_vmcnt<6 * B_LOADS>();
        }
        barrier_no_fence();
        Frags f0, f1;
        read_all(0, f0);

        // Step s: a barrier publishes step s+1 once its loads have landed, then
        // 32 MFMAs with the step's loads spread among them and the 16 block reads
        // of step s+1 after MFMAs 16..31, one per MFMA.  nn: as the k-grouped kernel (at most 16 /
        // 20 later loads outstanding for odd / even s).  nt: step s+1 needs, for
        // odd s, B stage (s+1)/2 (issued first in step s-2): 8 later loads may
        // remain; for even s nothing newer than B stage s/2 (step s-3): 20.
        auto body = [&](int s, auto odd_tag, Frags& cur, Frags& nxt) __attribute__((always_inline)) {
            constexpr bool odd = decltype(odd_tag)::value;
            wait_lgkmcnt0();
            if constexpr (BT) {
                if constexpr (odd) wait_vmcnt<8>();
                else wait_vmcnt<20>();
            } else {
                if constexpr (odd) wait_vmcnt<4 * B_LOADS>();
                else wait_vmcnt<5 * B_LOADS>();
            }
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                mfma_one(cur, k >> 4, k & 15);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (BT) {
                    // odd: 12 loads at MFMAs 8q + {0, 2, 5}; even: 4 at MFMAs 8q
                    const int r8 = k & 7;
                    if constexpr (odd) {
                        if (r8 == 0 || r8 == 2 || r8 == 5) dma_step(s, 3 * (k >> 3) + (r8 == 0 ? 0 : (r8 == 2 ? 1 : 2)));
                    } else {
                        if (r8 == 0) dma_step(s, k >> 3);
                    }
                } else {
                    if ((k & 3) == 0) dma_step(s, k >> 2);
                }
                if (k >= 16) read_one(s + 1, k - 16, nxt);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int s = 0; s < ksteps; s += 2) {
            body(s, std::false_type{}, f0, f1);
            body(s + 1, std::true_type{}, f1, f0);
        }
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier_no_fence();
        // each wave stores its own 128 x 128; a half of no group is left as is, and each half
        // of a split tile is stored by its own item
        const bool mine = split ? wm == live_half : (wm ? v1 : v0);
        if (mine)
            store_wave_tile_staged<OUT>(p, 0, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

template <bool BT>
static void launch_layout(const MGroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((mgrouped_bf16_kernel<kOutBf16, BT>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((mgrouped_bf16_kernel<kOutF16, BT>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((mgrouped_bf16_kernel<kOutF32, BT>), dim3(grid), dim3(NT), 0, stream, p);
}

}  // namespace

hipError_t launch_mgrouped_bf16(const MGroupedParams& p, bool nt, int out_kind, int grid, hipStream_t stream) {
    if (nt) launch_layout<true>(p, out_kind, grid, stream);
    else launch_layout<false>(p, out_kind, grid, stream);
    return hipGetLastError();
}

}  // namespace kgw
