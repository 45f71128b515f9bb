// Persistent K-grouped weight-gradient kernel, bf16 operands, fp32 accumulation
// (gfx950), for every operand layout of the cuDNN "Grouped GEMM + WGrad
// (Unified)" page's BF16 contract (A K-major or M-major, B K-major or N-major,
// and the `tensor_ragged` order of per-expert K-contiguous blocks).  For expert e
// with token range [begin, end) from the inclusive cumulative offsets (section
// "Operation"):
//     out[e] (=|+=) A[:, begin:end] @ B[begin:end, :]
//
// Work decomposition: one item per (expert, K chunk, 256x256 output tile).
// Items run expert-major, then K chunk (one unless split-K), then tile, M
// first in columns of p.group_m tiles (four, or eight for short experts: see
// the host's choice); a persistent grid of one workgroup per CU strides over
// them (for long experts, odd rounds take the slots in reverse).  For long
// experts workgroup ids are remapped so each XCD owns a contiguous run of items
// (shared A/B panels in its L2); for short ones the host turns the remap off.  An item whose expert has no tokens
// zero-fills its tile in overwrite mode and does nothing in accumulate mode.
//
// Inside an item (MFMA 32x32x16, fp32 accumulation): 4 waves, each a 128x128
// quarter of the tile computed transposed (a lane ends up holding four
// consecutive N values of one output row), K step 32 tokens.  Operands reach LDS
// through direct global->LDS loads (no register staging); an operand is staged
// one of two ways, by which of its axes is contiguous:
//   TC  tokens contiguous (A K-major, B K-major, ragged blocks): rows of the
//       output axis (m or n), staged 64 tokens at a time so every row moves as
//       one full 128-byte line (half-line rows cost the L2 twice per byte);
//       swizzle 16-byte chunk ^ ((row>>1)&7); fragments are 16-byte LDS reads;
//   TR  rows of tokens (A M-major, B N-major): 32-token stages of 512-byte rows,
//       swizzle chunk ^ 4*(k&3); fragments come from transposing
//       ds_read_b64_tr_b16 (two 4-token halves joined at the MFMA).
// Pairs, rings (LDS) and load schedules (each wave issues eight 1 KiB loads per
// step on average, spread between its MFMAs: a burst of loads from all waves
// queues at the CU's path from L2 and stalls MFMA issue):
//   A TC + B TR (default): A 3 two-step slots, B 4 one-step slots (160 KiB);
//                 step s issues B step s+4, then half of an A stage;
//   A TR + B TR:  4 one-step slots each (128 KiB; with five, the slot arithmetic
//                 modulo 5 pushed the loop past 256 VGPRs); step s issues B and A
//                 step s+4;
//   A TR + B TC:  the default with the operands' roles swapped;
//   A TC + B TC:  A 3 two-step slots, B 2 two-step slots; odd steps issue a
//                 whole B stage (two steps ahead) and half an A stage, even
//                 steps the other half of an A stage.
// One barrier per step publishes step s+1 and frees what step s read; the 16
// block reads of step s+1 follow MFMAs 16..31 of step s, one per MFMA (this
// spacing measured 4% faster than two reads per MFMA for the first eight).  Steps
// past an expert's range load from an empty buffer range, so the loop has no
// branches and uniform vmcnt counts.  The finished tile leaves through the idle
// rings (each wave transposes its accumulators through 32 KiB of LDS so the
// global stores write whole row segments).
// Ragged (A TC + B TC only): expert e's A block is (hidden, n_e) and its B block
// (n, n_e), each row-major, stored back to back from element begin*hidden
// (A) / begin*n (B); only the base and the row stride of the staging change.
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kBf16BM, BN = kBf16BN, BK = kBf16BK;
constexpr int NT = 256;
constexpr int TC_STAGE = 256 * 2 * BK * 2;  // 32 KiB: 256 rows x 128 B (two K steps)
constexpr int TR_STAGE = BK * 256 * 2;      // 16 KiB: 32 token rows x 512 B (one K step)

enum Pair { kTRTR = 0, kTRTC = 1, kTCTC = 2, kTCTR = 3 };

template <int PAIR>
struct Rings {
    static constexpr bool a_tr = PAIR == kTRTR || PAIR == kTRTC;
    static constexpr bool b_tc = PAIR == kTRTC || PAIR == kTCTC;
    static constexpr int na = PAIR == kTRTR ? 4 : (PAIR == kTRTC ? 4 : 3);
    static constexpr int nb = PAIR == kTRTR ? 4 : (PAIR == kTRTC ? 3 : (PAIR == kTCTC ? 2 : 4));
    static constexpr int a_stage = a_tr ? TR_STAGE : TC_STAGE;
    static constexpr int b_stage = b_tc ? TC_STAGE : TR_STAGE;
    static constexpr int b_ring = na * a_stage;
    static constexpr int total = b_ring + nb * b_stage;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int OUT, int PAIR>
__global__ __launch_bounds__(NT, 1) void wgrad_bf16_kernel(GroupedParams p) {
    using R = Rings<PAIR>;
    constexpr bool A_TR = R::a_tr, B_TC = R::b_tc;
    constexpr int NA = R::na, NB = R::nb;
    __shared__ __attribute__((aligned(1024))) char smem[R::total];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;
    const bool ragged = p.ragged != 0;

    // Direct-load slots.  TC: wave instruction t (0..7) fills LDS rows 64*wave +
    // 8*t + (lane>>3), 16-byte slot lane&7 = logical chunk ^ ((row>>1)&7).  TR:
    // instruction t (0..3) fills token rows 8*wave + 2*t + (lane>>5), slot
    // lane&31 = logical chunk ^ 4*(k&3).
    int c_q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) c_q[t] = (lane & 7) ^ ((4 * t + (lane >> 4)) & 7);
    int r_q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) r_q[t] = (lane & 31) ^ (((2 * t + (lane >> 5)) & 3) << 2);

    // Fragment read offsets.  TC: row (half h)*128 + 32i + l32, chunk
    // (4*(s&1) + 2*ks + lhi) ^ sw.  TR: the transposed 4x16 blocks of column
    // block j of half h, chunk XOR 4*(k&3) as written.
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_tc_row = (uint32_t)(wm * 128 + l32) * 128u;
    const uint32_t b_tc_row = (uint32_t)(wn * 128 + l32) * 128u;
    const int c_sw = (l32 >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    uint32_t a_tr_frag[4], b_tr_frag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 8 * (g16 >> 1) + (i16 >> 2);
        const int tail = 2 * (g16 & 1) + ((i16 & 3) >> 1) + 4 * (j ^ (i16 >> 2));
        a_tr_frag[j] = (uint32_t)krow * 512u + (uint32_t)(16 * wm + tail) * 16u + (uint32_t)(i16 & 1) * 8u;
        b_tr_frag[j] = (uint32_t)krow * 512u + (uint32_t)(16 * wn + tail) * 16u + (uint32_t)(i16 & 1) * 8u;
    }

    const int TT = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);

    // Static schedule: round r covers items [r*G, (r+1)*G); with p.snake the slots of odd
    // rounds run in reverse, so a workgroup alternates between the front and the back of
    // consecutive rounds (each XCD still holds a contiguous run of 32 items).
    //
    // Dynamic schedule (p.sched): the same runs of G/nq items per round form nq queues, one
    // per XCD (queue q: the q-th run of every round), claimed one item at a time through
    // the queue's counter; a workgroup drains the queue of its XCD (block id mod nq, the
    // hardware's round-robin placement), then those of the next ones, so every claimed
    // index is unique and every workgroup stops after at most nq empty claims.  Experts
    // run longest first: lane k of every wave holds the expert of rank k (ties by index),
    // so the last items to be claimed are the shortest.  Thread 0 claims the next item
    // while the current one writes its output, and passes it on through LDS word 0 (the
    // rings are idle between items) between two barriers.
    const bool dyn = p.sched != nullptr;
    int perm = lane;
    if (dyn) {
        const int E = p.num_experts;                        // <= kSchedMaxExperts
        int cnt = -1;
        if (lane < E) {
            const int64_t b0 = lane ? (int64_t)p.offsets[lane - 1] : 0, e0 = p.offsets[lane];
            const int64_t b1 = b0 < 0 ? 0 : (b0 > T ? T : b0);
            const int64_t e1 = e0 < 0 ? 0 : (e0 > T ? T : e0);
            cnt = (int)(e1 > b1 ? e1 - b1 : 0);
        }
        int rank = lane;
        if (lane < E) {
            rank = 0;
            for (int j = 0; j < E; ++j) {
                const int cj = __builtin_amdgcn_readlane(cnt, j);
                rank += (cj > cnt || (cj == cnt && j < lane)) ? 1 : 0;
            }
        }
        perm = __builtin_amdgcn_ds_permute(rank << 2, lane);
    }
    const int nq = p.num_xcds, qrun = G / p.num_xcds;
    int q = (int)(blockIdx.x % (unsigned)nq), left = nq;    // thread 0's queue state
    int r = 0;                                              // static: next round
    // thread 0: the item of raw claim `idx` in queue q; an exhausted queue sends it on to
    // the next one (claiming there), -1 once every queue is exhausted
    auto resolve = [&](int idx) -> int {
        for (;;) {
            const int it = (idx / qrun) * G + q * qrun + idx % qrun;
            if (it < p.num_items) return it;
            if (--left == 0) return -1;
            q = q + 1 == nq ? 0 : q + 1;
            idx = atomicAdd(p.sched + q, 1);
        }
    };
    auto broadcast = [&](int v) -> int {
        if (tid == 0) *(__attribute__((address_space(3))) int*)tiles = v;
        barrier_no_fence();
        v = *(__attribute__((address_space(3))) int*)tiles;
        barrier_no_fence();
        return __builtin_amdgcn_readfirstlane(v);
    };
    auto next_static = [&]() -> int {
        while (r * G < p.num_items) {
            const int it = r * G + ((r & 1) && p.snake ? G - 1 - slot : slot);
            ++r;
            if (it < p.num_items) return it;
        }
        return -1;
    };
    int pend = 0;                                           // thread 0: raw claim of the next item
    auto claim_next = [&]() {
        if (dyn && tid == 0) pend = atomicAdd(p.sched + q, 1);
    };
    auto next_item = [&]() -> int {
        if (!dyn) return next_static();
        return broadcast(tid == 0 ? resolve(pend) : 0);
    };
    if (dyn && tid == 0) pend = atomicAdd(p.sched + q, 1);
    for (int item = next_item(); item >= 0; item = next_item()) {
        const int ec = item / TT;
        const int local = item - ec * TT;
        const int e = dyn ? __builtin_amdgcn_readlane(perm, ec) : ec / p.split;   // dynamic: split is 1
        const int c = ec - (dyn ? ec : e * p.split);
        const int eo = c * p.num_experts + e;
        if (p.out_ptrs && !p.out_ptrs[eo]) {
            claim_next();
            continue;
        }
        int tm, tn;
        tile_coords(local, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        const int64_t raw_begin = e ? (int64_t)p.offsets[e - 1] : 0;
        const int64_t raw_end = p.offsets[e];
        const int32_t ebegin = (int32_t)(raw_begin < 0 ? 0 : (raw_begin > T ? T : raw_begin));
        const int32_t eend = max(ebegin, (int32_t)(raw_end < 0 ? 0 : (raw_end > T ? T : raw_end)));
        int32_t begin = ebegin, end = eend;
        if (p.split > 1) {
            const int32_t len = ((end - begin + p.split - 1) / p.split + kSplitUnit - 1) & ~(kSplitUnit - 1);
            const int32_t cb = (int32_t)min<int64_t>(end, (int64_t)begin + (int64_t)c * len);
            end = (int32_t)min<int64_t>(end, (int64_t)cb + len);
            begin = cb;
        }
        // Whole 64-token units; ragged blocks are counted from their own start, so
        // the loads stay inside the expert's block even for malformed offsets.
        if (ragged) begin = ebegin + ((begin - ebegin) & ~(2 * BK - 1));
        else begin &= ~(2 * BK - 1);
        const int ksteps = ((end - begin) / (2 * BK)) * 2;
        if (ksteps == 0) {
            claim_next();
            if (!p.accumulate) zero_slab_part<OUT, NT>(p, eo, local, TT, tid);
            continue;
        }
        const int rows_valid = (int)min<int64_t>(BM, H - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);

        // Operand bases (bytes) at token `begin`, and row strides (elements).
        //   A TC: rows m, stride T (2-D) or n_e (ragged: expert block (H, n_e) from begin*H);
        //   A TR: token rows, stride H;   B TR: token rows, stride N;
        //   B TC: rows n, stride T (2-D) or n_e (ragged block (N, n_e) from begin*N).
        const int64_t ne = (int64_t)eend - ebegin;
        int64_t a_stride, b_stride;
        const char* Abase;
        const char* Bbase;
        if constexpr (A_TR) {
            a_stride = H;
            Abase = (const char*)p.A + ((int64_t)begin * H + m0) * 2;
        } else {
            a_stride = ragged ? ne : T;
            Abase = (const char*)p.A + (ragged ? ((int64_t)ebegin * H + m0 * ne + (begin - ebegin))
                                               : (m0 * T + begin)) * 2;
        }
        if constexpr (B_TC) {
            b_stride = ragged ? ne : T;
            Bbase = (const char*)p.B + (ragged ? ((int64_t)ebegin * N + n0 * ne + (begin - ebegin))
                                               : (n0 * T + begin)) * 2;
        } else {
            b_stride = N;
            Bbase = (const char*)p.B + ((int64_t)begin * N + n0) * 2;
        }
        // Per-lane byte offsets inside a stage (rows past the valid extent are
        // clamped onto the last valid one: they only feed outputs never stored).
        uint32_t a_voff[8], b_voff[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (A_TR) {
                if (t < 4) {
                    const int krow = 8 * wave + 2 * t + (lane >> 5);
                    a_voff[t] = (uint32_t)krow * (uint32_t)(a_stride * 2) +
                                (uint32_t)min(8 * r_q[t], rows_valid - 8) * 2u;
                }
            } else {
                const int row = min(64 * wave + 8 * t + (lane >> 3), rows_valid - 1);
                a_voff[t] = (uint32_t)row * (uint32_t)(a_stride * 2) + (uint32_t)c_q[t] * 16u;
            }
            if constexpr (B_TC) {
                const int row = min(64 * wave + 8 * t + (lane >> 3), cols_valid - 1);
                b_voff[t] = (uint32_t)row * (uint32_t)(b_stride * 2) + (uint32_t)c_q[t] * 16u;
            } else {
                if (t < 4) {
                    const int krow = 8 * wave + 2 * t + (lane >> 5);
                    b_voff[t] = (uint32_t)krow * (uint32_t)(b_stride * 2) +
                                (uint32_t)min(8 * r_q[t], cols_valid - 8) * 2u;
                }
            }
        }

        // TC stage x (steps 2x, 2x+1) / TR step x of each operand; stages past the
        // range use an empty buffer range (no traffic, uniform vmcnt counts).
        auto dma_a = [&](int x, int t) __attribute__((always_inline)) {
            const uint32_t dst = tiles_addr + (uint32_t)((x % NA) * R::a_stage) +
                                 (uint32_t)((A_TR ? 4 : 8) * wave + t) * 1024u;
            const int64_t step_bytes = A_TR ? (int64_t)BK * a_stride * 2 : 4 * BK;
            const bool live = A_TR ? x < ksteps : 2 * x < ksteps;
            dma_16B(rsrc_words(Abase + (int64_t)x * step_bytes, live ? 0xFFFFFFFFu : 0u), a_voff[t], dst);
        };
        auto dma_b = [&](int x, int t) __attribute__((always_inline)) {
            const uint32_t dst = tiles_addr + (uint32_t)(R::b_ring + (x % NB) * R::b_stage) +
                                 (uint32_t)((B_TC ? 8 : 4) * wave + t) * 1024u;
            const int64_t step_bytes = B_TC ? 4 * BK : (int64_t)BK * b_stride * 2;
            const bool live = B_TC ? 2 * x < ksteps : x < ksteps;
            dma_16B(rsrc_words(Bbase + (int64_t)x * step_bytes, live ? 0xFFFFFFFFu : 0u), b_voff[t], dst);
        };
        // Loads of step s (also the prologue's virtual steps s < 0), in issue order.
        constexpr int LOADS_ODD = PAIR == kTCTC ? 12 : 8;
        constexpr int LOADS_EVEN = PAIR == kTCTC ? 4 : 8;
        auto dma_step = [&](int s, int d) __attribute__((always_inline)) {
            if constexpr (PAIR == kTRTR) {
                if (s + 4 >= 0) {
                    if (d < 4) dma_b(s + 4, d);
                    else dma_a(s + 4, d - 4);
                }
            } else if constexpr (PAIR == kTRTC) {
                if (d < 4) {
                    if (s + 4 >= 0) dma_a(s + 4, d);
                } else if (s & 1) {
                    dma_b((s + 5) / 2, d - 4);
                } else {
                    dma_b((s + 4) / 2, d);
                }
            } else if constexpr (PAIR == kTCTR) {
                if (d < 4) {
                    if (s + 4 >= 0) dma_b(s + 4, d);
                } else if (s & 1) {
                    dma_a((s + 5) / 2, d - 4);
                } else {
                    dma_a((s + 4) / 2, d);
                }
            } else {
                if (s & 1) {
                    if (d < 8) {
                        if ((s + 3) / 2 >= 0) dma_b((s + 3) / 2, d);
                    } else {
                        dma_a((s + 5) / 2, d - 8);
                    }
                } else {
                    dma_a((s + 4) / 2, d + 4);
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

        // One K step's operands: 4 M blocks (A) and 4 N blocks (B) per sub-step ks;
        // a TR block is kept as its two transposed 4-token halves and joined into
        // one operand only at its MFMA (joining at read time doubles the live
        // registers of every block in flight).
        struct Frags {
            i32x4 a[2][4];
            i16x4 alo[2][4], ahi[2][4];
            i32x4 b[2][4];
            i16x4 blo[2][4], bhi[2][4];
        };
        // Reads of one block of an operand: TC one 16-byte read, TR two
        // transposing reads (4 tokens each).
        auto read_a = [&](int s, int ks, int i, Frags& f) __attribute__((always_inline)) {
            if constexpr (A_TR) {
                const lds_char* S = tiles + (s % NA) * R::a_stage;
                f.alo[ks][i] = lds_read_tr16(S, a_tr_frag[i] + ks * 8192u);
                f.ahi[ks][i] = lds_read_tr16(S, a_tr_frag[i] + ks * 8192u + 2048u);
            } else {
                const lds_char* S = tiles + ((s >> 1) % NA) * R::a_stage;
                const uint32_t chunk = (uint32_t)(((4 * (s & 1) + 2 * ks + lhi) ^ c_sw) << 4);
                f.a[ks][i] = lds_load_16B(S, a_tc_row + i * 4096u + chunk);
            }
        };
        auto read_b = [&](int s, int ks, int j, Frags& f) __attribute__((always_inline)) {
            if constexpr (B_TC) {
                const lds_char* S = tiles + R::b_ring + ((s >> 1) % NB) * R::b_stage;
                const uint32_t chunk = (uint32_t)(((4 * (s & 1) + 2 * ks + lhi) ^ c_sw) << 4);
                f.b[ks][j] = lds_load_16B(S, b_tc_row + j * 4096u + chunk);
            } else {
                const lds_char* S = tiles + R::b_ring + (s % NB) * R::b_stage;
                f.blo[ks][j] = lds_read_tr16(S, b_tr_frag[j] + ks * 8192u);
                f.bhi[ks][j] = lds_read_tr16(S, b_tr_frag[j] + ks * 8192u + 2048u);
            }
        };
        // Block read r (0..15) of step s: per ks, the four A blocks then the four B blocks.
        auto read_one = [&](int s, int r, Frags& f) __attribute__((always_inline)) {
            const int ks = r >> 3, q = r & 7;
            if (q < 4) read_a(s, ks, q, f);
            else read_b(s, ks, q - 4, f);
        };
        auto join = [](i16x4 lo, i16x4 hi) __attribute__((always_inline)) {
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(i32x4, v);
        };
        auto mfma_one = [&](const Frags& f, int ks, int k) __attribute__((always_inline)) {
            const int j = k >> 2, i = k & 3;
            const i32x4 av = A_TR ? join(f.alo[ks][i], f.ahi[ks][i]) : f.a[ks][i];
            const i32x4 bv = B_TC ? f.b[ks][j] : join(f.blo[ks][j], f.bhi[ks][j]);
            acc[j][i] = mfma_bf16_32x32x16(bv, av, acc[j][i]);
        };

        wait_vmcnt<0>();
        // Prologue: virtual steps -5..-1, then wait for step 0's operands:
        //   TR+TR: steps 0..3 issued, step 0 first: 24 later loads may remain;
        //   TR+TC: as the default kernel mirrored (A steps 0..3, B stages 0-1 and the
        //          first half of 2): 24 after the second half of B stage 0;
        //   TC+TC: A stage 0 (-5, -4), B stage 0 and half of A stage 1 (-3), the rest
        //          of A stage 1 (-2), B stage 1 and half of A stage 2 (-1): 20 after B 0.
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
        if constexpr (PAIR == kTCTC) wait_vmcnt<20>();
        else wait_vmcnt<24>();
        barrier_no_fence();
        Frags f0, f1;
#pragma unroll
        for (int r = 0; r < 16; ++r) read_one(0, r, f0);

        // Step s: a barrier publishes step s+1 once its loads have landed (at most
        // this many later loads outstanding: TR+TR 16; TR+TC 16 odd / 20 even; TC+TC
        // 8 odd / 20 even), then 32 MFMAs with the step's loads spread among them
        // and the 16 block reads of step s+1 after the 16th MFMA.
        auto body = [&](int s, auto odd_tag, Frags& cur, Frags& nxt) __attribute__((always_inline)) {
            constexpr bool odd = decltype(odd_tag)::value;
            wait_lgkmcnt0();
            if constexpr (PAIR == kTRTR) wait_vmcnt<16>();
            else if constexpr (PAIR == kTRTC || PAIR == kTCTR) {
                if constexpr (odd) wait_vmcnt<16>();
                else wait_vmcnt<20>();
            } else {
                if constexpr (odd) wait_vmcnt<8>();
                else wait_vmcnt<20>();
            }
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                mfma_one(cur, k >> 4, k & 15);
                __builtin_amdgcn_sched_barrier(0);
                const int r8 = k & 7;
                if constexpr (PAIR == kTCTC) {
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
        claim_next();
        store_wave_tile_staged<OUT>(p, eo, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

template <int PAIR>
static void launch_pair(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((wgrad_bf16_kernel<kOutBf16, PAIR>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((wgrad_bf16_kernel<kOutF16, PAIR>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((wgrad_bf16_kernel<kOutF32, PAIR>), dim3(grid), dim3(NT), 0, stream, p);
}

}  // namespace

hipError_t launch_wgrad_bf16(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    launch_pair<kTCTR>(p, out_kind, grid, stream);
    return hipGetLastError();
}

hipError_t launch_wgrad_bf16_layout(const GroupedParams& p, bool a_m_major, bool b_k_major, int out_kind, int grid,
                                    hipStream_t stream) {
    if (a_m_major && !b_k_major) launch_pair<kTRTR>(p, out_kind, grid, stream);
    else if (a_m_major) launch_pair<kTRTC>(p, out_kind, grid, stream);
    else if (b_k_major) launch_pair<kTCTC>(p, out_kind, grid, stream);
    else launch_pair<kTCTR>(p, out_kind, grid, stream);
    return hipGetLastError();
}

}  // namespace kgw
