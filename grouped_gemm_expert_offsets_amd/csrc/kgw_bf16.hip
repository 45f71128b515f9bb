// Persistent K-grouped weight-gradient kernel, bf16 operands, fp32 accumulation (gfx950).
//
// Computes, for every expert e with token range [begin, end) taken from the
// inclusive cumulative offsets (cuDNN "Grouped GEMM + WGrad (Unified)",
// section "Operation"):
//     out[e] (=|+=) A[:, begin:end] @ B[begin:end, :]
//
// Work decomposition: one work item per (expert, 256x256 output tile).  Items
// are laid out expert-major; inside an expert, tiles walk M first in columns
// of four tiles.  A persistent grid of one workgroup per CU strides over the
// items; workgroup ids are remapped so that each XCD owns a contiguous run of
// items (shared A/B panels in its L2).  An item whose expert has no tokens
// zero-fills its tile in overwrite mode and does nothing in accumulate mode
// (section "Operation": an empty expert produces zero when overwriting).
//
// Inside an item (MFMA 32x32x16, fp32 accumulation as the page's BF16 contract
// requires):
//   - 4 waves, each owning a 128 (M) x 128 (N) quarter of the tile; the MFMA
//     computes the transposed block Wgrad^T so that every lane ends up holding
//     four consecutive N values of one output row (16-byte stores);
//   - K step of 32 tokens.  Operands reach LDS through direct global->LDS
//     loads (no register staging): A in three 64-token stages (each A row
//     then moves as one full 128-byte line; half-line rows cost the L2 twice
//     per byte) and B in four 32-token stages, so loads run up to four
//     steps ahead.  The rings take all 160 KiB of LDS; the
//     per-expert token ranges come from scalar loads of the offsets.
//     The fragments of step s+1 are read from LDS while the second half of
//     step s's MFMAs runs, so the MFMAs never wait on LDS latency; one
//     barrier per step both publishes the next stage and frees the stage
//     just consumed.  Each wave issues eight 1 KiB loads per step, one after
//     every fourth MFMA: the CU's path from L2 moves about 60 B per clock,
//     and a burst of loads from all four waves at once queues there and
//     stalls their MFMA issue (one wave per SIMD has no other wave to cover
//     the stall);
//   - the XOR swizzles live on the global-address side: each lane of a direct
//     load fetches the chunk that belongs at its LDS slot.  A rows (128 B):
//     16-byte chunk ^ ((row>>1)&7); B rows (512 B): chunk ^ 4*(k&3).  Both keep
//     the fragment reads free of bank conflicts;
//   - A is token-contiguous, so its fragments are plain 16-byte LDS reads; B is
//     N-contiguous, so its fragments come from transposing ds_read_b64_tr_b16;
//   - the finished tile leaves through the (then idle) ring: each wave
//     transposes its accumulators through 32 KiB of LDS so that the global
//     stores write whole row segments.
#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kBf16BM, BN = kBf16BN, BK = kBf16BK;
constexpr int NT = 256;
// A is staged 64 tokens (two K steps) at a time, so every A row moves as one
// full 128-byte line; B is staged one 32-token step at a time.
constexpr int NA = 3;                       // A ring: 3 stages of 2 K steps
constexpr int NB = 4;                       // B ring: 4 stages of 1 K step
constexpr int A_STAGE = BM * 2 * BK * 2;    // 32 KiB: 256 rows x 128 B
constexpr int B_STAGE = BK * BN * 2;        // 16 KiB: 32 rows x 512 B
constexpr int B_RING = NA * A_STAGE;        // byte offset of the B ring
constexpr int LDS_TILES = NA * A_STAGE + NB * B_STAGE;  // 160 KiB: all of the CU's LDS
constexpr int GROUP_M = 4;
constexpr int A_LOADS = 8;                  // direct loads per wave per A stage
constexpr int B_LOADS = 4;                  // direct loads per wave per B stage

static_assert(BM == 256 && BN == 256 && BK == 32, "index math below assumes 256x256x32");

template <int OUT>
__global__ __launch_bounds__(NT, 1) void wgrad_bf16_kernel(GroupedParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TILES];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;

    // Direct-load slots of this lane.  A: wave instruction t (0..7) fills LDS
    // rows 64*wave + 8*t + (lane>>3), 16-byte slot lane&7, which holds logical
    // chunk (lane&7) ^ ((row>>1)&7).  B: instruction t (0..3) fills k-rows
    // 8*wave + 2*t + (lane>>5), slot lane&31 = logical chunk slot ^ 4*(k&3).
    int a_q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) a_q[t] = (lane & 7) ^ ((4 * t + (lane >> 4)) & 7);
    int b_q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b_q[t] = (lane & 31) ^ (((2 * t + (lane >> 5)) & 3) << 2);

    // Fragment read offsets (fixed per lane).
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u;
    const int a_sw = (l32 >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    uint32_t b_frag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 8 * (g16 >> 1) + (i16 >> 2);
        const int chunk = 16 * wn + 2 * (g16 & 1) + ((i16 & 3) >> 1) + 4 * (j ^ (i16 >> 2));
        b_frag[j] = (uint32_t)krow * 512u + (uint32_t)chunk * 16u + (uint32_t)(i16 & 1) * 8u;
    }

    const int TT = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);

    for (int item = slot; item < p.num_items; item += G) {
        // Items run expert-major, then K chunk (one unless the K range is split),
        // then tile; chunk c of expert e writes output slab c*E + e (the split-K
        // partials; slab e itself when unsplit).
        const int ec = item / TT;
        const int local = item - ec * TT;
        const int e = ec / p.split;
        const int c = ec - e * p.split;
        const int eo = c * p.num_experts + e;
        if (p.out_ptrs && !p.out_ptrs[eo]) continue;     // the caller wants no output for this expert
        int tm, tn;
        tile_coords(local, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        // Token range, clamped into [0, tokens_sum] (uniform: scalar loads of the
        // offsets, which stay hot in L2; the LDS is all taken by the rings).
        const int64_t raw_begin = e ? (int64_t)p.offsets[e - 1] : 0;
        const int64_t raw_end = p.offsets[e];
        int32_t begin = (int32_t)(raw_begin < 0 ? 0 : (raw_begin > T ? T : raw_begin));
        int32_t end = max(begin, (int32_t)(raw_end < 0 ? 0 : (raw_end > T ? T : raw_end)));
        if (p.split > 1) {
            // chunk c of the range: split_unit-aligned pieces of ceil(count / split)
            const int32_t len = ((end - begin + p.split - 1) / p.split + kSplitUnit - 1) & ~(kSplitUnit - 1);
            const int32_t cb = (int32_t)min<int64_t>(end, (int64_t)begin + (int64_t)c * len);
            end = (int32_t)min<int64_t>(end, (int64_t)cb + len);
            begin = cb;
        }
        // The loop below takes K steps in pairs: a range is used in whole
        // 64-token units (every well-formed count is a multiple of 256).
        begin &= ~(2 * BK - 1);
        const int ksteps = ((end - begin) / (2 * BK)) * 2;
        if (ksteps == 0) {
            if (!p.accumulate) zero_tile<OUT, BM, BN, NT>(p, eo, m0, n0, tid);
            continue;
        }

        const char* Abase = (const char*)p.A + (m0 * T + begin) * 2;
        const char* Bbase = (const char*)p.B + ((int64_t)begin * N + n0) * 2;
        const int rows_valid = (int)min<int64_t>(BM, H - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        uint32_t a_voff[8], b_voff[4];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = min(64 * wave + 8 * t + (lane >> 3), rows_valid - 1);
            a_voff[t] = (uint32_t)row * (uint32_t)(T * 2) + (uint32_t)a_q[t] * 16u;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int krow = 8 * wave + 2 * t + (lane >> 5);
            b_voff[t] = (uint32_t)krow * (uint32_t)(N * 2) + (uint32_t)min(8 * b_q[t], cols_valid - 8) * 2u;
        }

        // Direct loads.  A stage a (steps 2a, 2a+1) goes to A slot a % NA in two
        // halves of four loads per wave, B step s to B slot s % NB.  Stages past
        // the expert's range use an empty buffer range: the loads fetch nothing
        // (the slot is never read by an MFMA), which keeps the loop below free of
        // branches and its vmcnt counts uniform.
        auto dma_a = [&](int a, int t) {
            const uint32_t dst = tiles_addr + (uint32_t)((a % NA) * A_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(Abase + (int64_t)a * (4 * BK), 2 * a < ksteps ? 0xFFFFFFFFu : 0u);
            dma_16B(r, a_voff[t], dst);
        };
        auto dma_b = [&](int sb, int t) {
            const uint32_t dst = tiles_addr + (uint32_t)(B_RING + (sb % NB) * B_STAGE) + (uint32_t)(4 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(Bbase + (int64_t)sb * BK * N * 2, sb < ksteps ? 0xFFFFFFFFu : 0u);
            dma_16B(r, b_voff[t], dst);
        };
        // The loads of step s (also for the prologue's virtual steps s < 0), in
        // issue order: B step s+4, then half of an A stage -- for odd s the first
        // half of A stage (s+5)/2, for even s the second half of A stage (s+4)/2.
        // Every slot written this way was last read by the fragment reads made
        // during step s-1 or earlier.
        auto dma_step = [&](int s, int d) {
            if (d < B_LOADS) {
                if (s + NB >= 0) dma_b(s + NB, d);
            } else if (s & 1) {
                dma_a((s + 5) / 2, d - B_LOADS);
            } else {
                dma_a((s + 4) / 2, d);
            }
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        // Fragments of one K step: A[ks][i] (M blocks); B[ks][j] (N blocks) as the
        // two transposed 4-token halves that form one MFMA operand.
        struct Frags {
            i32x4 a[2][4];
            i16x4 blo[2][4];
            i16x4 bhi[2][4];
        };
        // Fragment read number r (0..23) of step s: per k sub-step ks, the four
        // A blocks then the eight transposed B halves.
        auto read_one = [&](int s, int r, Frags& f) {
            const int ks = r / 12, q = r % 12;
            if (q < 4) {
                const lds_char* As = tiles + ((s >> 1) % NA) * A_STAGE;
                const uint32_t a_chunk = (uint32_t)(((4 * (s & 1) + 2 * ks + lhi) ^ a_sw) << 4);
                f.a[ks][q] = lds_load_16B(As, a_frag_row + q * 4096u + a_chunk);
            } else {
                const lds_char* Bs = tiles + B_RING + (s % NB) * B_STAGE;
                const int j = (q - 4) >> 1, hi = (q - 4) & 1;
                const i16x4 v = lds_read_tr16(Bs, b_frag[j] + ks * 8192u + hi * 2048u);
                if (hi) f.bhi[ks][j] = v;
                else f.blo[ks][j] = v;
            }
        };
        auto read_all = [&](int s, Frags& f) {
#pragma unroll
            for (int r = 0; r < 24; ++r) read_one(s, r, f);
        };
        // MFMA number k (0..15) of sub-step ks: N block k/4 times M block k%4.
        auto mfma_one = [&](const Frags& f, int ks, int k) {
            const int j = k >> 2, i = k & 3;
            const i16x4 lo = f.blo[ks][j], hi = f.bhi[ks][j];
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[j][i] = mfma_bf16_32x32x16(__builtin_bit_cast(i32x4, v), f.a[ks][i], acc[j][i]);
        };
        // The partial vmcnt waits count only this item's direct loads, so the
        // previous item's output stores must have drained first.
        wait_vmcnt<0>();
        // Prologue: the loads of virtual steps -5..-1 (A0 B0 A0' B1 A1 B2 A1' B3
        // A2).  Step 0's fragments need A stage 0 and B step 0; 24 loads were
        // issued after the second half of A stage 0.
#pragma unroll
        for (int d = B_LOADS; d < 2 * B_LOADS; ++d) dma_step(-5, d);
#pragma unroll
        for (int v = -4; v < 0; ++v)
#pragma unroll
            for (int d = 0; d < 2 * B_LOADS; ++d) dma_step(v, d);
        wait_vmcnt<6 * B_LOADS>();
        barrier_no_fence();
        Frags f0, f1;
        read_all(0, f0);

        // Step s with its fragments in `cur`:
        //   once this wave's reads of step s and its loads of step s+1 are done,
        //   a barrier publishes step s+1 and certifies that every wave is done
        //   reading step s;
        //   32 MFMAs, every fourth one followed by one of the step's eight direct
        //   loads (spread out so that the four waves do not queue their loads at
        //   the memory unit at once, which would stall their MFMA issue), and the
        //   last 16 followed by the 24 fragment reads of step s+1 (so the LDS
        //   latency hides behind MFMAs).
        // Step s+1 needs B step s+1 (issued during step s-3, first of its eight
        // loads) and, for odd s, A stage (s+1)/2 (second half issued during step
        // s-3, last of its loads): at most 20 (even s) or 16 (odd s) later loads
        // may remain outstanding.  sched_barrier(0) pins this interleaving; the
        // compiler would otherwise cluster the memory operations.
        auto body = [&](int s, bool odd, Frags& cur, Frags& nxt) {
            wait_lgkmcnt0();
            if (odd) wait_vmcnt<4 * B_LOADS>();
            else wait_vmcnt<5 * B_LOADS>();
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                mfma_one(cur, k >> 4, k & 15);
                __builtin_amdgcn_sched_barrier(0);
                if ((k & 3) == 0) dma_step(s, k >> 2);
                if (k >= 16) {
                    const int q = k - 16;
                    if (q < 8) {
                        read_one(s + 1, 2 * q, nxt);
                        read_one(s + 1, 2 * q + 1, nxt);
                    } else {
                        read_one(s + 1, 8 + q, nxt);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int s = 0; s < ksteps; s += 2) {
            body(s, false, f0, f1);
            body(s + 1, true, f1, f0);
        }
        // The ring becomes the output staging area: every wave must be done
        // reading it and every direct load (the empty ones past the range
        // included) must have landed.
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier_no_fence();
        store_wave_tile_staged<OUT>(p, eo, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        // The next item's direct loads overwrite the staging areas.
        barrier_no_fence();
    }
}

}  // namespace

hipError_t launch_wgrad_bf16(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL(wgrad_bf16_kernel<kOutBf16>, dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL(wgrad_bf16_kernel<kOutF16>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(wgrad_bf16_kernel<kOutF32>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kgw
