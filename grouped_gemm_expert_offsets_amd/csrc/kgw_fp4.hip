// Persistent K-grouped weight-gradient kernel, FP4 (OCP e2m1) operands with one
// UE8M0 scale per 32 tokens, on the native scaled MFMA (gfx950).
//
// Same operation and work decomposition as the bf16 and fp8 kernels (cuDNN
// "Grouped GEMM + WGrad (Unified)", section "Operation"); the operands are the
// DeepGEMM k-grouped page's FP4 cast with gran_k = 32: e2m1 values, two tokens
// per byte (the even token in the low nibble), both operands keeping the token
// axis contiguous (A (hidden, T/2 bytes), B (n, T/2 bytes)), and one UE8M0 scale
// per 32 tokens packed four to a word (one word per row per 128 tokens).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both formats e2m1 takes 16 bytes per
// lane and operand: lane half h holds K 32h .. 32h+31 (32 consecutive tokens),
// and the scale of lanes 0-31 covers K 0-31, that of lanes 32-63 K 32-63 (probed
// on the GPU).  So each lane's fragment is exactly one 32-token scale block and
// the lane passes that block's byte.  Every product of two e2m1 values times
// their scales is exact, and the products of one 32-token block span at most
// 2^8, well inside the ~13 bits the instruction keeps below a group's largest
// product: each block sum is exact and the only rounding is the fp32
// accumulation across blocks.
//
// Pipeline: K step 64 tokens (16 MFMAs per wave; 4 waves, each 128x128 of the
// 256x256 tile).  A and B move in 256-token stages (256 rows x 128 B: one full
// 128-byte line per row) through 2-slot rings, their scale words through a
// 2-slot scale ring; a stage covers four steps.  Stage y's 24 loads per wave
// (8 A, 8 B, 4 + 4 scale words) are issued in steps 4y-5, 4y-4 and 4y-3, eight
// each, spread between the MFMAs, so they have two to four steps to land (two
// steps of twelve measured 2% slower, four of six 2% slower again).  When the
// scale rows allow 16-byte loads (hidden and n multiples of 4, 16-byte aligned
// scale arrays) the scale words take one load per operand instead of four
// (18 loads: A and B, A and B, then the two scale loads).  Slots only
// change at stage boundaries, so the only barrier is at the start of each
// stage's last step: it publishes the next stage (after all its loads have
// landed) and certifies that the stage before has been read.  The fragments
// of step s+1 are read during the second half of step s.
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int KS = 64;                      // tokens per K step
constexpr int STAGE_TOKENS = 256;           // tokens per stage (4 steps)
constexpr int NT = 256;
constexpr int ROW_BYTES = STAGE_TOKENS / 2; // 128 B per row and stage
constexpr int A_STAGE = BM * ROW_BYTES;     // 32 KiB
constexpr int B_STAGE = BN * ROW_BYTES;     // 32 KiB
constexpr int NSLOT = 2;
constexpr int B_RING = NSLOT * A_STAGE;
constexpr int SC_WAVE = 2048;               // per wave and stage: 2 x 128 sa words, 2 x 128 sb words
constexpr int SC_STAGE = 4 * SC_WAVE;       // 8 KiB
constexpr int SC_RING = B_RING + NSLOT * B_STAGE;
constexpr int LDS_TOTAL = SC_RING + NSLOT * SC_STAGE;   // 144 KiB
constexpr int GROUP_M = 4;

static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
static_assert(4 * 32768 <= SC_RING, "output staging must fit below the scale ring");

// e2m1 x e2m1 -> f32, scale byte 0 of sa/sb per lane (the instruction reads four
// dwords per operand for e2m1; the upper half of the 8-dword argument is unused).
__device__ __forceinline__ f32x16 mfma_scale_e2m1_32x32x64(i32x4 a, i32x4 b, f32x16 c, int sa, int sb) {
    const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// SC16: scale words by 16-byte loads (the host checks hidden % 4 == 0, n % 4 == 0 and
// 16-byte aligned scale arrays), else by dword loads.
template <int OUT, bool SC16>
__global__ __launch_bounds__(NT, 1) void wgrad_fp4_kernel(GroupedParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;
    const int64_t RB = T / 2;               // bytes per operand row

    // Direct-load slots: wave instruction t (0..7) fills stage rows 64*wave + 8*t
    // + (lane>>3), 16-byte slot lane&7 = logical chunk ^ ((row>>1)&7).
    int c_q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) c_q[t] = (lane & 7) ^ ((4 * t + (lane >> 4)) & 7);
    // Fragment reads: row (half)*128 + 32i + l32, logical chunk 2*(step in stage) + lhi.
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_row = (uint32_t)(wm * 128 + l32) * (uint32_t)ROW_BYTES;
    const uint32_t b_row = (uint32_t)(wn * 128 + l32) * (uint32_t)ROW_BYTES;
    const int c_sw = (l32 >> 1) & 7;
    // Scale words of this wave: sa word w of row r at 4*(128w + r), sb at 1024 + 4*(128w + c).
    const uint32_t sc_wave = (uint32_t)(SC_RING + wave * SC_WAVE);

    const int TT = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);

    for (int item = slot; item < p.num_items; item += G) {
        const int ec = item / TT;
        const int local = item - ec * TT;
        const int e = ec / p.split;
        const int c = ec - e * p.split;
        const int eo = c * p.num_experts + e;
        if (p.out_ptrs && !p.out_ptrs[eo]) continue;
        int tm, tn;
        tile_coords(local, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        const int64_t raw_begin = e ? (int64_t)p.offsets[e - 1] : 0;
        const int64_t raw_end = p.offsets[e];
        int32_t begin = (int32_t)(raw_begin < 0 ? 0 : (raw_begin > T ? T : raw_begin));
        int32_t end = max(begin, (int32_t)(raw_end < 0 ? 0 : (raw_end > T ? T : raw_end)));
        if (p.split > 1) {
            const int32_t len = ((end - begin + p.split - 1) / p.split + kSplitUnit - 1) & ~(kSplitUnit - 1);
            const int32_t cb = (int32_t)min<int64_t>(end, (int64_t)begin + (int64_t)c * len);
            end = (int32_t)min<int64_t>(end, (int64_t)cb + len);
            begin = cb;
        }
        begin &= ~(STAGE_TOKENS - 1);
        const int nstages = (end - begin) / STAGE_TOKENS;
        const int ksteps = 4 * nstages;
        if (ksteps == 0) {
            if (!p.accumulate) zero_tile<OUT, BM, BN, NT>(p, eo, m0, n0, tid);
            continue;
        }
        const int rows_valid = (int)min<int64_t>(BM, H - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        const uint8_t* Abase = (const uint8_t*)p.A + m0 * RB + begin / 2;
        const uint8_t* Bbase = (const uint8_t*)p.B + n0 * RB + begin / 2;
        uint32_t a_voff[8], b_voff[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int r = 64 * wave + 8 * t + (lane >> 3);
            a_voff[t] = (uint32_t)min(r, rows_valid - 1) * (uint32_t)RB + (uint32_t)c_q[t] * 16u;
            b_voff[t] = (uint32_t)min(r, cols_valid - 1) * (uint32_t)RB + (uint32_t)c_q[t] * 16u;
        }
        const int64_t gb0 = begin / 128;               // first 128-token scale word of the range
        const uint32_t sa_voff = (uint32_t)(m0 + wm * 128 + lane) * 4u;
        const uint32_t sb_voff = (uint32_t)(n0 + wn * 128 + lane) * 4u;
        // 16-byte form: lane L fetches rows 4(L&31) .. +3 of word L>>5 (the stage's two words)
        const uint32_t sa16_voff = (uint32_t)((int64_t)(lane >> 5) * H + m0 + wm * 128 + 4 * (lane & 31)) * 4u;
        const uint32_t sb16_voff = (uint32_t)((int64_t)(lane >> 5) * N + n0 + wn * 128 + 4 * (lane & 31)) * 4u;

        // Half `hf` (0, 1) of stage y's loads: A and B loads 4hf..4hf+3, then the
        // scale words w = hf of both halves of this wave's rows and columns.
        auto dma_half = [&](int y, int hf, int d) __attribute__((always_inline)) {
            const int sl = y & 1;
            const bool live = y < nstages;
            if (d < 4) {
                const int t = 4 * hf + d;
                const uint32_t dst = tiles_addr + (uint32_t)(sl * A_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
                dma_16B(rsrc_words(Abase + (int64_t)y * ROW_BYTES, live ? 0xFFFFFFFFu : 0u), a_voff[t], dst);
            } else if (d < 8) {
                const int t = 4 * hf + d - 4;
                const uint32_t dst = tiles_addr + (uint32_t)(B_RING + sl * B_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
                dma_16B(rsrc_words(Bbase + (int64_t)y * ROW_BYTES, live ? 0xFFFFFFFFu : 0u), b_voff[t], dst);
            } else {
                const int q = d - 8;                  // 0, 1: sa rows h = q; 2, 3: sb columns h = q - 2
                const bool bs = q >= 2;
                const int h = q & 1;
                const int64_t word = gb0 + 2 * y + hf;
                const int64_t mn = bs ? N : H;
                const uint8_t* base = (bs ? p.sfb : p.sfa) + word * mn * 4;
                const uint32_t dst = tiles_addr + sc_wave + (uint32_t)(sl * SC_STAGE) + (bs ? 1024u : 0u) +
                                     (uint32_t)(128 * hf + 64 * h) * 4u;
                dma_4B(rsrc_words(base, live ? (uint32_t)(mn * 4) : 0u), (bs ? sb_voff : sa_voff) + (uint32_t)h * 256u,
                       dst);
            }
        };
        // Both scale words of stage y for this wave's rows (q 0) or columns (q 1) in one 16-byte
        // load per lane; they land where the dword loads of dma_half put them.
        auto dma_scales16 = [&](int y, int q) __attribute__((always_inline)) {
            const bool bs = q == 1;
            const int64_t mn = bs ? N : H;
            const uint8_t* base = (bs ? p.sfb : p.sfa) + (gb0 + 2 * y) * mn * 4;
            const uint32_t dst = tiles_addr + sc_wave + (uint32_t)((y & 1) * SC_STAGE) + (bs ? 1024u : 0u);
            dma_16B(rsrc_words(base, y < nstages ? (uint32_t)(mn * 8) : 0u), bs ? sb16_voff : sa16_voff, dst);
        };
        // Loads of step s (and of the prologue's virtual steps): steps with
        // s & 3 == 3, 0 and 1 issue the first, second and third eight of the 24 loads
        // of stage (s+5)/4, (s+4)/4 and (s+3)/4 (dma_half order: A, B, scale words).
        // With 16-byte scale loads: A and B of half 0, A and B of half 1, then the two
        // scale loads (18 in all).
        auto dma_third = [&](int y, int k, int d) __attribute__((always_inline)) {
            if constexpr (SC16) {
                if (k < 2) dma_half(y, k, d);
                else if (d < 2) dma_scales16(y, d);
                return;
            }
            const int g = 8 * k + d;
            dma_half(y, g >= 12 ? 1 : 0, g >= 12 ? g - 12 : g);
        };
        auto dma_step = [&](int s, int d) __attribute__((always_inline)) {
            if ((s & 3) == 3) dma_third((s + 5) / 4, 0, d);
            else if ((s & 3) == 0) dma_third((s + 4) / 4, 1, d);
            else if ((s & 3) == 1) dma_third((s + 3) / 4, 2, d);
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        struct Frags {
            i32x4 a[4], b[4];
            int sa[4], sb[4];
        };
        // Read r (0..15) of step s: A blocks (4), B blocks (4), then the scale words,
        // shifted so that byte 0 is the scale of this lane's 32-token block.
        auto read_one = [&](int s, int r, Frags& f) __attribute__((always_inline)) {
            const int y = s >> 2, q = s & 3;
            const int sl = y & 1;
            const uint32_t chunk = (uint32_t)(((2 * q + lhi) ^ c_sw) << 4);
            if (r < 4) {
                f.a[r] = lds_load_16B(tiles + sl * A_STAGE, a_row + r * 32u * ROW_BYTES + chunk);
            } else if (r < 8) {
                f.b[r - 4] = lds_load_16B(tiles + B_RING + sl * B_STAGE, b_row + (r - 4) * 32u * ROW_BYTES + chunk);
            } else {
                const int x = r - 8;                  // 0..3 sa blocks, 4..7 sb blocks
                const lds_char* Sc = tiles + sc_wave + sl * SC_STAGE;
                const uint32_t w = (uint32_t)(q >> 1);
                const uint32_t off = (x < 4 ? 0u : 1024u) + (128u * w + 32u * (uint32_t)(x & 3) + (uint32_t)l32) * 4u;
                const int word = (int)((uint32_t)lds_load_4B(Sc, off) >> (8 * (2 * (q & 1) + lhi)));
                if (x < 4) f.sa[x] = word;
                else f.sb[x - 4] = word;
            }
        };
        auto mfma_one = [&](const Frags& f, int k) __attribute__((always_inline)) {
            const int j = k >> 2, i = k & 3;
            acc[j][i] = mfma_scale_e2m1_32x32x64(f.b[j], f.a[i], acc[j][i], f.sb[j], f.sa[i]);
        };

        // The partial vmcnt waits count only this item's direct loads.
        wait_vmcnt<0>();
        // Prologue: stage 0 (virtual steps -5, -4, -3) and the first third of stage 1
        // (-1); step 0 needs stage 0, with the 8 loads of stage 1's third later.
#pragma unroll
        for (int d = 0; d < 8; ++d) dma_step(-5, d);
#pragma unroll
        for (int d = 0; d < 8; ++d) dma_step(-4, d);
#pragma unroll
        for (int d = 0; d < 8; ++d) dma_step(-3, d);
#pragma unroll
        for (int d = 0; d < 8; ++d) dma_step(-1, d);
        wait_vmcnt<8>();
        barrier_no_fence();
        Frags f0, f1;
#pragma unroll
        for (int r = 0; r < 16; ++r) read_one(0, r, f0);

        // Step s = 4y + Q.  At the start of a stage's last step (Q == 3) the next
        // stage must have landed (its loads were issued in steps s-4, s-3 and s-2,
        // none since): wait for all loads, then a barrier publishes it and certifies
        // that every wave is done reading the stage before (its slot is refilled
        // from this step on).  16 MFMAs; the eight loads of steps with Q != 2 after
        // the even MFMAs; the 16 reads of step s+1 after MFMAs 8..15, two each.
        // sched_barrier(0) pins the interleaving.
        auto body = [&](int s, auto q_tag, Frags& cur, Frags& nxt) __attribute__((always_inline)) {
            constexpr int Q = decltype(q_tag)::value;
            wait_lgkmcnt0();
            if constexpr (Q == 3) {
                wait_vmcnt<0>();
                barrier_no_fence();
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                mfma_one(cur, k);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (Q != 2) {
                    if ((k & 1) == 0) dma_step(s, k >> 1);
                }
                if (k >= 8) {
                    read_one(s + 1, 2 * (k - 8), nxt);
                    read_one(s + 1, 2 * (k - 8) + 1, nxt);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int s = 0; s < ksteps; s += 4) {
            body(s, std::integral_constant<int, 0>{}, f0, f1);
            body(s + 1, std::integral_constant<int, 1>{}, f1, f0);
            body(s + 2, std::integral_constant<int, 2>{}, f0, f1);
            body(s + 3, std::integral_constant<int, 3>{}, f1, f0);
        }
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        barrier_no_fence();
        store_wave_tile_staged<OUT>(p, eo, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

template <bool SC16>
hipError_t launch_fp4(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((wgrad_fp4_kernel<kOutBf16, SC16>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((wgrad_fp4_kernel<kOutF16, SC16>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((wgrad_fp4_kernel<kOutF32, SC16>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_wgrad_fp4(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    // scale words move 16 bytes per lane (four rows) when every such load is aligned: one
    // load per operand and stage instead of four dword loads
    const bool sc16 = ((p.hidden | p.n) & 3) == 0 && (((uintptr_t)p.sfa | (uintptr_t)p.sfb) & 15u) == 0;
    if (sc16) return launch_fp4<true>(p, out_kind, grid, stream);
    return launch_fp4<false>(p, out_kind, grid, stream);
}

}  // namespace kgw
