// Persistent K-grouped weight-gradient kernel, OCP e4m3 operands with one UE8M0
// scale per 128 tokens (or per 32 tokens, MX), fp32 accumulation on the bf16
// MFMA (gfx950).  This is the kernel behind kgw_wgrad_fp8.
//
// Same operation and work decomposition as the bf16 kernel (cuDNN "Grouped GEMM
// + WGrad (Unified)", section "Operation"); the operands are fp8 with per-block
// 1x128 power-of-two scales (llm-infra-atlas "05 Grouped GEMM", section 3),
// the blocks running along the contracted token axis.  The MX instantiation
// takes one scale per 32 tokens instead (the DeepGEMM k-grouped page's
// gran_k = 32), packed four to a word: one word per row per 128-token stage.
//
// The fp8 bytes travel from HBM to LDS as fp8 (half the bytes of bf16).  Each
// MFMA operand fragment -- eight tokens of one output row m (from A) or one
// output column n (from B) -- is read from LDS and converted to bf16 with its
// block scale folded in (v_cvt_scalef32_pk_bf16_fp8).  Both steps are exact: an
// e4m3 value times a power of two is a bf16 number.  The bf16 MFMA then forms
// and sums the products in fp32, so the result carries only fp32 accumulation
// rounding, unlike the native fp8 MFMA whose internal sum drops low-order bits
// (see kgw_fp8_native.hip).
//
// Loads and LDS layout are those of the native fp8 kernel (both kernels move
// the same bytes): A in 128-token stages (256 rows x 128 B, one scale block)
// in a 3-slot ring, B in 64-token stages (64 rows x 256 B) in a 3-slot ring,
// the block's scale bytes by byte-wide direct loads (the MX scale words by
// dword-wide ones) into a 3-slot scale ring,
// ten direct loads per wave per 64-token step spread over its MFMAs, one
// barrier per step.  The K loop is unrolled by six steps (the period of the
// three-slot rings), so every ring slot is a constant and a fragment read is
// one LDS instruction on a per-lane offset: one wave issues every instruction of
// its SIMD, and each one between two MFMAs costs MFMA time once there are more
// than about five.  Inside a step the wave runs four 16-token groups of 16
// bf16 MFMAs (32x32x16; 4 waves, each 128x128 of the 256x256 tile):
//   - raw fp8 fragments of step s+1 (16-byte A reads, each serving two
//     groups, and transposing ds_read_b64_tr_b8 B reads) are read from LDS
//     during the matching group of step s, the scale dwords of a new block
//     during group 0;
//   - the eight fragments of group g+1 are converted while group g's MFMAs run
//     (two converted sets alternate), and group 0 of step s+1 while group 3
//     runs, so the conversions hide behind the MFMAs;
//   - the finished tile leaves through the idle rings (LDS transpose, whole
//     row segments per store).
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kFp8BM, BN = kFp8BN;
constexpr int KS = 64;                      // tokens per K step
constexpr int NT = 256;
constexpr int NA = 3;                       // A ring: 3 stages of 128 tokens (2 K steps)
constexpr int NB = 3;                       // B ring: 3 stages of 64 tokens (1 K step)
constexpr int A_STAGE = BM * 2 * KS;        // 32 KiB: 256 rows x 128 B
constexpr int B_STAGE = KS * BN;            // 16 KiB: 64 rows x 256 B
constexpr int SC_WAVE = 1024;               // per wave and block: 128 sa + 128 sb dwords
constexpr int SC_STAGE = 4 * SC_WAVE;       // 4 KiB per block
constexpr int B_RING = NA * A_STAGE;        // byte offsets of the rings
constexpr int SC_RING = B_RING + NB * B_STAGE;
constexpr int LDS_TOTAL = SC_RING + NA * SC_STAGE;   // 156 KiB
constexpr int GROUP_M = 4;
constexpr int B_LOADS = 4;                  // direct loads per wave per B stage
constexpr int LOADS_PER_STEP = 10;          // 4 B + 4 A + 2 scale

static_assert(BM == 256 && BN == 256 && kFp8BK == 2 * KS, "index math below assumes 256x256, 128-token blocks");
static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
static_assert(2 * 128 * 512 <= SC_RING, "output staging must fit below the scale ring");

template <int OUT, int FMT>
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_kernel(GroupedParams p) {
    constexpr bool MX = FMT == kScalesPacked32;           // one scale per 32 tokens
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;

    // Direct-load slots (as in the native fp8 kernel).  A: wave instruction t
    // (0..7) fills LDS rows 64*wave + 8*t + (lane>>3), 16-byte slot lane&7 =
    // logical chunk ^ ((row>>1)&7), a function of t&1.  B: instruction t (0..3)
    // fills k-rows 16*wave + 4*t + (lane>>4), slot lane&15 = chunk ^ 2*(k&7).
    const int a_q0 = (lane & 7) ^ ((lane >> 4) & 7);
    const int a_q1 = (lane & 7) ^ ((4 + (lane >> 4)) & 7);
    const int b_q0 = (lane & 15) ^ (2 * ((lane >> 4) & 7));
    const int b_q1 = (lane & 15) ^ (2 * ((4 + (lane >> 4)) & 7));

    // Fragment reads.  An MFMA's 16 K slots may hold any 16 tokens as long as
    // both operands agree; the step's 64 tokens are four 16-token chunks, and
    // 16-token group g takes, in lane half lhi, tokens 8*(g&1) + 0..7 of chunk
    // 2*(g>>1) + lhi.  So one 16-byte A read (a whole chunk of one row) serves
    // groups 2p and 2p+1, and groups 0-1 / 2-3 stay the step's first / second
    // 32 tokens (one 32-token scale block each).  A: row wm*128 + 32i + l32,
    // chunk 4*(s&1) + 2p + lhi of the 128-token stage row: offset a_rd[s&1][p],
    // block i adds 4096.  B: column 32j + l32 of the wave's half, one transposed
    // 8x16 block at k-rows 32*(g>>1) + 16*lhi + 8*(g&1) + 0..7: offset b_rd[j],
    // group g adds 8192*(g>>1) + 2048*(g&1).  All per lane and fixed for the
    // kernel; each step adds only its ring slot's constant base.
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_row = (uint32_t)(wm * 128 + l32) * 128u;
    const int a_sw = (l32 >> 1) & 7;
    uint32_t a_rd[2][2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) a_rd[par][pr] = a_row + (uint32_t)(((4 * par + 2 * pr + lhi) ^ a_sw) << 4);
    const int g16 = lane >> 4, i16 = lane & 15;
    const uint32_t b_frag0 = (uint32_t)(16 * (g16 >> 1) + (i16 >> 1)) * 256u +
                             (uint32_t)((8 * wn + (g16 & 1)) ^ (2 * (i16 >> 1))) * 16u + (uint32_t)(i16 & 1) * 8u;
    uint32_t b_rd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b_rd[j] = b_frag0 ^ (uint32_t)(32 * j);
    // Scale dwords of this wave: sa row r at 4r, sb column c at 512 + 4c.
    const uint32_t sc_wave = (uint32_t)(SC_RING + wave * SC_WAVE);
    const uint32_t sc_rd = sc_wave + 4u * (uint32_t)l32;

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
        // Token range, clamped into [0, tokens_sum], used in whole 128-token blocks.
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
        begin &= ~(2 * KS - 1);
        const int nblocks = (end - begin) / (2 * KS);
        const int ksteps = 2 * nblocks;
        if (ksteps == 0) {
            if (!p.accumulate) zero_tile<OUT, BM, BN, NT>(p, eo, m0, n0, tid);
            continue;
        }

        const uint8_t* Abase = (const uint8_t*)p.A + m0 * T + begin;
        const uint8_t* Bbase = (const uint8_t*)p.B + (int64_t)begin * N + n0;
        const int64_t gb0 = begin / (2 * KS);          // global index of the item's first 128-token block
        // Rows of A past hidden and columns of B past n belong to outputs that are
        // never stored; the buffer ranges end at the last valid A row and at the
        // end of B, so such lanes read zeros or bytes of B's next row, never
        // memory outside the operands.
        const int64_t a_rows_bytes = min<int64_t>(BM, H - m0) * T - begin;
        const int64_t b_bytes = (T - begin) * N - n0;
        const int64_t b_step_bytes = (int64_t)KS * N;
        const uint32_t a_voff0 = (uint32_t)(64 * wave + (lane >> 3)) * (uint32_t)T;
        const uint32_t b_voff0 = (uint32_t)(16 * wave + (lane >> 4)) * (uint32_t)N;
        // Scales: sa for rows m0 + wm*128 + 64h + lane, sb for columns
        // n0 + wn*128 + 64h + lane (h = 0, 1), one byte (or, packed, one byte or
        // word at a 4-byte stride) each; values past hidden / n read as 0 through
        // the buffer range and belong to rows / columns never stored.
        constexpr uint32_t sstride = FMT == kScalesU8 ? 1u : 4u;
        const uint32_t sa_voff = (uint32_t)(m0 + wm * 128 + lane) * sstride;
        const uint32_t sb_voff = (uint32_t)(n0 + wn * 128 + lane) * sstride;
        // Per-lane global offsets of the direct loads (the row offset of
        // instruction t is uniform and added per load).
        const uint32_t a_voff_even = a_voff0 + (uint32_t)a_q0 * 16u;
        const uint32_t a_voff_odd = a_voff0 + (uint32_t)a_q1 * 16u;
        const uint32_t b_voff_even = b_voff0 + (uint32_t)b_q0 * 16u;
        const uint32_t b_voff_odd = b_voff0 + (uint32_t)b_q1 * 16u;
        const uint32_t a_m0 = tiles_addr + (uint32_t)(8 * wave) * 1024u;
        const uint32_t b_m0 = tiles_addr + (uint32_t)B_RING + (uint32_t)(4 * wave) * 1024u;
        const uint32_t s_m0 = tiles_addr + sc_wave;

        // Buffer resources of the loads: A stage a (steps 2a, 2a+1; scale block a),
        // B step sb, the scales of block a; a stage past the expert's range gets
        // an empty range (its loads fetch nothing).  All of it is wave-uniform.
        auto rsrc_a = [&](int a) {
            return rsrc_words(Abase + (int64_t)a * (2 * KS),
                              a < nblocks ? (uint32_t)(a_rows_bytes - (int64_t)a * (2 * KS)) : 0u);
        };
        auto rsrc_s = [&](int a, bool b_side) {
            const ScaleSource src = scale_source<FMT>(b_side ? p.sfb : p.sfa, b_side ? N : H, gb0 + a);
            return rsrc_words(src.base, a < nblocks ? src.limit : 0u);
        };
        // B: a running base and remaining byte count, advanced one step at a time.
        const uint8_t* b_next = Bbase;
        int64_t b_left = b_bytes;
        int b_step = 0;
        auto rsrc_b_next = [&]() {
            // b_left stays positive while b_step < ksteps; a range beyond 4 GiB is cut to 4 GiB
            const uint32_t lim = b_step < ksteps ? ((uint32_t)((uint64_t)b_left >> 32) ? 0xFFFFFFFFu : (uint32_t)b_left)
                                                 : 0u;
            const i32x4 r = rsrc_words(b_next, lim);
            b_next += b_step_bytes;
            b_left -= b_step_bytes;
            ++b_step;
            return r;
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        // Raw fp8 fragments of one K step (A: [block][group pair], 16 bytes; B:
        // [block][group], 8 bytes) plus the step's scale dwords; one group's
        // converted bf16 operands; and the scale operands the conversions use
        // now (A blocks 0-3, B blocks 0-3): those of the block being converted,
        // switched to the next block in the group that starts converting it.
        struct Raw {
            i32x4 a[4][2];
            i32x2 b[4][4];
            int sa[4], sb[4];
        };
        struct Conv {
            i32x4 a[4];
            i32x4 b[4];
        };
        float fa[4], fb[4];
        // With one scale per 128 tokens, steps 2b and 2b+1 share block b: only the
        // odd steps read and switch scales for the step after them.
        auto reads_scales = [](int r_next) { return MX || (r_next & 1) == 0; };
        // Read (g, m) of step r (r = the step's index modulo 6, which fixes its
        // ring slots: A stage (r >> 1) % NA, B step r % NB), made after MFMA m of
        // group g: for m < 4 in groups 0 and 2 A block m of the group pair, for
        // 4 <= m < 8 B block m-4 of the group; in group 0, for m >= 8 the step's
        // scale dword m-8 (sa blocks 0-3, then sb 0-3) when its block is new.
        // Every address is a per-lane offset plus a constant.
        auto read_one = [&](auto rc, int g, int m, Raw& f) {
            constexpr int r = decltype(rc)::value;
            constexpr uint32_t a_slot = (uint32_t)(((r >> 1) % NA) * A_STAGE);
            constexpr uint32_t b_slot = (uint32_t)(B_RING + (r % NB) * B_STAGE);
            constexpr uint32_t s_slot = (uint32_t)(((r >> 1) % NA) * SC_STAGE);
            if (m >= 8) {
                if (g != 0 || !reads_scales(r)) return;
                const int x = m - 8;
                if (x < 4) f.sa[x] = lds_load_4B(tiles + s_slot, sc_rd + (uint32_t)(128 * x));
                else f.sb[x - 4] = lds_load_4B(tiles + s_slot, sc_rd + (uint32_t)(512 + 128 * (x - 4)));
            } else if (m < 4) {
                if (g & 1) return;
                f.a[m][g >> 1] = lds_load_16B(tiles + a_slot + m * 4096, a_rd[r & 1][g >> 1]);
            } else {
                f.b[m - 4][g] = lds_read_tr8(tiles + b_slot + (g >> 1) * 8192 + (g & 1) * 2048, b_rd[m - 4]);
            }
        };
        // Scale operand x (A blocks 0-3, then B blocks 4-7) from the step's scale
        // dwords, for the 32-token block `sub` (0..3) of the stage (MX) or for the
        // stage's single block.
        auto decode_one = [&](const Raw& f, int x, int sub) {
            const uint32_t w = (uint32_t)(x < 4 ? f.sa[x] : f.sb[x - 4]);
            const float v = e8m0_scale_operand(MX ? (w >> (8 * sub)) & 0xFFu : w);
            if (x < 4) fa[x] = v;
            else fb[x - 4] = v;
        };
        // Conversion number c (0..7) of group g: A block c, then B block c-4.
        auto convert_one = [&](const Raw& f, int g, int c, Conv& cv) {
            if (c < 4) {
                const i32x4 q = f.a[c][g >> 1];
                const i32x2 h = (g & 1) ? i32x2{q[2], q[3]} : i32x2{q[0], q[1]};
                cv.a[c] = cvt_e4m3x8_bf16(h, fa[c]);
            } else {
                cv.b[c - 4] = cvt_e4m3x8_bf16(f.b[c - 4][g], fb[c - 4]);
            }
        };
        // MFMA number m (0..15) of a group: N block m/4 times M block m%4.
        auto mfma_one = [&](const Conv& cv, int m) {
            const int j = m >> 2, i = m & 3;
            acc[j][i] = mfma_bf16_32x32x16(cv.b[j], cv.a[i], acc[j][i]);
        };
        // The loads of step s (also the prologue's virtual steps s < 0), in issue
        // order d = 0..9: B step s+3 (its four instructions), then half of an A
        // stage and two scale loads of its block -- for odd s the first half of
        // A stage (s+5)/2 and its sa bytes, for even s the second half of A stage
        // (s+4)/2 and its sb bytes.  Every slot written this way was last read
        // during step s-1 or earlier.  `rb` is B step s+3's resource, `ra` / `rs`
        // those of the A stage and its scales.
        auto dma_step = [&](auto rc, int d, const i32x4& rb, const i32x4& ra, const i32x4& rs) {
            constexpr int r = decltype(rc)::value;             // the step modulo 6 (>= 0)
            constexpr int a_slot = ((r & 1) ? (r + 5) / 2 : (r + 4) / 2) % NA;
            if (d < B_LOADS) {
                const uint32_t dst = b_m0 + (uint32_t)(((r + NB) % NB) * B_STAGE) + (uint32_t)d * 1024u;
                dma_16B(rb, ((d & 1) ? b_voff_odd : b_voff_even) + (uint32_t)(4 * d) * (uint32_t)N, dst);
            } else if (d < 2 * B_LOADS) {
                const int t = (r & 1) ? d - B_LOADS : d;
                const uint32_t dst = a_m0 + (uint32_t)(a_slot * A_STAGE) + (uint32_t)t * 1024u;
                dma_16B(ra, ((t & 1) ? a_voff_odd : a_voff_even) + (uint32_t)(8 * t) * (uint32_t)T, dst);
            } else {
                const int h = d - 2 * B_LOADS;
                constexpr bool b_side = !(r & 1);
                const uint32_t dst = s_m0 + (uint32_t)(a_slot * SC_STAGE) + (b_side ? 512u : 0u) + (uint32_t)h * 256u;
                const uint32_t voff = (b_side ? sb_voff : sa_voff) + (uint32_t)h * 64u * sstride;
                if constexpr (MX) dma_4B(rs, voff, dst);
                else dma_1B(rs, voff, dst);
            }
        };
        // The prologue's virtual step v (-5..-1): its residue modulo 6 is v + 6.
        auto dma_all = [&](auto rc, int v) {
            const int a = (v & 1) ? (v + 5) / 2 : (v + 4) / 2;
            const i32x4 rb = v + NB >= 0 ? rsrc_b_next() : i32x4{0, 0, 0, 0};
            const i32x4 ra = rsrc_a(a);
            const i32x4 rs = rsrc_s(a, !(v & 1));
#pragma unroll
            for (int d = 0; d < LOADS_PER_STEP; ++d)
                if (d >= B_LOADS || v + NB >= 0) dma_step(rc, d, rb, ra, rs);
        };

        // The partial vmcnt waits count only this item's direct loads, so the
        // previous item's output stores must have drained first.
        wait_vmcnt<0>();
        // Prologue: the loads of virtual steps -5..-1.  Step 0's fragments need
        // A stage 0 with its scales and B step 0; 26 loads were issued after B 0.
        dma_all(std::integral_constant<int, 1>(), -5);
        dma_all(std::integral_constant<int, 2>(), -4);
        dma_all(std::integral_constant<int, 3>(), -3);
        dma_all(std::integral_constant<int, 4>(), -2);
        dma_all(std::integral_constant<int, 5>(), -1);
        wait_vmcnt<26>();
        barrier_no_fence();
        Raw r0, r1;
        Conv c0, c1;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int m = 0; m < 16; ++m) read_one(std::integral_constant<int, 0>(), g, m, r0);
        wait_lgkmcnt0();
#pragma unroll
        for (int x = 0; x < 8; ++x) decode_one(r0, x, 0);       // step 0 opens block 0
#pragma unroll
        for (int c = 0; c < 8; ++c) convert_one(r0, 0, c, c0);

        // Step s, its raw fragments in `cur` and group 0 already converted in c0:
        // once this wave's reads and the loads step s+1 needs are done, a barrier
        // publishes step s+1 (B step s+1 issued first in step s-2, A stage
        // (s+1)/2 and its scales completed in step s-3: at most 16 later loads
        // may remain) and certifies that every wave is done reading step s.
        // Then 64 MFMAs in four groups; after MFMA k = 16g + m: direct load k/6
        // when k%6 == 2 (their buffer resources made a few MFMAs earlier), read (g, m)
        // of step s+1 (group g's raw fragments, and the scales in group 0), and
        // every other MFMA one conversion for the next group (group 0 of step s+1
        // during group 3, each conversion after the MFMA that decodes its scale,
        // once the scale reads of group 0 are in).  With 32-token scales (MX)
        // groups 2g and 2g+1 share block 2*(s&1) + g of the stage: during group 1
        // (whose conversions are group 2's) the scale operands of `cur` are
        // switched to the second block the same way.  sched_barrier(0) pins the
        // interleaving.
        // `rc` carries s modulo 6 (the period of the three-slot rings), so every
        // ring slot below is a constant.
        auto body = [&](auto rc, int s, Raw& cur, Raw& nxt) {
            constexpr int R = decltype(rc)::value;
            const auto next = std::integral_constant<int, (R + 1) % 6>();
            const int a = (R & 1) ? (s + 5) / 2 : (s + 4) / 2;
            wait_lgkmcnt0();
            wait_vmcnt<16>();
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            i32x4 rb, ra, rs;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                Conv& cv = (g & 1) ? c1 : c0;
                Conv& cn = (g & 1) ? c0 : c1;
                if (g == 3) {
                    // the scale reads of group 0 are older than the 12 reads of groups 1-2
                    wait_lgkmcnt<12>();
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int k = 16 * g + m;
                    mfma_one(cv, m);
                    __builtin_amdgcn_sched_barrier(0);
                    if (k == 0) rb = rsrc_b_next();
                    if (k == 20) ra = rsrc_a(a);
                    if (k == 44) rs = rsrc_s(a, !(R & 1));
                    if (k % 6 == 2 && k / 6 < LOADS_PER_STEP) dma_step(rc, k / 6, rb, ra, rs);
                    read_one(next, g, m, nxt);
                    if (m & 1) {
                        if (g < 3) convert_one(cur, g + 1, m >> 1, cn);
                        else convert_one(nxt, 0, m >> 1, cn);
                    } else {
                        if (MX && g == 1) decode_one(cur, m >> 1, 2 * (R & 1) + 1);
                        if (g == 3 && reads_scales((R + 1) % 6)) decode_one(nxt, m >> 1, MX ? 2 * ((R + 1) & 1) : 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // Six steps per iteration, then the remaining two or four (ksteps is even).
        int s = 0;
        for (; s + 6 <= ksteps; s += 6) {
            body(std::integral_constant<int, 0>(), s, r0, r1);
            body(std::integral_constant<int, 1>(), s + 1, r1, r0);
            body(std::integral_constant<int, 2>(), s + 2, r0, r1);
            body(std::integral_constant<int, 3>(), s + 3, r1, r0);
            body(std::integral_constant<int, 4>(), s + 4, r0, r1);
            body(std::integral_constant<int, 5>(), s + 5, r1, r0);
        }
        if (s < ksteps) {
            body(std::integral_constant<int, 0>(), s, r0, r1);
            body(std::integral_constant<int, 1>(), s + 1, r1, r0);
            if (s + 2 < ksteps) {
                body(std::integral_constant<int, 2>(), s + 2, r0, r1);
                body(std::integral_constant<int, 3>(), s + 3, r1, r0);
            }
        }
        // The rings become the output staging area: every wave must be done
        // reading them and every direct load (the empty ones past the range
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

template <int FMT>
static void launch_exact(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((wgrad_fp8_kernel<kOutBf16, FMT>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((wgrad_fp8_kernel<kOutF16, FMT>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((wgrad_fp8_kernel<kOutF32, FMT>), dim3(grid), dim3(NT), 0, stream, p);
}

hipError_t launch_wgrad_fp8(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (p.scale_format == kScalesPacked32) launch_exact<kScalesPacked32>(p, out_kind, grid, stream);
    else if (p.scale_format == kScalesPacked) launch_exact<kScalesPacked>(p, out_kind, grid, stream);
    else launch_exact<kScalesU8>(p, out_kind, grid, stream);
    return hipGetLastError();
}

}  // namespace kgw
