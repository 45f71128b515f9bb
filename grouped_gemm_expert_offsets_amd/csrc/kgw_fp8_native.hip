// Persistent K-grouped weight-gradient kernel on the native scaled fp8 MFMA,
// OCP e4m3 operands with one UE8M0 scale per 128 tokens (gfx950).
//
// Accuracy note: v_mfma_scale_f32_32x32x64_f8f6f4 does not round its
// internal sum correctly.  Products that share a K group inside one
// instruction are aligned to the group's largest product and only about 13
// bits below it are kept (1 + 2^-12 survives, 1 + 2^-14 loses the small
// term); groups and the fp32 accumulator are added in full fp32.  On
// block-quantised Gaussian operands this gives a relative Frobenius error of
// about 1.5e-5 against the exact sum: far below the resolution of a bf16
// output, above the 1e-5 asked of an fp32 output.  kgw_fp8_exact.hip converts
// to bf16 and uses the bf16 MFMA instead.
//
// Same operation and work decomposition as the bf16 kernel (cuDNN "Grouped GEMM
// + WGrad (Unified)", section "Operation"); the operands are fp8 with per-block
// 1x128 power-of-two scales (llm-infra-atlas "05 Grouped GEMM", section 3),
// the blocks running along the contracted token axis.  The scales are applied
// inside the MFMA: each lane hands the instruction the scale byte of its row
// (A) or column (B).  Every 64-token MFMA lies inside one 128-token block, so
// each output row m uses the single byte sfa[block][m] and each column n the
// single byte sfb[block][n]: the products are qa*qb*2^(ea-127)*2^(eb-127) with
// no dequantisation pass.
//
// The instruction's K order: lane l of an operand holds K 16*(l>>5) + 0..15 in
// bytes 0..15 and K 32 + 16*(l>>5) + 0..15 in bytes 16..31, and it applies the
// scale of lanes 0..31 to K 0..31 and that of lanes 32..63 to K 32..63 (one
// scale per row / column per 32 K).  The fragment reads below follow that
// order, so each 32-token half of a step is one hardware scale block: with
// 32-token scales (the MX instantiation, the DeepGEMM k-grouped page's
// gran_k = 32, packed four to a word) each lane passes the byte of its half.
//
// Pipeline (the bf16 kernel's, in bytes): K step of 64 tokens = 16 MFMAs of
// 32x32x64 per wave (4 waves, each 128x128 of the 256x256 tile).  Direct
// global->LDS loads, no register staging:
//   - A in 128-token stages (256 rows x 128 B, one scale block, every row a
//     full 128-byte line) in a 3-slot ring, swizzle chunk ^ ((row>>1)&7);
//     fragments are two 16-byte LDS reads;
//   - B in 64-token stages (64 rows x 256 B) in a 3-slot ring, swizzle
//     chunk ^ 2*(k&7); fragments are four transposing ds_read_b64_tr_b8;
//   - the scale bytes of each block travel with its A stage into a 3-slot
//     scale ring: byte-wide direct loads, each lane's byte landing as one
//     zero-extended dword (so a lane reads its scale as a ready MFMA operand
//     and any hidden / n is handled byte by byte);
//   - each wave issues ten loads per step (B step s+3, half an A stage, two
//     scale loads), spread over its 16 MFMAs; one barrier per step; the
//     fragments of step s+1 are read during the second half of step s;
//   - the finished tile leaves through the idle rings (LDS transpose, whole
//     row segments per store).
#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kFp8BM, BN = kFp8BN;
constexpr int KS = 64;                      // tokens per K step (one MFMA deep)
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
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_native_kernel(GroupedParams p) {
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

    // Direct-load slots of this lane.  A: wave instruction t (0..7) fills LDS
    // rows 64*wave + 8*t + (lane>>3), 16-byte slot lane&7, which holds logical
    // chunk (lane&7) ^ ((row>>1)&7) -- that depends on t only through t&1.  B:
    // instruction t (0..3) fills k-rows 16*wave + 4*t + (lane>>4), slot lane&15
    // = logical chunk ^ 2*(k&7), again a function of t&1.
    const int a_q0 = (lane & 7) ^ ((lane >> 4) & 7);
    const int a_q1 = (lane & 7) ^ ((4 + (lane >> 4)) & 7);
    const int b_q0 = (lane & 15) ^ (2 * ((lane >> 4) & 7));
    const int b_q1 = (lane & 15) ^ (2 * ((4 + (lane >> 4)) & 7));

    // Fragment read offsets (fixed per lane), in the instruction's K order:
    // tokens 16*lhi + 0..15 and 32 + 16*lhi + 0..15 of the step.  A: row
    // wm*128 + 32i + l32, two 16-byte reads (chunks 4*(s&1) + lhi and + 2 of the
    // stage row).  B: lane l gets column 32j + l32 of the wave's half from four
    // 8x16 transposed blocks at k-rows 16*lhi + {0, 8, 32, 40}; block j's offset
    // is block 0's with the 16-byte chunk index XOR 2j (the unswizzled chunk
    // 8wn + (g16&1) + 2j has no carry).
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u;
    const int a_sw = (l32 >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    const uint32_t b_frag0 = (uint32_t)(16 * (g16 >> 1) + (i16 >> 1)) * 256u +
                             (uint32_t)((8 * wn + (g16 & 1)) ^ (2 * (i16 >> 1))) * 16u + (uint32_t)(i16 & 1) * 8u;
    // Scale dwords of this wave: sa row r at 4r, sb column c at 512 + 4c.
    const uint32_t sc_wave = (uint32_t)(SC_RING + wave * SC_WAVE);

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
        // never stored; the buffer ranges below end at the last valid A row and at
        // the end of B, so such lanes read zeros or bytes of B's next row, never
        // memory outside the operands.
        const int64_t a_rows_bytes = min<int64_t>(BM, H - m0) * T - begin;
        const int64_t b_bytes = (T - begin) * N - n0;
        const uint32_t a_voff0 = (uint32_t)(64 * wave + (lane >> 3)) * (uint32_t)T;
        const uint32_t b_voff0 = (uint32_t)(16 * wave + (lane >> 4)) * (uint32_t)N;
        // Scales: sa for rows m0 + wm*128 + 64h + lane, sb for columns
        // n0 + wn*128 + 64h + lane (h = 0, 1), one byte (or, packed, one byte or
        // word at a 4-byte stride) each; values past hidden / n read as 0 through
        // the buffer range and belong to rows / columns never stored.
        constexpr uint32_t sstride = FMT == kScalesU8 ? 1u : 4u;
        const uint32_t sa_voff = (uint32_t)(m0 + wm * 128 + lane) * sstride;
        const uint32_t sb_voff = (uint32_t)(n0 + wn * 128 + lane) * sstride;

        // Direct loads.  A stage a (steps 2a, 2a+1; scale block a) goes to A slot
        // a % NA, B step s to B slot s % NB.  Stages past the expert's range use
        // an empty buffer range: the loads fetch nothing (the slot is never read
        // by an MFMA), keeping the loop free of branches and its vmcnt counts
        // uniform.
        auto dma_a = [&](int a, int t) {
            const uint32_t dst = tiles_addr + (uint32_t)((a % NA) * A_STAGE) + (uint32_t)(8 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(Abase + (int64_t)a * (2 * KS),
                                       a < nblocks ? (uint32_t)(a_rows_bytes - (int64_t)a * (2 * KS)) : 0u);
            const uint32_t voff = a_voff0 + (uint32_t)(8 * t) * (uint32_t)T + (uint32_t)((t & 1) ? a_q1 : a_q0) * 16u;
            dma_16B(r, voff, dst);
        };
        auto dma_b = [&](int sb, int t) {
            const uint32_t dst = tiles_addr + (uint32_t)(B_RING + (sb % NB) * B_STAGE) + (uint32_t)(4 * wave + t) * 1024u;
            const i32x4 r = rsrc_words(Bbase + (int64_t)sb * KS * N,
                                       sb < ksteps ? (uint32_t)min<int64_t>(b_bytes - (int64_t)sb * KS * N, 0xFFFFFFFFll) : 0u);
            const uint32_t voff = b_voff0 + (uint32_t)(4 * t) * (uint32_t)N + (uint32_t)((t & 1) ? b_q1 : b_q0) * 16u;
            dma_16B(r, voff, dst);
        };
        // Scale load h (0, 1) of block a: operand B (sb) or A (sa).
        auto dma_s = [&](int a, bool b_side, int h) {
            const uint32_t dst = tiles_addr + sc_wave + (uint32_t)((a % NA) * SC_STAGE) +
                                 (b_side ? 512u : 0u) + (uint32_t)h * 256u;
            const ScaleSource src = scale_source<FMT>(b_side ? p.sfb : p.sfa, b_side ? N : H, gb0 + a);
            const i32x4 r = rsrc_words(src.base, a < nblocks ? src.limit : 0u);
            const uint32_t voff = (b_side ? sb_voff : sa_voff) + (uint32_t)h * 64u * sstride;
            if constexpr (MX) dma_4B(r, voff, dst);
            else dma_1B(r, voff, dst);
        };
        // The loads of step s (also for the prologue's virtual steps s < 0), in
        // issue order: B step s+3, then half of an A stage and two scale loads
        // of its block -- for odd s the first half of A stage (s+5)/2 and its sa
        // bytes, for even s the second half of A stage (s+4)/2 and its sb bytes.
        // Every slot written this way was last read during step s-1 or earlier.
        auto dma_step = [&](int s, int d) {
            if (d < B_LOADS) {
                if (s + NB >= 0) dma_b(s + NB, d);
            } else if (d < 2 * B_LOADS) {
                if (s & 1) dma_a((s + 5) / 2, d - B_LOADS);
                else dma_a((s + 4) / 2, d);
            } else {
                if (s & 1) dma_s((s + 5) / 2, false, d - 2 * B_LOADS);
                else dma_s((s + 4) / 2, true, d - 2 * B_LOADS);
            }
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        // Fragments of one K step plus the scales of its block: MFMA operands of
        // 32 bytes (tokens 32*lhi + 0..31 of one row m or column n).
        struct Frags {
            i32x8 a[4];
            i32x8 b[4];
            int sa[4], sb[4];
        };
        // Fragment read number r (0..31) of step s: A halves (8), B pieces (16),
        // then the block's scale dwords (8); an MX word is shifted so that byte 0
        // is the scale of the lane's 32-token half, block 2*(s&1) + lhi of the stage.
        auto read_one = [&](int s, int r, Frags& f) {
            if (r < 8) {
                const int i = r >> 1, h = r & 1;
                const lds_char* As = tiles + ((s >> 1) % NA) * A_STAGE;
                const uint32_t chunk = (uint32_t)(((4 * (s & 1) + lhi + 2 * h) ^ a_sw) << 4);
                const i32x4 v = lds_load_16B(As, a_frag_row + i * 4096u + chunk);
#pragma unroll
                for (int x = 0; x < 4; ++x) f.a[i][4 * h + x] = v[x];
            } else if (r < 24) {
                const int j = (r - 8) >> 2, q = (r - 8) & 3;
                const lds_char* Bs = tiles + B_RING + (s % NB) * B_STAGE;
                const i32x2 v = lds_read_tr8(Bs, (b_frag0 ^ (uint32_t)(32 * j)) + q * 2048u + (q >> 1) * 4096u);
                f.b[j][2 * q] = v[0];
                f.b[j][2 * q + 1] = v[1];
            } else {
                const lds_char* Sc = tiles + sc_wave + ((s >> 1) % NA) * SC_STAGE;
                const int q = r - 24;
                int w;
                if (q < 4) w = lds_load_4B(Sc, (uint32_t)(4 * (32 * q + l32)));
                else w = lds_load_4B(Sc, (uint32_t)(512 + 4 * (32 * (q - 4) + l32)));
                if constexpr (MX) w = (int)((uint32_t)w >> (8 * (2 * (s & 1) + lhi)));
                if (q < 4) f.sa[q] = w;
                else f.sb[q - 4] = w;
            }
        };
        auto read_all = [&](int s, Frags& f) {
#pragma unroll
            for (int r = 0; r < 32; ++r) read_one(s, r, f);
        };
        // MFMA number k (0..15): N block k/4 times M block k%4.
        auto mfma_one = [&](const Frags& f, int k) {
            const int j = k >> 2, i = k & 3;
            acc[j][i] = mfma_scale_e4m3_32x32x64(f.b[j], f.a[i], acc[j][i], f.sb[j], f.sa[i]);
        };

        // The partial vmcnt waits count only this item's direct loads, so the
        // previous item's output stores must have drained first.
        wait_vmcnt<0>();
        // Prologue: the loads of virtual steps -5..-1.  Step 0's fragments need
        // A stage 0 with its scales and B step 0; 26 loads were issued after B 0.
#pragma unroll
        for (int v = -5; v < 0; ++v)
#pragma unroll
            for (int d = 0; d < LOADS_PER_STEP; ++d) dma_step(v, d);
        wait_vmcnt<26>();
        barrier_no_fence();
        Frags f0, f1;
        read_all(0, f0);

        // Step s with its fragments in `cur`: once this wave's reads of step s
        // and the loads step s+1 needs are done, a barrier publishes step s+1 and
        // certifies that every wave is done reading step s.  Step s+1 needs B
        // step s+1 (issued first in step s-2) and, for odd s, A stage (s+1)/2 and
        // its scales (completed in step s-3): at most 16 later loads may remain.
        // 16 MFMAs, the step's ten loads spread among them (one or two MFMAs
        // apart), the 32 fragment reads of step s+1 after the last eight.
        // sched_barrier(0) pins this interleaving.
        auto body = [&](int s, Frags& cur, Frags& nxt) {
            wait_lgkmcnt0();
            wait_vmcnt<16>();
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                mfma_one(cur, k);
                __builtin_amdgcn_sched_barrier(0);
                // loads d at MFMAs 0,1,3,4,6,8,9,11,12,14
                constexpr int slot_of[LOADS_PER_STEP] = {0, 1, 3, 4, 6, 8, 9, 11, 12, 14};
#pragma unroll
                for (int d = 0; d < LOADS_PER_STEP; ++d)
                    if (slot_of[d] == k) dma_step(s, d);
                if (k >= 8) {
#pragma unroll
                    for (int r = 4 * (k - 8); r < 4 * (k - 7); ++r) read_one(s + 1, r, nxt);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int s = 0; s < ksteps; s += 2) {
            body(s, f0, f1);
            body(s + 1, f1, f0);
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
static void launch_native(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((wgrad_fp8_native_kernel<kOutBf16, FMT>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((wgrad_fp8_native_kernel<kOutF16, FMT>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((wgrad_fp8_native_kernel<kOutF32, FMT>), dim3(grid), dim3(NT), 0, stream, p);
}

hipError_t launch_wgrad_fp8_native(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (p.scale_format == kScalesPacked32) launch_native<kScalesPacked32>(p, out_kind, grid, stream);
    else if (p.scale_format == kScalesPacked) launch_native<kScalesPacked>(p, out_kind, grid, stream);
    else launch_native<kScalesU8>(p, out_kind, grid, stream);
    return hipGetLastError();
}

}  // namespace kgw
