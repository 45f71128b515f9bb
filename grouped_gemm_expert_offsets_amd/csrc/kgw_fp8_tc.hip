// fp8 e4m3 products whose two operands both keep the contracted axis contiguous
// ("TC": every row of an output axis holds its contracted values back to back),
// with one UE8M0 scale per 128 contracted values, exact fp32 accumulation on the
// bf16 MFMA (gfx950):
//   - the k-grouped weight gradient with B stored K-major, B (n, tokens_sum) (the
//     cuDNN "Grouped GEMM + WGrad (Unified)" page's BF16-contract operand layouts
//     carried over to fp8; the DeepGEMM k-grouped page's pair a (M, K), b (N, K));
//   - the m-grouped forward product out[m] = A[m] @ W[g(m)]^T of the same MoE layer
//     (llm-infra-atlas "05 Grouped GEMM", section 2.1, m_grouped_fp8_gemm_nt_contiguous;
//     section 3: each fp8 input comes with one scale per 1x128 block along K, the
//     scales mn-major).
//
// As in kgw_wgrad_fp8's kernel, every MFMA operand fragment is converted exactly to
// bf16 with its block scale folded in (v_cvt_scalef32_pk_bf16_fp8) and the bf16 MFMA
// sums the products in fp32.  The K loop differs in that both operands are staged
// alike: a 128-value block of 256 rows moves as one full 128-byte line per row (32
// KiB per operand), so each operand has a two-slot ring (A 64 KiB + B 64 KiB + 8 KiB
// of scales = 136 KiB of LDS).  Stage x is loaded during step 2x-3 (20 direct loads
// per wave: 8 A, 8 B, 2 + 2 scale), read during steps 2x-1 and 2x, and its slot is
// free again at the start of step 2x+1.  Fragments of both operands are 16-byte LDS
// reads of one row's chunk, each serving two MFMA groups (16-token group g takes,
// in lane half lhi, values 8*(g&1) + 0..7 of the step's chunk 2*(g>>1) + lhi, the
// same for both operands).  The K loop is unrolled by four steps (the period of the
// two-slot rings), so every ring slot is a constant.
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int KS = 64;                      // contracted values per MFMA step
constexpr int NT = 256;
constexpr int STAGE = 32 * 1024;            // 256 rows x 128 B: one 128-value block of one operand
constexpr int B_RING = 2 * STAGE;
constexpr int SC_RING = 4 * STAGE;
constexpr int SC_WAVE = 1024;               // per wave and block: 128 sa + 128 sb dwords
constexpr int SC_STAGE = 4 * SC_WAVE;
constexpr int LDS_TOTAL = SC_RING + 2 * SC_STAGE;   // 136 KiB
constexpr int LOADS = 20;                   // direct loads per wave per stage
constexpr int GROUP_M = 4;

static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
static_assert(4 * 32768 <= SC_RING, "output staging must fit below the scale ring");

// The K loop of one 256 x 256 tile over `nstages` 128-value blocks (nstages > 0):
// acc[j][i] (+)= the product of A rows (wm*128 + 32i + ..) and B rows (wn*128 + 32j
// + ..), the MFMA computing the transposed block (a lane ends up with four
// consecutive N values of one output row, as store_wave_tile_staged expects).
// rsrc_a / rsrc_b / rsrc_sa / rsrc_sb (stage x) give the buffer resources of stage
// x's rows (an empty range for stages to be read as zeros); the lane offsets inside
// them are row * stride + chunk for the operands and sa_voff / sb_voff (+64 for the
// second 64 rows) for the scale bytes.
template <class RA, class RB, class RSA, class RSB>
__device__ __forceinline__ void tc_kloop(f32x16 (&acc)[4][4], lds_char* tiles, uint32_t tiles_addr, int wave,
                                         int lane, int nstages, uint32_t a_stride, uint32_t b_stride,
                                         uint32_t sa_voff, uint32_t sb_voff, RA rsrc_a, RB rsrc_b, RSA rsrc_sa,
                                         RSB rsrc_sb) {
    const int wm = wave & 1, wn = wave >> 1;
    // Direct loads: wave instruction t (0..7) fills LDS rows 64*wave + 8*t + (lane>>3),
    // 16-byte slot lane&7 = logical chunk ^ ((row>>1)&7), a function of t&1.
    const uint32_t q0 = (uint32_t)((lane & 7) ^ ((lane >> 4) & 7));
    const uint32_t q1 = (uint32_t)((lane & 7) ^ ((4 + (lane >> 4)) & 7));
    const uint32_t row0 = (uint32_t)(64 * wave + (lane >> 3));
    const uint32_t a_v[2] = {row0 * a_stride + q0 * 16u, row0 * a_stride + q1 * 16u};
    const uint32_t b_v[2] = {row0 * b_stride + q0 * 16u, row0 * b_stride + q1 * 16u};
    const uint32_t m0_a = tiles_addr + (uint32_t)(8 * wave) * 1024u;
    const uint32_t m0_b = tiles_addr + (uint32_t)B_RING + (uint32_t)(8 * wave) * 1024u;
    const uint32_t sc_wave = (uint32_t)(SC_RING + wave * SC_WAVE);
    const uint32_t m0_s = tiles_addr + sc_wave;
    // Fragment reads: row wm*128 + 32i + l32 (A) / wn*128 + 32j + l32 (B), chunk
    // 4*par + 2*p + lhi of the 128-byte row, swizzled as written; block i adds 4096.
    const int l32 = lane & 31, lhi = lane >> 5;
    const int sw = (l32 >> 1) & 7;
    uint32_t a_rd[2][2], b_rd[2][2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const uint32_t ch = (uint32_t)(((4 * par + 2 * pr + lhi) ^ sw) << 4);
            a_rd[par][pr] = (uint32_t)(wm * 128 + l32) * 128u + ch;
            b_rd[par][pr] = (uint32_t)(wn * 128 + l32) * 128u + ch;
        }
    const uint32_t sc_rd = sc_wave + 4u * (uint32_t)l32;

    // Loads of stage x (into slot x & 1), load number d = 0..19: A t = d (0..7), B
    // t = d-8, then the sa bytes of rows 0-63 / 64-127 of this wave's half, then sb.
    auto dma = [&](auto slot_c, int d, const i32x4& r) {
        constexpr int slot = decltype(slot_c)::value;
        if (d < 8) {
            dma_16B(r, a_v[d & 1] + (uint32_t)(8 * d) * a_stride, m0_a + (uint32_t)(slot * STAGE) + (uint32_t)d * 1024u);
        } else if (d < 16) {
            const int t = d - 8;
            dma_16B(r, b_v[t & 1] + (uint32_t)(8 * t) * b_stride, m0_b + (uint32_t)(slot * STAGE) + (uint32_t)t * 1024u);
        } else {
            const int h = (d - 16) & 1;
            const bool bside = d >= 18;
            dma_1B(r, (bside ? sb_voff : sa_voff) + (uint32_t)h * 64u,
                   m0_s + (uint32_t)(slot * SC_STAGE) + (bside ? 512u : 0u) + (uint32_t)h * 256u);
        }
    };
    auto rsrc_of = [&](int d, int x) -> i32x4 {
        return d < 8 ? rsrc_a(x) : d < 16 ? rsrc_b(x) : d < 18 ? rsrc_sa(x) : rsrc_sb(x);
    };

    struct Raw {
        i32x4 a[4][2];
        i32x4 b[4][2];
        int sa[4], sb[4];
    };
    struct Conv {
        i32x4 a[4];
        i32x4 b[4];
    };
    float fa[4], fb[4];       // scale operands of the block being converted
    // Read (g, m) of step r (r = the step modulo 4: stage slot (r >> 1) & 1, half r & 1
    // of its 128-value rows): in groups 0 and 2, after MFMA m < 4 A block m of the group
    // pair, after MFMA 4..7 B block m-4; in group 0, after MFMAs 8..15, the scale dwords
    // of a stage's first step.
    auto read_one = [&](auto rc, int g, int m, Raw& f) {
        constexpr int r = decltype(rc)::value;
        constexpr int slot = (r >> 1) & 1;
        if (g & 1) return;
        if (m < 4) {
            f.a[m][g >> 1] = lds_load_16B(tiles + slot * STAGE + m * 4096, a_rd[r & 1][g >> 1]);
        } else if (m < 8) {
            f.b[m - 4][g >> 1] = lds_load_16B(tiles + B_RING + slot * STAGE + (m - 4) * 4096, b_rd[r & 1][g >> 1]);
        } else if (g == 0 && (r & 1) == 0) {
            const int x = m - 8;
            if (x < 4) f.sa[x] = lds_load_4B(tiles + slot * SC_STAGE, sc_rd + (uint32_t)(128 * x));
            else f.sb[x - 4] = lds_load_4B(tiles + slot * SC_STAGE, sc_rd + (uint32_t)(512 + 128 * (x - 4)));
        }
    };
    auto decode_one = [&](const Raw& f, int x) {
        if (x < 4) fa[x] = e8m0_scale_operand((uint32_t)f.sa[x]);
        else fb[x - 4] = e8m0_scale_operand((uint32_t)f.sb[x - 4]);
    };
    auto half_of = [](const i32x4 q, int g) { return (g & 1) ? i32x2{q[2], q[3]} : i32x2{q[0], q[1]}; };
    auto convert_one = [&](const Raw& f, int g, int c, Conv& cv) {
        if (c < 4) cv.a[c] = cvt_e4m3x8_bf16(half_of(f.a[c][g >> 1], g), fa[c]);
        else cv.b[c - 4] = cvt_e4m3x8_bf16(half_of(f.b[c - 4][g >> 1], g), fb[c - 4]);
    };
    auto mfma_one = [&](const Conv& cv, int m) {
        const int j = m >> 2, i = m & 3;
        acc[j][i] = mfma_bf16_32x32x16(cv.b[j], cv.a[i], acc[j][i]);
    };

    // The partial vmcnt waits count only these loads: earlier memory traffic drains first.
    wait_vmcnt<0>();
    // Prologue: stage 0 (virtual step -3) and stage 1 (virtual step -1) into slots 0, 1.
#pragma unroll
    for (int d = 0; d < LOADS; ++d) dma(std::integral_constant<int, 0>(), d, rsrc_of(d, 0));
#pragma unroll
    for (int d = 0; d < LOADS; ++d) dma(std::integral_constant<int, 1>(), d, rsrc_of(d, 1));
    wait_vmcnt<LOADS>();
    barrier_no_fence();
    Raw r0, r1;
    Conv c0, c1;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int m = 0; m < 16; ++m) read_one(std::integral_constant<int, 0>(), g, m, r0);
    wait_lgkmcnt0();
#pragma unroll
    for (int x = 0; x < 8; ++x) decode_one(r0, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) convert_one(r0, 0, c, c0);

    // Step s (R = s % 4), its raw fragments in `cur`, group 0 converted in c0.  Odd s:
    // step s+1 opens stage (s+1)/2, loaded during step s-2 and nothing since: wait for
    // every load; even s: step s+1's stage is already in.  The barrier also certifies
    // that every wave is done reading step s.  Then 64 MFMAs in four groups; odd steps
    // load stage (s+3)/2 into the slot stage (s-1)/2 left (load d after MFMA 3d+1),
    // and every other MFMA converts one fragment for the next group.
    auto body = [&](auto rc, int s, Raw& cur, Raw& nxt) {
        constexpr int R = decltype(rc)::value;
        constexpr bool odd = R & 1;
        constexpr bool opens = ((R + 1) & 1) == 0;        // step s+1 is a stage's first step
        const auto next = std::integral_constant<int, (R + 1) % 4>();
        const auto load_slot = std::integral_constant<int, ((R + 3) >> 1) & 1>();
        const int lx = (s + 3) >> 1;
        wait_lgkmcnt0();
        if constexpr (odd) wait_vmcnt<0>();
        else wait_vmcnt<LOADS>();
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        i32x4 rr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            Conv& cv = (g & 1) ? c1 : c0;
            Conv& cn = (g & 1) ? c0 : c1;
            if (g == 3) {
                wait_lgkmcnt<8>();        // group 0's reads are older than group 2's eight
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int k = 16 * g + m;
                mfma_one(cv, m);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (odd) {
                    if (k == 0 || k == 23 || k == 47 || k == 53) rr = rsrc_of(k == 0 ? 0 : k == 23 ? 8 : k == 47 ? 16 : 18, lx);
                    if (k % 3 == 1 && k / 3 < LOADS) dma(load_slot, k / 3, rr);
                }
                read_one(next, g, m, nxt);
                if (m & 1) {
                    if (g < 3) convert_one(cur, g + 1, m >> 1, cn);
                    else convert_one(nxt, 0, m >> 1, cn);
                } else if (g == 3 && opens) {
                    decode_one(nxt, m >> 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    const int ksteps = 2 * nstages;
    int s = 0;
    for (; s + 4 <= ksteps; s += 4) {
        body(std::integral_constant<int, 0>(), s, r0, r1);
        body(std::integral_constant<int, 1>(), s + 1, r1, r0);
        body(std::integral_constant<int, 2>(), s + 2, r0, r1);
        body(std::integral_constant<int, 3>(), s + 3, r1, r0);
    }
    if (s < ksteps) {
        body(std::integral_constant<int, 0>(), s, r0, r1);
        body(std::integral_constant<int, 1>(), s + 1, r1, r0);
    }
    // The rings become the output staging area: every wave done reading them and every
    // direct load (the empty ones past the range included) landed.
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier_no_fence();
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
}

// k-grouped weight gradient, A (hidden, T) and B (n, T) both token-contiguous, one
// UE8M0 byte per 128 tokens for each (sfa (T/128, hidden), sfb (T/128, n)).  Items,
// token ranges, split-K chunks, zero-fill and output as in kgw_wgrad_fp8's kernel.
template <int OUT>
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_bk_kernel(GroupedParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;
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
        begin &= ~127;
        const int nblocks = (end - begin) / 128;
        if (nblocks == 0) {
            if (!p.accumulate) zero_tile<OUT, BM, BN, NT>(p, eo, m0, n0, tid);
            continue;
        }
        // Rows past hidden / n read as zeros through the buffer ranges (their outputs
        // are never stored), so no access leaves the operands.
        const uint8_t* Abase = (const uint8_t*)p.A + m0 * T + begin;
        const uint8_t* Bbase = (const uint8_t*)p.B + n0 * T + begin;
        const int64_t a_bytes = min<int64_t>(BM, H - m0) * T - begin;
        const int64_t b_bytes = min<int64_t>(BN, N - n0) * T - begin;
        const int64_t gb0 = begin / 128;
        auto rsrc_a = [&](int x) {
            return rsrc_words(Abase + (int64_t)x * 128, x < nblocks ? (uint32_t)(a_bytes - (int64_t)x * 128) : 0u);
        };
        auto rsrc_b = [&](int x) {
            return rsrc_words(Bbase + (int64_t)x * 128, x < nblocks ? (uint32_t)(b_bytes - (int64_t)x * 128) : 0u);
        };
        auto rsrc_sa = [&](int x) { return rsrc_words(p.sfa + (gb0 + x) * H, x < nblocks ? (uint32_t)H : 0u); };
        auto rsrc_sb = [&](int x) { return rsrc_words(p.sfb + (gb0 + x) * N, x < nblocks ? (uint32_t)N : 0u); };
        f32x16 acc[4][4];
        zero_acc(acc);
        tc_kloop(acc, tiles, tiles_addr, wave, lane, nblocks, (uint32_t)T, (uint32_t)T,
                 (uint32_t)(m0 + wm * 128 + lane), (uint32_t)(n0 + wn * 128 + lane), rsrc_a, rsrc_b, rsrc_sa, rsrc_sb);
        store_wave_tile_staged<OUT>(p, eo, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

// m-grouped forward product with fp8 operands: A (M, K) with sa (K/128, M); W (E, N, K)
// with sw (E, K/128, N); K a multiple of 128; groups from offsets or m_indices, each
// starting on a multiple of 128 rows.  Items and the two-pass treatment of a tile whose
// 128-row halves lie in two groups follow kgw_mgrouped_bf16's kernel: in each pass the
// other half's A rows (and their scales) read as zeros, both passes accumulate into the
// same registers, and a half of no group is not stored.
template <int OUT>
__global__ __launch_bounds__(NT, 1) void mgrouped_fp8_kernel(MGroupedParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    lds_char* tiles = (lds_char*)smem;
    const uint32_t tiles_addr = lds_addr(smem);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t M = p.hidden, N = p.n, K = p.k;
    const int nbk = (int)(K / 128);              // blocks of one pass
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);
    // The A loads of waves 0-1 cover tile rows 0-127 and those of waves 2-3 rows 128-255;
    // the sa bytes of wave w cover rows (w & 1) * 128 ..
    const int a_half = wave >> 1, s_half = wm;

    for (int item = slot; item < p.num_items; item += G) {
        int tm, tn;
        tile_coords(item, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        const int g0 = group_of_row(p, m0);
        const int g1 = m0 + 128 < M ? group_of_row(p, m0 + 128) : -1;
        const bool v0 = g0 >= 0 && g0 < p.num_groups;
        const bool v1 = g1 >= 0 && g1 < p.num_groups;
        if (!v0 && !v1) continue;
        const bool two = v0 && v1 && g0 != g1;
        const int pg0 = v0 ? g0 : g1;
        const int pg1 = two ? g1 : pg0;
        const int nstages = (two ? 2 : 1) * nbk;
        if (nstages == 0) {
            if (!p.accumulate) {
                if (v0) zero_tile<OUT, 128, BN, NT>(p, 0, m0, n0, tid);
                if (v1) zero_tile<OUT, 128, BN, NT>(p, 0, m0 + 128, n0, tid);
            }
            continue;
        }
        const int rows_valid = (int)min<int64_t>(BM, M - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        const uint8_t* Abase = (const uint8_t*)p.A + m0 * K;
        // the pass's group as an offset from the first (pointers selected per pass
        // would keep the captures in scratch memory)
        const uint8_t* W0 = (const uint8_t*)p.W + ((int64_t)pg0 * N + n0) * K;
        const int64_t wdelta = (int64_t)(pg1 - pg0) * N * K;
        const uint8_t* SW0 = p.sw + (int64_t)pg0 * nbk * N + n0;
        const int64_t swdelta = (int64_t)(pg1 - pg0) * nbk * N;
        auto pass_of = [&](int x) { return (two && x >= nbk) ? 1 : 0; };
        auto rsrc_a = [&](int x) {
            const int ps = pass_of(x), lx = x - ps * nbk;
            const bool live = x < nstages && (!two || ps == a_half);
            return rsrc_words(Abase + (int64_t)lx * 128, live ? (uint32_t)((int64_t)rows_valid * K - (int64_t)lx * 128) : 0u);
        };
        auto rsrc_b = [&](int x) {
            const int ps = pass_of(x), lx = x - ps * nbk;
            return rsrc_words(W0 + (ps ? wdelta : 0) + (int64_t)lx * 128,
                              x < nstages ? (uint32_t)((int64_t)cols_valid * K - (int64_t)lx * 128) : 0u);
        };
        auto rsrc_sa = [&](int x) {
            const int ps = pass_of(x), lx = x - ps * nbk;
            const bool live = x < nstages && (!two || ps == s_half);
            return rsrc_words(p.sa + (int64_t)lx * M + m0, live ? (uint32_t)rows_valid : 0u);
        };
        auto rsrc_sb = [&](int x) {
            const int ps = pass_of(x), lx = x - ps * nbk;
            return rsrc_words(SW0 + (ps ? swdelta : 0) + (int64_t)lx * N, x < nstages ? (uint32_t)cols_valid : 0u);
        };
        f32x16 acc[4][4];
        zero_acc(acc);
        tc_kloop(acc, tiles, tiles_addr, wave, lane, nstages, (uint32_t)K, (uint32_t)K, (uint32_t)(wm * 128 + lane),
                 (uint32_t)(wn * 128 + lane), rsrc_a, rsrc_b, rsrc_sa, rsrc_sb);
        const bool mine = wm ? v1 : v0;
        if (mine) store_wave_tile_staged<OUT>(p, 0, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

}  // namespace

hipError_t launch_wgrad_fp8_bk(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL(wgrad_fp8_bk_kernel<kOutBf16>, dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL(wgrad_fp8_bk_kernel<kOutF16>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(wgrad_fp8_bk_kernel<kOutF32>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mgrouped_fp8(const MGroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL(mgrouped_fp8_kernel<kOutBf16>, dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL(mgrouped_fp8_kernel<kOutF16>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(mgrouped_fp8_kernel<kOutF32>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kgw
