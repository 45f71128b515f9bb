// fp8 e4m3 products in every operand layout, one UE8M0 scale per 128 contracted
// values, exact fp32 accumulation on the bf16 MFMA (gfx950):
//   - the k-grouped weight gradient in the operand majors of the cuDNN "Grouped
//     GEMM + WGrad (Unified)" page's "BF16 contract" table other than kgw_wgrad_fp8's
//     own: B stored K-major (n, tokens_sum) -- with A (hidden, tokens_sum) the DeepGEMM
//     k-grouped page's pair a (M, K), b (N, K) -- and A stored M-major
//     (tokens_sum, hidden), with B either way;
//   - the m-grouped forward product out[m] = A[m] @ W[g(m)]^T of the same MoE layer
//     (llm-infra-atlas "05 Grouped GEMM", section 2.1, m_grouped_fp8_gemm_nt_contiguous;
//     section 3: each fp8 input comes with one scale per 1x128 block along K, the
//     scales mn-major), and its dgrad out[m] = A[m] @ W[g(m)] with W stored (E, K, N).
//
// As in kgw_wgrad_fp8's kernel, every MFMA operand fragment is converted exactly to
// bf16 with its block scale folded in (v_cvt_scalef32_pk_bf16_fp8) and the bf16 MFMA
// sums the products in fp32.  One K loop serves every layout, each operand staged in
// one of two ways:
//   - "TC" (contracted axis contiguous: rows of m or n): a 128-value block of the
//     tile's 256 rows moves as one 128-byte line per row (32 KiB) into a two-slot
//     ring; stage x is loaded during step 2x-3 (8 direct loads per wave) and read
//     during steps 2x-1 and 2x with 16-byte reads, each serving two MFMA groups;
//   - "TR" (rows of the contracted axis: tokens x m or tokens x n): one 64-token step
//     of 64 rows x 256 B (16 KiB) into a four-slot ring; step s is loaded during step
//     s-3 (4 direct loads per wave) and read during step s-1 with transposing 8-byte
//     reads (ds_read_b64_tr_b8), one per MFMA group.
// The scale bytes of a 128-value block arrive with the TC cadence (2 + 2 byte loads
// per wave) into a two-slot ring.  A 64 KiB + B 64 KiB + 8 KiB of scales = 136 KiB of
// LDS.  In both modes the 16-token group g of a step takes, in lane half h, values
// 8*(g&1) + 0..7 of the step's 16-value chunk 2*(g>>1) + h, the same for both
// operands (and the same as kgw_wgrad_fp8's kernel, so every layout gives that
// kernel's result bit for bit).  One barrier per step; the loop is unrolled by four
// steps (the period of the rings), so every ring slot is a constant.
#include <type_traits>

#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int KS = 64;                      // contracted values per MFMA step
constexpr int NT = 256;
constexpr int TC_STAGE = 32 * 1024;         // 256 rows x 128 B: one 128-value block, TC
constexpr int TR_STAGE = 16 * 1024;         // 64 rows x 256 B: one step, TR
constexpr int RING = 64 * 1024;             // per operand: 2 TC stages or 4 TR steps
constexpr int B_RING = RING;
constexpr int SC_RING = 2 * RING;
constexpr int SC_WAVE = 1024;               // per wave and block: 128 sa + 128 sb dwords
constexpr int SC_STAGE = 4 * SC_WAVE;
constexpr int LDS_TOTAL = SC_RING + 2 * SC_STAGE;   // 136 KiB
constexpr int GROUP_M = 4;

static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
static_assert(4 * 32768 <= SC_RING, "output staging must fit below the scale ring");

// One operand's staging: TC or TR (see the file comment).  `rsrc(x)` gives the buffer
// resource of TC stage x / TR step x, `voff` the lane's byte offsets of its direct
// loads inside it, `rd` the per-lane LDS offsets of its fragment reads.
template <bool TR>
struct Operand;

template <>
struct Operand<false> {                     // TC
    static constexpr int kLoads = 8;        // per wave per 128-value stage
    uint32_t v[2];                          // load t: v[t & 1] + 8 t * stride
    uint32_t stride;
    uint32_t m0;                            // LDS address of this wave's rows in slot 0
    uint32_t rd[2][2];                      // [step half][group pair]
    __device__ __forceinline__ void init(int wave, int lane, int wsel, uint32_t stride_, uint32_t ring_addr) {
        const uint32_t q0 = (uint32_t)((lane & 7) ^ ((lane >> 4) & 7));
        const uint32_t q1 = (uint32_t)((lane & 7) ^ ((4 + (lane >> 4)) & 7));
        const uint32_t row0 = (uint32_t)(64 * wave + (lane >> 3));
        stride = stride_;
        v[0] = row0 * stride + q0 * 16u;
        v[1] = row0 * stride + q1 * 16u;
        m0 = ring_addr + (uint32_t)(8 * wave) * 1024u;
        const int l32 = lane & 31, lhi = lane >> 5, sw = (l32 >> 1) & 7;
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
                rd[par][pr] = (uint32_t)(wsel * 128 + l32) * 128u + (uint32_t)(((4 * par + 2 * pr + lhi) ^ sw) << 4);
    }
    // Load t (0..7) of a stage into slot `slot`: rows 64 wave + 8 t + (lane >> 3), 16-byte
    // slot lane & 7 = chunk ^ ((row >> 1) & 7).
    __device__ __forceinline__ void dma(int slot, int t, const i32x4& r) const {
        dma_16B(r, v[t & 1] + (uint32_t)(8 * t) * stride, m0 + (uint32_t)(slot * TC_STAGE) + (uint32_t)t * 1024u);
    }
};

template <>
struct Operand<true> {                      // TR
    static constexpr int kLoads = 4;        // per wave per 64-token step
    uint32_t v[2];                          // load t: v[t & 1] + 4 t * stride
    uint32_t stride;
    uint32_t m0;
    uint32_t rd0;                           // block b: rd0 ^ 32 b; group g adds 8192 (g>>1) + 2048 (g&1)
    __device__ __forceinline__ void init(int wave, int lane, int wsel, uint32_t stride_, uint32_t ring_addr) {
        const uint32_t q0 = (uint32_t)((lane & 15) ^ (2 * ((lane >> 4) & 7)));
        const uint32_t q1 = (uint32_t)((lane & 15) ^ (2 * ((4 + (lane >> 4)) & 7)));
        const uint32_t row0 = (uint32_t)(16 * wave + (lane >> 4));
        stride = stride_;
        v[0] = row0 * stride + q0 * 16u;
        v[1] = row0 * stride + q1 * 16u;
        m0 = ring_addr + (uint32_t)(4 * wave) * 1024u;
        const int g16 = lane >> 4, i16 = lane & 15;
        rd0 = (uint32_t)(16 * (g16 >> 1) + (i16 >> 1)) * 256u +
              (uint32_t)((8 * wsel + (g16 & 1)) ^ (2 * (i16 >> 1))) * 16u + (uint32_t)(i16 & 1) * 8u;
    }
    // Load t (0..3) of a step into slot `slot`: token rows 16 wave + 4 t + (lane >> 4),
    // 16-byte slot lane & 15 = chunk ^ 2 (row & 7).
    __device__ __forceinline__ void dma(int slot, int t, const i32x4& r) const {
        dma_16B(r, v[t & 1] + (uint32_t)(4 * t) * stride, m0 + (uint32_t)(slot * TR_STAGE) + (uint32_t)t * 1024u);
    }
};

// Raw fragments of one operand for one step: TC [block][group pair] 16 bytes, TR
// [block][group] 8 bytes.
template <bool TR>
struct RawOp {
    i32x4 q[4][2];
};
template <>
struct RawOp<true> {
    i32x2 q[4][4];
};

// The K loop of one 256 x 256 tile over `nstages` 128-value blocks (nstages > 0):
// acc[j][i] (+)= the product of A rows (wm*128 + 32i + ..) and B rows / columns
// (wn*128 + 32j + ..), the MFMA computing the transposed block (a lane ends up with
// four consecutive N values of one output row, as store_wave_tile_staged expects).
// rsrc_a / rsrc_b (TC stage x or TR step x) and rsrc_sa / rsrc_sb (block x) give the
// buffer resources (an empty range for anything past the range, read as zeros).
// sa_voff / sb_voff: the lane's scale byte offsets (+64 for the second 64 rows).  With
// both operands TC the two strides must be equal (they are: tokens_sum, an expert's
// count for ragged blocks, or K): the loads of both then share their per-lane offsets.
template <bool A_TR, bool B_TR, class RA, class RB, class RSA, class RSB>
__device__ __forceinline__ void fp8_kloop(f32x16 (&acc)[4][4], lds_char* tiles, uint32_t tiles_addr, int wave,
                                          int lane, int nstages, uint32_t a_stride, uint32_t b_stride,
                                          uint32_t sa_voff, uint32_t sb_voff, RA rsrc_a, RB rsrc_b, RSA rsrc_sa,
                                          RSB rsrc_sb) {
    const int wm = wave & 1, wn = wave >> 1;
    Operand<A_TR> opa;
    Operand<B_TR> opb;
    opa.init(wave, lane, wm, a_stride, tiles_addr);
    opb.init(wave, lane, wn, b_stride, tiles_addr + (uint32_t)B_RING);
    if constexpr (!A_TR && !B_TR) {
        // the same rows and chunks at the same stride: one set of load offsets (registers)
        opb.v[0] = opa.v[0];
        opb.v[1] = opa.v[1];
        opb.stride = opa.stride;
    }
    const uint32_t sc_wave = (uint32_t)(SC_RING + wave * SC_WAVE);
    const uint32_t m0_s = tiles_addr + sc_wave;
    const uint32_t sc_rd = sc_wave + 4u * (uint32_t)(lane & 31);

    // Loads issued during step s (modulo 4: R), in order: the TR steps s+3 (A, then B),
    // then for odd s the TC stages (s+3)/2 (A, then B) and the block's scale bytes (sa
    // rows 0-63 / 64-127 of this wave's half, then sb).
    constexpr int TR_LOADS = (A_TR ? Operand<true>::kLoads : 0) + (B_TR ? Operand<true>::kLoads : 0);
    constexpr int TC_LOADS = (A_TR ? 0 : Operand<false>::kLoads) + (B_TR ? 0 : Operand<false>::kLoads) + 4;
    auto loads_in = [](int R) { return TR_LOADS + ((R & 1) ? TC_LOADS : 0); };
    // Load d of step s belongs to one of six groups, in issue order: 0 A TR, 1 B TR (the
    // TR steps s+3), 2 A TC, 3 B TC (the TC stages (s+3)/2, odd s), 4 sa, 5 sb (two byte
    // loads each); group_first(q) is its first load number.
    constexpr int n_a_tr = A_TR ? Operand<true>::kLoads : 0, n_b_tr = B_TR ? Operand<true>::kLoads : 0;
    constexpr int n_a_tc = A_TR ? 0 : Operand<false>::kLoads, n_b_tc = B_TR ? 0 : Operand<false>::kLoads;
    auto group_of = [](int d) {
        if (d < n_a_tr) return 0;
        d -= n_a_tr;
        if (d < n_b_tr) return 1;
        d -= n_b_tr;
        if (d < n_a_tc) return 2;
        d -= n_a_tc;
        if (d < n_b_tc) return 3;
        d -= n_b_tc;
        return d < 2 ? 4 : 5;
    };
    auto group_first = [](int q) {
        const int f[6] = {0, n_a_tr, n_a_tr + n_b_tr, n_a_tr + n_b_tr + n_a_tc, n_a_tr + n_b_tr + n_a_tc + n_b_tc,
                          n_a_tr + n_b_tr + n_a_tc + n_b_tc + 2};
        return f[q];
    };
    // the buffer resource of group q's loads in step s
    auto group_rsrc = [&](int q, int s) -> i32x4 {
        const int x = (s + 3) >> 1;
        switch (q) {
            case 0: return rsrc_a(s + 3);
            case 1: return rsrc_b(s + 3);
            case 2: return rsrc_a(x);
            case 3: return rsrc_b(x);
            case 4: return rsrc_sa(x);
            default: return rsrc_sb(x);
        }
    };
    // load number d of step s (R = s % 4) with its group's resource r; the TR step's /
    // TC stage's slot is a constant of R
    auto dma = [&](auto rc, int d, const i32x4& r) {
        constexpr int R = decltype(rc)::value;
        constexpr int tr_slot = (R + 3) & 3;                // TR step s+3
        constexpr int tc_slot = ((R + 3) >> 1) & 1;         // TC stage (s+3)/2 (odd R)
        const int q = group_of(d), t = d - group_first(q);
        if (q == 0) {
            if constexpr (A_TR) opa.dma(tr_slot, t, r);
        } else if (q == 1) {
            if constexpr (B_TR) opb.dma(tr_slot, t, r);
        } else if (q == 2) {
            if constexpr (!A_TR) opa.dma(tc_slot, t, r);
        } else if (q == 3) {
            if constexpr (!B_TR) opb.dma(tc_slot, t, r);
        } else {
            const bool bside = q == 5;
            dma_1B(r, (bside ? sb_voff : sa_voff) + (uint32_t)t * 64u,
                   m0_s + (uint32_t)(tc_slot * SC_STAGE) + (bside ? 512u : 0u) + (uint32_t)t * 256u);
        }
    };
    auto dma_all = [&](auto rc, int s) {
        constexpr int R = decltype(rc)::value;
        i32x4 r = {0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < loads_in(R); ++d) {
            if (d == group_first(group_of(d))) r = group_rsrc(group_of(d), s);
            dma(rc, d, r);
        }
    };

    struct Raw {
        RawOp<A_TR> a;
        RawOp<B_TR> b;
        int sa[4], sb[4];
    };
    struct Conv {
        i32x4 a[4];
        i32x4 b[4];
    };
    float fa[4], fb[4];       // scale operands of the block being converted
    // Fragment x (0..3: A block x, 4..7: B block x-4) of group g of step r (modulo 4).
    auto read_frag = [&](auto rc, int g, int x, Raw& f) {
        constexpr int r = decltype(rc)::value;
        constexpr int tc_slot = (r >> 1) & 1, tr_slot = r & 3;
        if (x < 4) {
            if constexpr (A_TR)
                f.a.q[x][g] = lds_read_tr8(tiles + tr_slot * TR_STAGE + (g >> 1) * 8192 + (g & 1) * 2048,
                                           opa.rd0 ^ (uint32_t)(32 * x));
            else if ((g & 1) == 0)
                f.a.q[x][g >> 1] = lds_load_16B(tiles + tc_slot * TC_STAGE + x * 4096, opa.rd[r & 1][g >> 1]);
        } else {
            const int y = x - 4;
            if constexpr (B_TR)
                f.b.q[y][g] = lds_read_tr8(tiles + B_RING + tr_slot * TR_STAGE + (g >> 1) * 8192 + (g & 1) * 2048,
                                           opb.rd0 ^ (uint32_t)(32 * y));
            else if ((g & 1) == 0)
                f.b.q[y][g >> 1] = lds_load_16B(tiles + B_RING + tc_slot * TC_STAGE + y * 4096, opb.rd[r & 1][g >> 1]);
        }
    };
    auto read_scale = [&](auto rc, int x, Raw& f) {
        constexpr int r = decltype(rc)::value;
        constexpr int slot = (r >> 1) & 1;
        if (x < 4) f.sa[x] = lds_load_4B(tiles + slot * SC_STAGE, sc_rd + (uint32_t)(128 * x));
        else f.sb[x - 4] = lds_load_4B(tiles + slot * SC_STAGE, sc_rd + (uint32_t)(512 + 128 * (x - 4)));
    };
    // Reads after MFMA m of group g for step r: fragments m < 8 of the group, then in
    // group 0 of a stage's first step (r even) the eight scale dwords.
    auto read_one = [&](auto rc, int g, int m, Raw& f) {
        constexpr int r = decltype(rc)::value;
        if (m < 8) read_frag(rc, g, m, f);
        else if (g == 0 && (r & 1) == 0) read_scale(rc, m - 8, f);
    };
    auto decode_one = [&](const Raw& f, int x) {
        if (x < 4) fa[x] = e8m0_scale_operand((uint32_t)f.sa[x]);
        else fb[x - 4] = e8m0_scale_operand((uint32_t)f.sb[x - 4]);
    };
    auto half_of = [](const i32x4 q, int g) { return (g & 1) ? i32x2{q[2], q[3]} : i32x2{q[0], q[1]}; };
    auto convert_one = [&](const Raw& f, int g, int c, Conv& cv) {
        if (c < 4) {
            if constexpr (A_TR) cv.a[c] = cvt_e4m3x8_bf16(f.a.q[c][g], fa[c]);
            else cv.a[c] = cvt_e4m3x8_bf16(half_of(f.a.q[c][g >> 1], g), fa[c]);
        } else {
            if constexpr (B_TR) cv.b[c - 4] = cvt_e4m3x8_bf16(f.b.q[c - 4][g], fb[c - 4]);
            else cv.b[c - 4] = cvt_e4m3x8_bf16(half_of(f.b.q[c - 4][g >> 1], g), fb[c - 4]);
        }
    };
    auto mfma_one = [&](const Conv& cv, int m) {
        const int j = m >> 2, i = m & 3;
        acc[j][i] = mfma_bf16_32x32x16(cv.b[j], cv.a[i], acc[j][i]);
    };

    // The partial vmcnt waits count only these loads: earlier memory traffic drains first.
    wait_vmcnt<0>();
    // Prologue: the loads of virtual steps -3..-1 (TC stages 0 and 1 in -3 and -1, TR
    // steps 0..2), then wait for everything step 0 reads (all but virtual step -1's).
    dma_all(std::integral_constant<int, 1>(), -3);
    dma_all(std::integral_constant<int, 2>(), -2);
    dma_all(std::integral_constant<int, 3>(), -1);
    wait_vmcnt<loads_in(3)>();
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

    // Step s (R = s % 4), its raw fragments in `cur`, group 0 converted in c0.  It starts
    // by waiting for the loads of everything step s+1 reads (all but the ones step s-1
    // issued) and a barrier, which also certifies that every wave is done reading the
    // slots this step's loads refill (read during step s-2 or earlier); with both operands
    // TC only odd steps need that (an even step's successor reads the stage already in,
    // and it issues no loads).  Then 64 MFMAs in
    // four groups: after MFMA 3d+1 load d of this step, after MFMA m < 8 of group g the
    // fragment reads of step s+1 (and its scale dwords in group 0 when it opens a block),
    // and every other MFMA converts one fragment for the next group.
    auto body = [&](auto rc, int s, Raw& cur, Raw& nxt) {
        constexpr int R = decltype(rc)::value;
        constexpr bool opens = ((R + 1) & 1) == 0;        // step s+1 is a block's first step
        constexpr int nload = loads_in(R);
        const auto next = std::integral_constant<int, (R + 1) % 4>();
        // (with both operands TC an even step reads nothing new and issues no loads: no wait)
        if constexpr (A_TR || B_TR || (R & 1)) {
            wait_lgkmcnt0();
            wait_vmcnt<loads_in(R + 3)>();                // step s-1's loads may stay in flight
            barrier_no_fence();
        }
        __builtin_amdgcn_sched_barrier(0);
        i32x4 rr = {0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            Conv& cv = (g & 1) ? c1 : c0;
            Conv& cn = (g & 1) ? c0 : c1;
            if (g == 3) {
                // group 0's reads (converted in this group) and the scale dwords are
                // older than those of groups 1 and 2: four per TR operand in each, four
                // per TC operand in group 2
                constexpr int young = 4 * ((A_TR ? 2 : 1) + (B_TR ? 2 : 1));
                wait_lgkmcnt<(young > 15 ? 15 : young)>();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int k = 16 * g + m;
                mfma_one(cv, m);
                __builtin_amdgcn_sched_barrier(0);
                // a group's resource is built one MFMA before its first load
                if (k % 3 == 0 && k / 3 < nload && k / 3 == group_first(group_of(k / 3)))
                    rr = group_rsrc(group_of(k / 3), s);
                if (k % 3 == 1 && k / 3 < nload) dma(rc, k / 3, rr);
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

// A buffer resource of `bytes` bytes at `base`, or an empty one; ranges past 4 GiB are cut
// to 4 GiB (every access of one tile lies within its first 4 GiB).
__device__ __forceinline__ i32x4 rsrc_bytes(const void* base, int64_t bytes, bool live) {
    const uint32_t lim = !live || bytes <= 0 ? 0u : (bytes >= ((int64_t)1 << 32) ? 0xFFFFFFFFu : (uint32_t)bytes);
    return rsrc_words(base, lim);
}

// k-grouped weight gradient in the operand layouts other than kgw_wgrad_fp8's default
// (A_TR: A stored (tokens_sum, hidden); B_TR: B stored (tokens_sum, n), else (n,
// tokens_sum); with neither, p.ragged selects per-expert K-contiguous blocks), one UE8M0
// byte per 128 tokens for each operand (sfa (T/128, hidden), sfb (T/128, n)).  Items, token ranges, split-K chunks, zero-fill and output as in
// kgw_wgrad_fp8's kernel.
template <int OUT, bool A_TR, bool B_TR>
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_layout_kernel(GroupedParams p) {
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
        const int32_t ebegin = (int32_t)(raw_begin < 0 ? 0 : (raw_begin > T ? T : raw_begin));
        const int32_t eend = max(ebegin, (int32_t)(raw_end < 0 ? 0 : (raw_end > T ? T : raw_end)));
        int32_t begin = ebegin, end = eend;
        if (p.split > 1) {
            const int32_t len = ((end - begin + p.split - 1) / p.split + kSplitUnit - 1) & ~(kSplitUnit - 1);
            const int32_t cb = (int32_t)min<int64_t>(end, (int64_t)begin + (int64_t)c * len);
            end = (int32_t)min<int64_t>(end, (int64_t)cb + len);
            begin = cb;
        }
        // whole 128-token blocks; ragged blocks are counted from their own start, so the loads
        // stay inside the expert's block even for malformed offsets
        const bool ragged = !A_TR && !B_TR && p.ragged;
        if (ragged) begin = ebegin + ((begin - ebegin) & ~127);
        else begin &= ~127;
        const int nblocks = (end - begin) / 128;
        if (nblocks == 0) {
            if (!p.accumulate) zero_tile<OUT, BM, BN, NT>(p, eo, m0, n0, tid);
            continue;
        }
        const int nsteps = 2 * nblocks;
        // TC: rows m (n) at stride T from token `begin`; rows past hidden (n) read as zeros
        // through the range (at most 256 T < 2^32 bytes).  TR: token rows at stride hidden
        // (n) from row `begin`, the tile's 256 columns at m0 (n0); columns past hidden (n)
        // read the next row's bytes (outputs that are never stored), the range ending at the
        // end of the operand.
        // Ragged (both TC): expert e's A block is (hidden, n_e) row-major from element
        // ebegin*hidden, its B block (n, n_e) from ebegin*n; rows at stride n_e.
        // (bases and byte counts per item; a stage / step only adds a multiple of its size)
        const int64_t ne = (int64_t)eend - ebegin, koff = (int64_t)begin - ebegin;
        const int64_t tc_stride = ragged ? ne : T;
        const uint8_t* Abase = (const uint8_t*)p.A +
                               (A_TR ? (int64_t)begin * H + m0 : ragged ? ebegin * H + m0 * ne + koff : m0 * T + begin);
        const uint8_t* Bbase = (const uint8_t*)p.B +
                               (B_TR ? (int64_t)begin * N + n0 : ragged ? ebegin * N + n0 * ne + koff : n0 * T + begin);
        const int64_t a_bytes = A_TR ? T * H - ((int64_t)begin * H + m0)
                                     : min<int64_t>(BM, H - m0) * tc_stride - (ragged ? koff : begin);
        const int64_t b_bytes = B_TR ? T * N - ((int64_t)begin * N + n0)
                                     : min<int64_t>(BN, N - n0) * tc_stride - (ragged ? koff : begin);
        const int64_t a_step = A_TR ? (int64_t)KS * H : 128;      // bytes per TR step / TC stage
        const int64_t b_step = B_TR ? (int64_t)KS * N : 128;
        const int a_units = A_TR ? nsteps : nblocks, b_units = B_TR ? nsteps : nblocks;
        auto rsrc_a = [&](int x) {
            const int64_t o = (int64_t)x * a_step;
            if constexpr (A_TR) return rsrc_bytes(Abase + o, a_bytes - o, x < a_units);
            else return rsrc_words(Abase + o, x < a_units ? (uint32_t)(a_bytes - o) : 0u);
        };
        auto rsrc_b = [&](int x) {
            const int64_t o = (int64_t)x * b_step;
            if constexpr (B_TR) return rsrc_bytes(Bbase + o, b_bytes - o, x < b_units);
            else return rsrc_words(Bbase + o, x < b_units ? (uint32_t)(b_bytes - o) : 0u);
        };
        const int64_t gb0 = begin / 128;
        auto rsrc_sa = [&](int x) { return rsrc_words(p.sfa + (gb0 + x) * H, x < nblocks ? (uint32_t)H : 0u); };
        auto rsrc_sb = [&](int x) { return rsrc_words(p.sfb + (gb0 + x) * N, x < nblocks ? (uint32_t)N : 0u); };
        f32x16 acc[4][4];
        zero_acc(acc);
        fp8_kloop<A_TR, B_TR>(acc, tiles, tiles_addr, wave, lane, nblocks, (uint32_t)(A_TR ? H : tc_stride),
                              (uint32_t)(B_TR ? N : tc_stride), (uint32_t)(m0 + wm * 128 + lane),
                              (uint32_t)(n0 + wn * 128 + lane), rsrc_a, rsrc_b, rsrc_sa, rsrc_sb);
        store_wave_tile_staged<OUT>(p, eo, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

// m-grouped product with fp8 operands: A (M, K) with sa (K/128, M); W with sw (E, K/128, N),
// stored (E, N, K) for the forward (NTL, "nt": W staged TC) or (E, K, N) for dgrad ("nn":
// W staged TR); K a multiple of 128; groups from offsets or m_indices, each starting on a
// multiple of 128 rows.  Items, and the treatment of a tile whose 128-row halves lie in two
// groups (one item per half), follow kgw_mgrouped_bf16's kernel; a half of no group is not
// stored.
template <int OUT, bool NTL>
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
        // Items num_tiles.. are the second halves of the tiles whose 128-row halves lie in
        // two groups (see kgw_mgrouped_bf16's kernel): the first item computes half 0 with
        // group g0, the second half 1 with g1, the other half's A rows (and scales) read as
        // zeros.
        const bool second = item >= p.num_tiles;
        int tm, tn;
        tile_coords(second ? item - p.num_tiles : item, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        const int g0 = group_of_row(p, m0);
        const int g1 = m0 + 128 < M ? group_of_row(p, m0 + 128) : -1;
        const bool v0 = g0 >= 0 && g0 < p.num_groups;
        const bool v1 = g1 >= 0 && g1 < p.num_groups;
        if (!v0 && !v1) continue;
        const bool split = v0 && v1 && g0 != g1;
        if (second && !split) continue;
        const int grp = second ? g1 : (v0 ? g0 : g1);
        const int live_half = split ? (second ? 1 : 0) : -1;   // -1: both halves' rows
        if (nbk == 0) {
            if (!p.accumulate && !second) {
                if (v0) zero_tile<OUT, 128, BN, NT>(p, 0, m0, n0, tid);
                if (v1) zero_tile<OUT, 128, BN, NT>(p, 0, m0 + 128, n0, tid);
            }
            continue;
        }
        const int rows_valid = (int)min<int64_t>(BM, M - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        const uint8_t* Abase = (const uint8_t*)p.A + m0 * K;
        // nt: the group's rows n0.. of (N, K); nn: its K rows of (K, N) from column n0, the
        // range running to the end of W (columns past N read the next row's bytes, outputs
        // that are never stored)
        const uint8_t* W0 = (const uint8_t*)p.W + (NTL ? ((int64_t)grp * N + n0) * K : (int64_t)grp * K * N + n0);
        const int64_t w_end = (int64_t)p.num_groups * K * N - ((int64_t)grp * K * N + n0);
        const uint8_t* SW0 = p.sw + (int64_t)grp * nbk * N + n0;
        const uint8_t* SA0 = p.sa + m0;
        const int64_t a_bytes = (int64_t)rows_valid * K, w_bytes = (int64_t)cols_valid * K;
        const bool a_live = live_half < 0 || a_half == live_half;
        const bool s_live = live_half < 0 || s_half == live_half;
        auto rsrc_a = [&](int x) {
            const int64_t o = (int64_t)x * 128;
            return rsrc_words(Abase + o, x < nbk && a_live ? (uint32_t)(a_bytes - o) : 0u);
        };
        auto rsrc_b = [&](int x) {
            if constexpr (NTL) {
                const int64_t o = (int64_t)x * 128;
                return rsrc_words(W0 + o, x < nbk ? (uint32_t)(w_bytes - o) : 0u);
            } else {
                const int64_t o = (int64_t)x * KS * N;
                return rsrc_bytes(W0 + o, w_end - o, x < 2 * nbk);
            }
        };
        auto rsrc_sa = [&](int x) {
            return rsrc_words(SA0 + (int64_t)x * M, x < nbk && s_live ? (uint32_t)rows_valid : 0u);
        };
        auto rsrc_sb = [&](int x) { return rsrc_words(SW0 + (int64_t)x * N, x < nbk ? (uint32_t)cols_valid : 0u); };
        f32x16 acc[4][4];
        zero_acc(acc);
        fp8_kloop<false, !NTL>(acc, tiles, tiles_addr, wave, lane, nbk, (uint32_t)K, (uint32_t)(NTL ? K : N),
                                (uint32_t)(wm * 128 + lane), (uint32_t)(wn * 128 + lane), rsrc_a, rsrc_b, rsrc_sa,
                                rsrc_sb);
        const bool mine = split ? wm == live_half : (wm ? v1 : v0);
        if (mine) store_wave_tile_staged<OUT>(p, 0, m0 + wm * 128, n0 + wn * 128, lane, acc, tiles + wave * 32768);
        barrier_no_fence();
    }
}

template <bool A_TR, bool B_TR>
hipError_t launch_layout(const GroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((wgrad_fp8_layout_kernel<kOutBf16, A_TR, B_TR>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((wgrad_fp8_layout_kernel<kOutF16, A_TR, B_TR>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((wgrad_fp8_layout_kernel<kOutF32, A_TR, B_TR>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_wgrad_fp8_layout(const GroupedParams& p, bool a_m_major, bool b_k_major, int out_kind, int grid,
                                   hipStream_t stream) {
    if (!a_m_major && b_k_major) return launch_layout<false, false>(p, out_kind, grid, stream);
    if (a_m_major && b_k_major) return launch_layout<true, false>(p, out_kind, grid, stream);
    if (a_m_major && !b_k_major) return launch_layout<true, true>(p, out_kind, grid, stream);
    return hipErrorInvalidValue;     // the default layout is kgw_wgrad_fp8's own kernel
}

template <bool NTL>
hipError_t launch_mg8(const MGroupedParams& p, int out_kind, int grid, hipStream_t stream) {
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL((mgrouped_fp8_kernel<kOutBf16, NTL>), dim3(grid), dim3(NT), 0, stream, p);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL((mgrouped_fp8_kernel<kOutF16, NTL>), dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((mgrouped_fp8_kernel<kOutF32, NTL>), dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mgrouped_fp8(const MGroupedParams& p, bool nt, int out_kind, int grid, hipStream_t stream) {
    return nt ? launch_mg8<true>(p, out_kind, grid, stream) : launch_mg8<false>(p, out_kind, grid, stream);
}

}  // namespace kgw
