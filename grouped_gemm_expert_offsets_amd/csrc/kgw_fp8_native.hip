// Persistent K-grouped weight-gradient kernel on the native scaled fp8 MFMA,
// OCP e4m3 operands with one UE8M0 scale per 128 tokens (gfx950).
//
// Accuracy note: v_mfma_scale_f32_32x32x64_f8f6f4 does not round its
// internal sum correctly.  Products that share a K group inside one
// instruction are aligned to the group's largest product and only about 13
// bits below it are kept (1 + 2^-12 survives, 1 + 2^-14 loses the small
// term); groups and the fp32 accumulator are added in full fp32.  On
// block-quantised Gaussian operands this gives a relative Frobenius error of
// about 1.5e-5 against the exact sum.  The default fp8 kernel
// (kgw_fp8_exact.hip) avoids this by converting to bf16 and using the bf16
// MFMA; this one is the opt-in fast path.
//
// Same operation and work decomposition as the bf16 kernel (cuDNN "Grouped GEMM
// + WGrad (Unified)", section "Operation"); the operands are fp8 with per-block
// 1x128 power-of-two scales (llm-infra-atlas "05 Grouped GEMM", section 3),
// the blocks running along the contracted token axis.
//
// The K step is one scale block (128 tokens).  The scales are applied inside
// the MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies each lane's operand by
// 2^(byte-127) of the scale byte it is given.  Because every 64-token MFMA
// lies inside one 128-token block, each output row m uses the single byte
// sfa[block][m] and each column n the single byte sfb[block][n], so the
// products are exactly qa*qb*2^(ea-127)*2^(eb-127) with no dequantisation
// pass and no rounding beyond the fp32 accumulation.
//
//   - A tile 256 x 128 bytes (token-contiguous rows): fragments are two
//     16-byte LDS reads (rows swizzled: chunk ^ ((row>>1)&7));
//   - B tile 128 x 256 bytes (N-contiguous rows): fragments are four
//     transposing ds_read_b64_tr_b8 (rows swizzled: chunk ^ 2*(k&7));
//   - double-buffered LDS ring, register staging, 4 waves of 128x128.
#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kFp8BM, BN = kFp8BN, BK = kFp8BK;
constexpr int NT = 256;
constexpr int A_STAGE = BM * BK;            // 32 KiB: 256 rows x 128 B
constexpr int B_STAGE = BK * BN;            // 32 KiB: 128 rows x 256 B
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int LDS_TILES = 2 * STAGE;
constexpr int GROUP_M = 4;

static_assert(BM == 256 && BN == 256 && BK == 128, "index math below assumes 256x256x128");

template <bool OUT_BF16>
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_native_kernel(GroupedParams p) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_TILES + kMaxExperts * 4];
    lds_char* tiles = (lds_char*)smem;
    int32_t* s_end = (int32_t*)(smem + LDS_TILES);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;

    for (int e = tid; e < p.num_experts; e += NT) {
        int64_t v = p.offsets[e];
        v = v < 0 ? 0 : (v > T ? T : v);
        s_end[e] = (int32_t)v;
    }
    __syncthreads();

    // A chunk c = tid + 256*pp: row (tid>>3) + 32*pp, 16-byte chunk tid&7.
    const uint32_t a_lds0 = (uint32_t)(tid >> 3) * 128u + (uint32_t)(((tid & 7) ^ ((tid >> 4) & 7)) << 4);
    // B chunk c = tid + 256*pp: k-row (tid>>4) + 16*pp, 16-byte chunk tid&15.
    const uint32_t b_lds0 = (uint32_t)(tid >> 4) * 256u + (uint32_t)(((tid & 15) ^ (2 * ((tid >> 4) & 7))) << 4);

    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u;
    const int a_sw = (lane >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    uint32_t b_frag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 32 * (g16 >> 1) + (i16 >> 1);
        const int chunk = (8 * wn + 2 * j + (g16 & 1)) ^ (2 * (i16 >> 1));
        b_frag[j] = (uint32_t)krow * 256u + (uint32_t)chunk * 16u + (uint32_t)(i16 & 1) * 8u;
    }

    const int TT = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G, p.num_xcds);

    for (int item = slot; item < p.num_items; item += G) {
        const int e = item / TT;
        const int local = item - e * TT;
        int tm, tn;
        tile_coords(local, p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
        const int64_t m0 = (int64_t)tm * BM;
        const int64_t n0 = (int64_t)tn * BN;
        int32_t begin = e ? s_end[e - 1] : 0;
        const int32_t end = max(begin, s_end[e]);
        begin &= ~(BK - 1);
        const int ksteps = (end - begin) / BK;
        if (ksteps == 0) {
            if (!p.accumulate) zero_tile<OUT_BF16, BM, BN, NT>(p, e, m0, n0, tid);
            continue;
        }

        const uint8_t* Abase = (const uint8_t*)p.A + m0 * T + begin;
        const uint8_t* Bbase = (const uint8_t*)p.B + (int64_t)begin * N + n0;
        const uint8_t* SAbase = p.sfa + (int64_t)(begin / BK) * H;
        const uint8_t* SBbase = p.sfb + (int64_t)(begin / BK) * N;
        const int rows_valid = (int)min<int64_t>(BM, H - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        uint32_t a_voff[8], b_voff[8], sa_voff[4], sb_voff[4];
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int row = min((tid >> 3) + 32 * pp, rows_valid - 1);
            a_voff[pp] = (uint32_t)row * (uint32_t)T + (uint32_t)(tid & 7) * 16u;
        }
        const uint32_t bcol = (uint32_t)min((tid & 15) * 16, cols_valid - 16);
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) b_voff[pp] = (uint32_t)((tid >> 4) + 16 * pp) * (uint32_t)N + bcol;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa_voff[i] = (uint32_t)(m0 + min(wm * 128 + 32 * i + l32, rows_valid - 1));
            sb_voff[i] = (uint32_t)(n0 + min(wn * 128 + 32 * i + l32, cols_valid - 1));
        }

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        i32x4 ra[8], rb[8];
        int sa_n[4], sb_n[4], sa_c[4], sb_c[4];
        auto gload = [&](int s) {
            const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase + (int64_t)s * BK, 0xFFFFFFFFu);
            const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + (int64_t)s * BK * N, 0xFFFFFFFFu);
            const __amdgpu_buffer_rsrc_t rSA = make_rsrc(SAbase + (int64_t)s * H, 0xFFFFFFFFu);
            const __amdgpu_buffer_rsrc_t rSB = make_rsrc(SBbase + (int64_t)s * N, 0xFFFFFFFFu);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) ra[pp] = buffer_load_16B(rA, a_voff[pp]);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) rb[pp] = buffer_load_16B(rB, b_voff[pp]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa_n[i] = buffer_load_u8(rSA, sa_voff[i]);
                sb_n[i] = buffer_load_u8(rSB, sb_voff[i]);
            }
        };
        auto lstore = [&](int buf) {
            lds_char* As = tiles + buf * STAGE;
            lds_char* Bs = As + A_STAGE;
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) lds_store_16B(As, a_lds0 + pp * 4096u, ra[pp]);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) lds_store_16B(Bs, b_lds0 + pp * 4096u, rb[pp]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa_c[i] = sa_n[i];
                sb_c[i] = sb_n[i];
            }
        };
        auto compute = [&](int buf) {
            const lds_char* As = tiles + buf * STAGE;
            const lds_char* Bs = As + A_STAGE;
#pragma unroll
            for (int ks = 0; ks < BK / 64; ++ks) {
                const int q0 = 4 * ks + 2 * lhi;
                const uint32_t c0 = (uint32_t)((q0 ^ a_sw) << 4);
                const uint32_t c1 = (uint32_t)(((q0 + 1) ^ a_sw) << 4);
                i32x8 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4 x = lds_load_16B(As, a_frag_row + i * 4096u + c0);
                    const i32x4 y = lds_load_16B(As, a_frag_row + i * 4096u + c1);
                    const i32x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
                    af[i] = v;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t base = b_frag[j] + ks * 16384u;
                    const i32x2 t0 = lds_read_tr8(Bs, base);
                    const i32x2 t1 = lds_read_tr8(Bs, base + 2048u);
                    const i32x2 t2 = lds_read_tr8(Bs, base + 4096u);
                    const i32x2 t3 = lds_read_tr8(Bs, base + 6144u);
                    const i32x8 v = {t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
                    bf[j] = v;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j][i] = mfma_scale_e4m3_32x32x64(bf[j], af[i], acc[j][i], sb_c[j], sa_c[i]);
            }
        };

        gload(0);
        lstore(0);
        __syncthreads();
        for (int s = 0; s < ksteps; ++s) {
            const int cur = s & 1;
            if (s + 1 < ksteps) gload(s + 1);
            compute(cur);
            if (s + 1 < ksteps) lstore(cur ^ 1);
            __syncthreads();
        }

        store_wave_tile<OUT_BF16>(p, e, m0 + wm * 128, n0 + wn * 128, lane, acc);
    }
}

}  // namespace

hipError_t launch_wgrad_fp8_native(const GroupedParams& p, bool out_bf16, int grid, hipStream_t stream) {
    if (out_bf16)
        hipLaunchKernelGGL(wgrad_fp8_native_kernel<true>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(wgrad_fp8_native_kernel<false>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kgw
