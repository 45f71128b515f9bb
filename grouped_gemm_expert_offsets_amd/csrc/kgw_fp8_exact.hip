// Persistent K-grouped weight-gradient kernel, OCP e4m3 operands with one UE8M0
// scale per 128 tokens, fp32 accumulation on the bf16 MFMA (gfx950).  This is
// the kernel behind kgw_wgrad_fp8.
//
// Same operation and work decomposition as the bf16 kernel (cuDNN "Grouped GEMM
// + WGrad (Unified)", section "Operation"); the operands are fp8 with per-block
// 1x128 power-of-two scales (llm-infra-atlas "05 Grouped GEMM", section 3),
// the blocks running along the contracted token axis.
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
//   - K step = one scale block of 128 tokens; per K step each lane needs one
//     scale per fragment: sfa[block][m] for its four M blocks and
//     sfb[block][n] for its four N blocks;
//   - A tile 256 x 128 bytes (token-contiguous rows, chunk ^ ((row>>1)&7)):
//     fragments are 8-byte LDS reads;
//   - B tile 128 x 256 bytes (N-contiguous rows, chunk ^ 2*(k&7)): fragments
//     are transposing ds_read_b64_tr_b8 reads, 8 tokens of one column per lane;
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
__global__ __launch_bounds__(NT, 1) void wgrad_fp8_kernel(GroupedParams p) {
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

    // Fragment of K sub-step ks (16 tokens): lane holds tokens 16ks + 8*lhi + 0..7.
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u + (uint32_t)lhi * 8u;
    const int a_sw = (lane >> 1) & 7;
    const int g16 = lane >> 4, i16 = lane & 15;
    uint32_t b_frag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int krow = 8 * (g16 >> 1) + (i16 >> 1);
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
        uint32_t sa_n[4], sb_n[4];
        float fa[4], fb[4];
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
                fa[i] = e8m0_to_f32(sa_n[i]);
                fb[i] = e8m0_to_f32(sb_n[i]);
            }
        };
        auto compute = [&](int buf) {
            const lds_char* As = tiles + buf * STAGE;
            const lds_char* Bs = As + A_STAGE;
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const uint32_t a_chunk = (uint32_t)((ks ^ a_sw) << 4);
                i32x4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = cvt_e4m3x8_bf16(lds_load_8B(As, a_frag_row + i * 4096u + a_chunk), fa[i]);
#pragma unroll
                for (int j = 0; j < 4; ++j) bf[j] = cvt_e4m3x8_bf16(lds_read_tr8(Bs, b_frag[j] + ks * 4096u), fb[j]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] = mfma_bf16_32x32x16(bf[j], af[i], acc[j][i]);
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

hipError_t launch_wgrad_fp8(const GroupedParams& p, bool out_bf16, int grid, hipStream_t stream) {
    if (out_bf16)
        hipLaunchKernelGGL(wgrad_fp8_kernel<true>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(wgrad_fp8_kernel<false>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kgw
