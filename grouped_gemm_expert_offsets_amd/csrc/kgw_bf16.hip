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
// Inside an item (MFMA tile 32x32x16, fp32 accumulation as the page's BF16
// contract requires):
//   - 4 waves, each owning a 128 (M) x 128 (N) quarter of the tile; the MFMA
//     computes the transposed block Wgrad^T so that every lane ends up holding
//     four consecutive N values of one output row (16-byte stores);
//   - K step of 64 tokens; A and B tiles are staged through registers into a
//     double-buffered LDS ring with XOR swizzles (A rows: 16-byte chunk ^
//     ((row>>1)&7); B rows: chunk ^ 4*(k&3)), which keeps both the stores and
//     the fragment reads free of bank conflicts;
//   - A is token-contiguous, so its fragments are plain 16-byte LDS reads; B is
//     N-contiguous, so its fragments come from transposing ds_read_b64_tr_b16.
#include "kgw_device.h"
#include "kgw_internal.h"
#include "kgw_tile_io.h"

namespace kgw {
namespace {

constexpr int BM = kBf16BM, BN = kBf16BN, BK = kBf16BK;
constexpr int NT = 256;
constexpr int A_STAGE = BM * BK * 2;        // 32 KiB: 256 rows x 128 B
constexpr int B_STAGE = BK * BN * 2;        // 32 KiB: 64 rows x 512 B
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int LDS_TILES = 2 * STAGE;        // double buffer
constexpr int GROUP_M = 4;

static_assert(BM == 256 && BN == 256 && BK == 64, "index math below assumes 256x256x64");

template <bool OUT_BF16>
__global__ __launch_bounds__(NT, 1) void wgrad_bf16_kernel(GroupedParams p) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_TILES + kMaxExperts * 4];
    lds_char* tiles = (lds_char*)smem;
    int32_t* s_end = (int32_t*)(smem + LDS_TILES);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int64_t T = p.tokens_sum, H = p.hidden, N = p.n;

    // Clamped offsets: every token range used below lies inside [0, tokens_sum).
    for (int e = tid; e < p.num_experts; e += NT) {
        int64_t v = p.offsets[e];
        v = v < 0 ? 0 : (v > T ? T : v);
        s_end[e] = (int32_t)v;
    }
    __syncthreads();

    // LDS store offsets of this thread's 8 A chunks and 8 B chunks (fixed per thread).
    // A chunk c = tid + 256*pp: row (tid>>3) + 32*pp, chunk tid&7.
    const uint32_t a_lds0 = (uint32_t)(tid >> 3) * 128u + (uint32_t)(((tid & 7) ^ ((tid >> 4) & 7)) << 4);
    // B chunk c = tid + 256*pp: k-row (tid>>5) + 8*pp, chunk tid&31.
    const uint32_t b_lds0 = (uint32_t)(tid >> 5) * 512u + (uint32_t)(((tid & 31) ^ (((tid >> 5) & 3) << 2)) << 4);

    // Fragment read offsets (fixed per lane).
    const int l32 = lane & 31, lhi = lane >> 5;
    const uint32_t a_frag_row = (uint32_t)(wm * 128 + l32) * 128u;
    const int a_sw = (lane >> 1) & 7;
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

        // Global offsets of this thread's chunks, relative to the tile origin at token `begin`.
        const uint16_t* Abase = (const uint16_t*)p.A + m0 * T + begin;
        const uint16_t* Bbase = (const uint16_t*)p.B + (int64_t)begin * N + n0;
        const int rows_valid = (int)min<int64_t>(BM, H - m0);
        const int cols_valid = (int)min<int64_t>(BN, N - n0);
        uint32_t a_voff[8], b_voff[8];
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int row = min((tid >> 3) + 32 * pp, rows_valid - 1);
            a_voff[pp] = (uint32_t)row * (uint32_t)(T * 2) + (uint32_t)(tid & 7) * 16u;
        }
        const uint32_t bcol = (uint32_t)min((tid & 31) * 8, cols_valid - 8) * 2u;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) b_voff[pp] = (uint32_t)((tid >> 5) + 8 * pp) * (uint32_t)(N * 2) + bcol;

        f32x16 acc[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

        i32x4 ra[8], rb[8];
        auto gload = [&](int s) {
            const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase + (int64_t)s * BK, 0xFFFFFFFFu);
            const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + (int64_t)s * BK * N, 0xFFFFFFFFu);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) ra[pp] = buffer_load_16B(rA, a_voff[pp]);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) rb[pp] = buffer_load_16B(rB, b_voff[pp]);
        };
        auto lstore = [&](int buf) {
            lds_char* As = tiles + buf * STAGE;
            lds_char* Bs = As + A_STAGE;
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) lds_store_16B(As, a_lds0 + pp * 4096u, ra[pp]);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) lds_store_16B(Bs, b_lds0 + pp * 4096u, rb[pp]);
        };
        auto compute = [&](int buf) {
            const lds_char* As = tiles + buf * STAGE;
            const lds_char* Bs = As + A_STAGE;
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const uint32_t a_chunk = (uint32_t)(((2 * ks + lhi) ^ a_sw) << 4);
                i32x4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = lds_load_16B(As, a_frag_row + i * 4096u + a_chunk);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const i16x4 lo = lds_read_tr16(Bs, b_frag[j] + ks * 8192u);
                    const i16x4 hi = lds_read_tr16(Bs, b_frag[j] + ks * 8192u + 2048u);
                    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    bf[j] = __builtin_bit_cast(i32x4, v);
                }
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

hipError_t launch_wgrad_bf16(const GroupedParams& p, bool out_bf16, int grid, hipStream_t stream) {
    if (out_bf16)
        hipLaunchKernelGGL(wgrad_bf16_kernel<true>, dim3(grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(wgrad_bf16_kernel<false>, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kgw
