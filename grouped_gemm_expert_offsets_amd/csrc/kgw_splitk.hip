// Split-K second pass (gfx950).  When an expert's token range is cut into
// `split` chunks, the GEMM kernels write each chunk's fp32 partial Wgrad into
// its own slab of the workspace (slab c*E + e, laid out like a dense output);
// this pass forms
//     out[e] (=|+=) ((P_0 + P_1) + P_2) + ... + P_{split-1}
// in chunk order, then applies the output mode once (cuDNN "Grouped GEMM +
// WGrad (Unified)", section "Operation": overwrite, or accumulate onto the
// caller's output; a 16-bit output rounded once, after the add).  In accumulate
// mode an expert without tokens is left untouched, as in the one-pass kernels.
// The output is the dense (E, hidden, n) tensor or, when out_ptrs is given,
// expert e's own (hidden, n) matrix out_ptrs[e] (NULL: skipped).
//
// Roofline: HBM.  Per output element it reads split fp32 partials (and the old
// value when accumulating) and writes one element.  Each thread handles four
// consecutive elements per grid-stride step with 16-byte loads; n is a
// multiple of 8, so a group of four never crosses a row.
#include "kgw_device.h"
#include "kgw_internal.h"

namespace kgw {
namespace {

constexpr int NT = 256;

template <int OUT>
__global__ __launch_bounds__(NT) void splitk_reduce_kernel(const float* ws, const int32_t* offsets, int32_t E,
                                                           int64_t H, int64_t N, int64_t T, int32_t split,
                                                           void* out, void* const* out_ptrs, int32_t accumulate) {
    constexpr int ESIZE = OUT == kOutF32 ? 4 : 2;
    const int64_t slab = H * N;                 // elements per expert
    const int64_t total4 = (int64_t)E * slab / 4;
    const int64_t chunk_stride = (int64_t)E * slab;
    for (int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x; q < total4; q += (int64_t)gridDim.x * NT) {
        const int64_t idx = 4 * q;
        // the expert (a 64-bit division) only where the mode needs it
        const int e = (out_ptrs || accumulate) ? (int)(idx / slab) : 0;
        char* obase;
        if (out_ptrs) {
            obase = (char*)out_ptrs[e];
            if (!obase) continue;
            obase += (idx - (int64_t)e * slab) * ESIZE;
        } else {
            obase = (char*)out + idx * ESIZE;
        }
        if (accumulate) {
            const int64_t b0 = e ? (int64_t)offsets[e - 1] : 0;
            const int64_t e0 = offsets[e];
            const int64_t begin = b0 < 0 ? 0 : (b0 > T ? T : b0);
            const int64_t end = e0 < 0 ? 0 : (e0 > T ? T : e0);
            if (end - begin < kSplitUnit / 2) continue;   // no whole 128-token block: nothing was added
        }
        f32x4 acc = *(const f32x4*)(ws + idx);
        for (int c = 1; c < split; ++c) acc += *(const f32x4*)(ws + (int64_t)c * chunk_stride + idx);
        if constexpr (OUT != kOutF32) {
            i32x2* dst = (i32x2*)obase;
            if (accumulate) {
                const i32x2 old = *dst;
                acc[0] += half_lo<OUT>((uint32_t)old[0]);
                acc[1] += half_hi<OUT>((uint32_t)old[0]);
                acc[2] += half_lo<OUT>((uint32_t)old[1]);
                acc[3] += half_hi<OUT>((uint32_t)old[1]);
            }
            const i32x2 w = {(int)pack_half2<OUT>(acc[0], acc[1]), (int)pack_half2<OUT>(acc[2], acc[3])};
            *dst = w;
        } else {
            f32x4* dst = (f32x4*)obase;
            if (accumulate) acc = *dst + acc;
            *dst = acc;
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const float* ws, const int32_t* offsets, int32_t num_experts, int64_t hidden,
                                int64_t n, int64_t tokens_sum, int32_t split, void* out, void* const* out_ptrs,
                                int out_kind, int32_t accumulate, int num_cus, hipStream_t stream) {
    const int64_t total4 = (int64_t)num_experts * hidden * n / 4;
    int64_t blocks = (total4 + NT - 1) / NT;
    const int64_t cap = (int64_t)num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (out_kind == kOutBf16)
        hipLaunchKernelGGL(splitk_reduce_kernel<kOutBf16>, dim3((unsigned)blocks), dim3(NT), 0, stream, ws, offsets,
                           num_experts, hidden, n, tokens_sum, split, out, out_ptrs, accumulate);
    else if (out_kind == kOutF16)
        hipLaunchKernelGGL(splitk_reduce_kernel<kOutF16>, dim3((unsigned)blocks), dim3(NT), 0, stream, ws, offsets,
                           num_experts, hidden, n, tokens_sum, split, out, out_ptrs, accumulate);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(NT), 0, stream, ws, offsets,
                           num_experts, hidden, n, tokens_sum, split, out, out_ptrs, accumulate);
    return hipGetLastError();
}

}  // namespace kgw
