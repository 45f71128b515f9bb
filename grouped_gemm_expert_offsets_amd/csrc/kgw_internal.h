// Host/device launch contract between the C-ABI layer (kgw_host.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kgw {

// Largest expert count the library accepts (the kernels read each expert's
// token range with scalar loads of the offsets; nothing is sized by it).
constexpr int kMaxExperts = 65536;

struct GroupedParams {
    const void* A;          // (hidden, tokens_sum), token axis contiguous
    const void* B;          // (tokens_sum, n), row-major
    const uint8_t* sfa;     // fp8 only: (tokens_sum/128, hidden) UE8M0 bytes
    const uint8_t* sfb;     // fp8 only: (tokens_sum/128, n) UE8M0 bytes
    const int32_t* offsets; // (num_experts,) inclusive cumulative token counts
    void* out;              // (num_experts, hidden, n) fp32, bf16 or fp16
    int64_t hidden;
    int64_t n;
    int64_t tokens_sum;
    int32_t num_experts;
    int32_t tiles_m;        // ceil(hidden / BM)
    int32_t tiles_n;        // ceil(n / BN)
    int32_t num_items;      // num_experts * tiles_m * tiles_n
    int32_t accumulate;     // 1: out += W, 0: out = W
    int32_t num_xcds;       // XCD count used to remap workgroup ids
    int32_t split;          // K chunks per expert: 1, or > 1 for split-K partials
};

// Split-K chunks start on multiples of this many tokens (a multiple of both
// token alignments, so no chunk splits a 128-token fp8 scale block).
constexpr int kSplitUnit = 256;

// Tile shape of the bf16 and fp8 kernels (output tile BM x BN, K step BK).
constexpr int kBf16BM = 256, kBf16BN = 256, kBf16BK = 32;
constexpr int kFp8BM = 256, kFp8BN = 256, kFp8BK = 128;

hipError_t launch_wgrad_bf16(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
// Split-K second pass: out[e] (=|+=) the sum over c = 0..split-1, in order, of the fp32
// partial slabs ws[c*E + e]; in accumulate mode an expert without tokens is left as is.
hipError_t launch_splitk_reduce(const float* ws, const int32_t* offsets, int32_t num_experts, int64_t hidden,
                                int64_t n, int64_t tokens_sum, int32_t split, void* out, int out_kind,
                                int32_t accumulate, int num_cus, hipStream_t stream);
hipError_t launch_wgrad_fp8(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
hipError_t launch_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis, void* q,
                               uint8_t* s, int num_cus, hipStream_t stream);
hipError_t launch_wgrad_fp8_native(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);

}  // namespace kgw
