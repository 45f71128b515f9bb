// Host/device launch contract between the C-ABI layer (kgw_host.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kgw {

// Largest expert count the library accepts (the kernels read each expert's
// token range with scalar loads of the offsets; nothing is sized by it).
constexpr int kMaxExperts = 65536;

// Scale layouts of the fp8 operands (the values of kgw_scale_format_t).
//   kScalesU8:       one byte per 128 tokens, (tokens_sum/128, mn) bytes;
//   kScalesPacked:   128-token blocks, four consecutive blocks per int32 word,
//                    (ceil(tokens_sum/512), mn) words, block b in byte b%4 of word b/4;
//   kScalesPacked32: 32-token blocks packed the same way: one word per 128 tokens,
//                    (tokens_sum/128, mn) words.
constexpr int kScalesU8 = 0, kScalesPacked = 1, kScalesPacked32 = 2;

struct GroupedParams {
    const void* A;          // (hidden, tokens_sum), token axis contiguous
    const void* B;          // (tokens_sum, n), row-major
    const uint8_t* sfa;     // fp8 only: UE8M0 scales of A, layout scale_format, mn = hidden
    const uint8_t* sfb;     // fp8 only: UE8M0 scales of B, layout scale_format, mn = n
    const int32_t* offsets; // (num_experts,) inclusive cumulative token counts
    void* out;              // (num_experts, hidden, n) fp32, bf16 or fp16 (when out_ptrs is NULL)
    void* const* out_ptrs;  // or: per-expert (hidden, n) outputs; a NULL entry skips its expert
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
    int32_t scale_format;   // fp8 only: kScalesU8, kScalesPacked or kScalesPacked32
    int32_t ragged;         // bf16 layouts: A and B are per-expert (., n_e) blocks back to back
    int32_t group_m;        // bf16: M tiles per column of the tile order (4 or 8)
    int32_t snake;          // bf16: odd rounds of the persistent stride run the slots in reverse
    int32_t* sched;         // bf16: kSchedWords zeroed counters -> dynamic schedule (NULL: static)
};

// Dynamic schedule of the bf16 kernel: one claim counter per XCD queue, zeroed by
// launch_sched_reset on the launch stream right before the kernel.  Experts run longest
// first (at most kSchedMaxExperts of them, each its own lane of a wave).
constexpr int kSchedWords = 64;              // 256 bytes of the caller's workspace
constexpr int kSchedMaxExperts = 64;

// Scales of the global 128-token block gb in layout FMT: the value for mn
// index i is the byte (kScalesU8, kScalesPacked) or the word of four 32-token
// scales (kScalesPacked32) at base + i * stride, stride 1 or 4 bytes; the first
// `limit` bytes from base are valid, so a buffer range of that size reads zero
// for i >= mn.
struct ScaleSource {
    const uint8_t* base;
    uint32_t limit;
};
template <int FMT>
__device__ __forceinline__ ScaleSource scale_source(const uint8_t* sf, int64_t mn, int64_t gb) {
    if constexpr (FMT == kScalesU8) return {sf + gb * mn, (uint32_t)mn};
    else if constexpr (FMT == kScalesPacked) return {sf + (gb >> 2) * 4 * mn + (gb & 3), (uint32_t)(4 * mn - (gb & 3))};
    else return {sf + gb * 4 * mn, (uint32_t)(4 * mn)};
}

// M-grouped GEMM (forward / dgrad): rows of A grouped along M, each group with
// its own weight.  Field names follow GroupedParams where the output helpers
// share them (`hidden` = rows of the output = M).
struct MGroupedParams {
    const void* A;          // (M, K), K contiguous
    const void* W;          // nt: (E, N, K); nn: (E, K, N)
    const int32_t* offsets; // (E,) inclusive cumulative row counts, or NULL
    const int32_t* m_indices; // (M,) group of every row, or NULL (then offsets)
    void* out;              // (M, N), row-major
    void* const* out_ptrs;  // always NULL (one output matrix)
    int64_t hidden;         // M
    int64_t n;              // N
    int64_t k;              // K, a multiple of 64 (fp8: of 128)
    const uint8_t* sa;      // fp8 only: UE8M0 scales of A, (K/128, M) bytes
    const uint8_t* sw;      // fp8 only: UE8M0 scales of W, (E, K/128, N) bytes
    int32_t num_groups;
    int32_t tiles_m;
    int32_t tiles_n;
    int32_t num_tiles;      // tiles_m * tiles_n
    int32_t num_items;      // 2 * num_tiles: item t < num_tiles is tile t, item num_tiles + t the
                            // second half of tile t when its 128-row halves lie in two groups
    int32_t accumulate;
    int32_t num_xcds;
};

// Group of A row `row` (any value outside [0, num_groups) is no group): the row's
// m_indices entry, else the first group whose inclusive offset exceeds the row
// (num_groups past the last offset).  Uniform across a workgroup.
__device__ __forceinline__ int group_of_row(const MGroupedParams& p, int64_t row) {
    if (p.m_indices) return p.m_indices[row];
    int lo = 0, hi = p.num_groups;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)p.offsets[mid] > row) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// Split-K chunks start on multiples of this many tokens (a multiple of both
// token alignments, so no chunk splits a 128-token fp8 scale block).
constexpr int kSplitUnit = 256;

// Tile shape of the bf16 and fp8 kernels (output tile BM x BN, K step BK).
constexpr int kBf16BM = 256, kBf16BN = 256, kBf16BK = 32;
constexpr int kFp8BM = 256, kFp8BN = 256, kFp8BK = 128;

hipError_t launch_wgrad_bf16(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
// The other operand majors (A M-major and / or B K-major; ragged blocks with both K-major).
hipError_t launch_wgrad_bf16_layout(const GroupedParams& p, bool a_m_major, bool b_k_major, int out_kind, int grid,
                                    hipStream_t stream);
// Split-K second pass: out[e] (=|+=) the sum over c = 0..split-1, in order, of the fp32
// partial slabs ws[c*E + e]; in accumulate mode an expert without tokens is left as is.
hipError_t launch_splitk_reduce(const float* ws, const int32_t* offsets, int32_t num_experts, int64_t hidden,
                                int64_t n, int64_t tokens_sum, int32_t split, void* out, void* const* out_ptrs,
                                int out_kind, int32_t accumulate, int num_cus, hipStream_t stream);
hipError_t launch_wgrad_fp8(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
// Zeroes the kSchedWords counters of the dynamic schedule (a kernel, so graph capture records no memset).
hipError_t launch_sched_reset(int32_t* sched, hipStream_t stream);
hipError_t launch_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                               void* q, void* s, int num_cus, hipStream_t stream);
hipError_t launch_quantize_fp4(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                               void* q, void* s, int num_cus, hipStream_t stream);
hipError_t launch_wgrad_fp8_native(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
hipError_t launch_wgrad_fp4(const GroupedParams& p, int out_kind, int grid, hipStream_t stream);
// First expert whose count breaks the offsets contract, or -1, into result[0] (one workgroup).
hipError_t launch_check_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum, int32_t alignment,
                                int32_t* result, hipStream_t stream);
// Measurement helper: MFMA-only loops on operand data from `src` (see kgw_mfma_ceiling).
hipError_t launch_mfma_ceiling(const void* src, int64_t src_bytes, int32_t kind, int32_t iters, int32_t workgroups,
                               uint64_t* cycles, hipStream_t stream);
hipError_t launch_mgrouped_bf16(const MGroupedParams& p, bool nt, int out_kind, int grid, hipStream_t stream);
// Exact fp8 (U8 scales) in the other operand layouts: A stored (tokens_sum, hidden) when
// a_m_major, B stored (n, tokens_sum) when b_k_major (at least one of them).
hipError_t launch_wgrad_fp8_layout(const GroupedParams& p, bool a_m_major, bool b_k_major, int out_kind, int grid,
                                   hipStream_t stream);
// m-grouped product with fp8 operands and 1x128 UE8M0 scales along K, forward (nt) or dgrad (nn).
hipError_t launch_mgrouped_fp8(const MGroupedParams& p, bool nt, int out_kind, int grid, hipStream_t stream);

}  // namespace kgw
