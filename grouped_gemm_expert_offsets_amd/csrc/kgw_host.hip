// C-ABI layer: argument checks, per-device properties, dispatch to the kernels.
// Declarations and the contract of every entry point are in include/kgw.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>
#include <vector>

#include "../../include/kgw.h"
#include "kgw_device.h"
#include "kgw_internal.h"

// Scratch of kgw_wgrad_bf16_noalloc, for callers that cannot allocate: the split-K
// partials live in this file-scope device array instead of a caller workspace.  Every
// device the library runs on holds its own copy until the process ends; its address on a
// device comes from hipGetSymbolAddress with that device current (in host code the
// array's name is not a device address).  Nothing in it needs to start at zero: every
// partial slab a call reads back was written earlier in the same call.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

struct DeviceProps {
    int num_cus = 0;
    int is_gfx950 = 0;
    int num_xcds = 1;
    bool ok = false;
};

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceProps g_props[kMaxDevices];

kgw_status_t current_props(DeviceProps* out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KGW_ERROR_DEVICE;
    std::call_once(g_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        DeviceProps& d = g_props[dev];
        d.num_cus = prop.multiProcessorCount;
        d.is_gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        // MI355X: 8 XCDs of 32 CUs; workgroups are dispatched round-robin over XCDs.
        d.num_xcds = (d.is_gfx950 && d.num_cus % 8 == 0) ? 8 : 1;
        d.ok = d.num_cus > 0;
    });
    if (!g_props[dev].ok) return KGW_ERROR_DEVICE;
    *out = g_props[dev];
    return KGW_SUCCESS;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch` (NULL if its address could not be obtained).
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

// Checks shared by both entry points; everything here is pure host logic.
kgw_status_t check_common(const void* A, const void* B, const int32_t* offsets, int32_t num_experts,
                          int64_t hidden, int64_t n, int64_t tokens_sum, const void* out, void* const* out_ptrs,
                          int32_t out_dtype, int32_t accumulate, int64_t token_align, int64_t n_align,
                          int64_t bm, int64_t bn) {
    if (num_experts < 1 || hidden < 0 || n < 0 || tokens_sum < 0) return KGW_ERROR_INVALID_VALUE;
    if (out_dtype != KGW_OUT_FP32 && out_dtype != KGW_OUT_BF16 && out_dtype != KGW_OUT_FP16)
        return KGW_ERROR_INVALID_VALUE;
    if (accumulate != 0 && accumulate != 1) return KGW_ERROR_INVALID_VALUE;
    if (!offsets) return KGW_ERROR_INVALID_VALUE;
    const bool has_output = hidden > 0 && n > 0;
    if (out && out_ptrs) return KGW_ERROR_INVALID_VALUE;              // one output form or the other
    if (has_output && !out && !out_ptrs) return KGW_ERROR_INVALID_VALUE;
    if (tokens_sum > 0 && has_output && (!A || !B)) return KGW_ERROR_INVALID_VALUE;
    if (num_experts > kgw::kMaxExperts) return KGW_ERROR_UNSUPPORTED;
    if (tokens_sum > INT32_MAX) return KGW_ERROR_UNSUPPORTED;
    if (hidden >= ((int64_t)1 << 28) || n >= ((int64_t)1 << 28)) return KGW_ERROR_UNSUPPORTED;
    if (tokens_sum % token_align != 0) return KGW_ERROR_BAD_OFFSETS;
    if (n % n_align != 0) return KGW_ERROR_MISALIGNED;
    if (!aligned16(A) || !aligned16(B) || !aligned16(out) || ((uintptr_t)offsets & 3u) ||
        ((uintptr_t)out_ptrs & 7u))
        return KGW_ERROR_MISALIGNED;
    // The kernels address one tile's rows with 32-bit byte offsets.
    if (bm * tokens_sum * 2 >= (int64_t)1 << 32 || 64 * n * 2 >= (int64_t)1 << 31) return KGW_ERROR_UNSUPPORTED;
    const int64_t tiles = ((hidden + bm - 1) / bm) * ((n + bn - 1) / bn);
    if (tiles * (int64_t)num_experts >= INT32_MAX) return KGW_ERROR_UNSUPPORTED;
    return KGW_SUCCESS;
}

enum class Kernel { kBf16, kFp8, kFp8Native, kFp4 };

// Split-K: cut every expert's token range into `split` chunks when the output
// tiles alone would leave most CUs idle (few experts, small hidden x n) and the
// experts hold enough tokens for each chunk to stay busy.  The partials go to
// the workspace as fp32 slabs shaped like the output.
constexpr int64_t kMaxSplit = 16;
constexpr int kDefaultCus = 256;                     // MI355X, when no device is visible
constexpr int64_t kMinChunkTokens = 1024;            // average tokens per chunk
constexpr size_t kMaxSplitWorkspace = (size_t)1 << 30;
constexpr int64_t kShortExpertTokens = 1024;         // bf16 tile order: see run()

struct SplitPlan {
    int32_t split = 1;
    size_t bytes = 0;
};

// Dynamic schedule of the bf16 kernel (claim counters in the workspace, experts longest
// first): for long experts and at least this many rounds of the persistent grid, where
// the static stride leaves CUs unevenly loaded (skewed counts: ~5% modelled).  With only a
// few rounds, which items meet on one CU is a matter of luck either way, and the static
// reversed rounds do as well; short experts are bound by their output stores.
constexpr int64_t kDynMinRounds = 8;

bool dynamic_plan(int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, int num_cus) {
    if (num_experts < 1 || num_experts > kgw::kSchedMaxExperts || hidden <= 0 || n <= 0 || num_cus <= 0) return false;
    if (num_cus % 8 != 0) return false;
    const int64_t items = ((hidden + kgw::kBf16BM - 1) / kgw::kBf16BM) * ((n + kgw::kBf16BN - 1) / kgw::kBf16BN) *
                          num_experts;
    const bool short_experts = tokens_sum < (int64_t)kShortExpertTokens * num_experts;
    return !short_experts && items >= kDynMinRounds * num_cus;
}

SplitPlan split_plan(int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, bool fp8, int num_cus) {
    SplitPlan plan;
    if (num_experts < 1 || hidden <= 0 || n <= 0 || tokens_sum <= 0 || num_cus <= 0) return plan;
    const int64_t bm = fp8 ? kgw::kFp8BM : kgw::kBf16BM;
    const int64_t bn = fp8 ? kgw::kFp8BN : kgw::kBf16BN;
    const int64_t items = ((hidden + bm - 1) / bm) * ((n + bn - 1) / bn) * num_experts;
    if (2 * items > num_cus) return plan;
    int64_t s = num_cus / items;
    if (s > kMaxSplit) s = kMaxSplit;
    const int64_t by_tokens = tokens_sum / ((int64_t)num_experts * kMinChunkTokens);
    if (s > by_tokens) s = by_tokens;
    if (s < 2) return plan;
    const size_t bytes = (size_t)s * (size_t)num_experts * (size_t)hidden * (size_t)n * sizeof(float);
    if (bytes > kMaxSplitWorkspace) return plan;
    plan.split = (int32_t)s;
    plan.bytes = bytes;
    return plan;
}

kgw_status_t run(Kernel kernel, const void* A, const void* sfa, const void* B, const void* sfb,
                 int32_t scale_format, const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                 int64_t tokens_sum, void* out, void* const* out_ptrs, int32_t out_dtype, int32_t accumulate,
                 void* workspace, size_t workspace_bytes, void* stream, int32_t layout = 0) {
    const bool fp8 = kernel != Kernel::kBf16;        // block-scaled operands (fp8 or fp4)
    const bool fp4 = kernel == Kernel::kFp4;
    const int64_t bm = fp8 ? kgw::kFp8BM : kgw::kBf16BM;
    const int64_t bn = fp8 ? kgw::kFp8BN : kgw::kBf16BN;
    const int64_t talign = fp4 ? KGW_FP4_TOKEN_ALIGN : (fp8 ? KGW_FP8_TOKEN_ALIGN : KGW_BF16_TOKEN_ALIGN);
    const int64_t nalign = (fp8 && !fp4) ? 16 : 8;
    static_assert(KGW_OUT_FP32 == kgw::kOutF32 && KGW_OUT_BF16 == kgw::kOutBf16 && KGW_OUT_FP16 == kgw::kOutF16,
                  "output kind codes");
    static_assert(KGW_SCALES_U8 == kgw::kScalesU8 && KGW_SCALES_PACKED == kgw::kScalesPacked &&
                      KGW_SCALES_PACKED_32 == kgw::kScalesPacked32,
                  "scale format codes");
    kgw_status_t st = check_common(A, B, offsets, num_experts, hidden, n, tokens_sum, out, out_ptrs, out_dtype,
                                   accumulate, talign, nalign, bm, bn);
    if (st != KGW_SUCCESS) return st;
    if (fp8 && scale_format != KGW_SCALES_U8 && scale_format != KGW_SCALES_PACKED &&
        scale_format != KGW_SCALES_PACKED_32)
        return KGW_ERROR_INVALID_VALUE;
    if (fp8 && tokens_sum > 0 && hidden > 0 && n > 0 && (!sfa || !sfb)) return KGW_ERROR_INVALID_VALUE;
    if (fp4 && scale_format != KGW_SCALES_PACKED_32) return KGW_ERROR_INVALID_VALUE;
    if (fp8 && scale_format == KGW_SCALES_PACKED_32 && (((uintptr_t)sfa | (uintptr_t)sfb) & 3u))
        return KGW_ERROR_MISALIGNED;
    if (layout & ~(KGW_A_M_MAJOR | KGW_B_K_MAJOR | KGW_RAGGED)) return KGW_ERROR_INVALID_VALUE;
    if ((layout & KGW_RAGGED) && (layout & (KGW_A_M_MAJOR | KGW_B_K_MAJOR)) != KGW_B_K_MAJOR)
        return KGW_ERROR_INVALID_VALUE;      // ragged blocks are K-contiguous for both operands
    if ((layout & KGW_A_M_MAJOR) && hidden % 8 != 0) return KGW_ERROR_MISALIGNED;
    // token rows of an M-major A are addressed with 32-bit offsets, as B's (check_common)
    if ((layout & KGW_A_M_MAJOR) && 64 * hidden * 2 >= ((int64_t)1 << 31)) return KGW_ERROR_UNSUPPORTED;
    // fp8 / fp4: the default layout, or (exact fp8, one byte per 128 tokens) A M-major and / or
    // B K-major, or ragged blocks; A M-major rows of tokens move in 16-byte pieces
    // (hidden % 16) with 32-bit offsets over 64 token rows
    if (fp8 && layout != 0) {
        if (kernel != Kernel::kFp8 || scale_format != KGW_SCALES_U8) return KGW_ERROR_UNSUPPORTED;
        if ((layout & KGW_A_M_MAJOR) && hidden % 16 != 0) return KGW_ERROR_MISALIGNED;
        if ((layout & KGW_A_M_MAJOR) && 64 * hidden >= ((int64_t)1 << 31)) return KGW_ERROR_UNSUPPORTED;
    }
    if (hidden == 0 || n == 0) return KGW_SUCCESS;                 // no output elements
    if (accumulate && tokens_sum == 0) return KGW_SUCCESS;         // adds nothing

    DeviceProps d;
    st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;

    kgw::GroupedParams p;
    p.A = A;
    p.B = B;
    p.sfa = (const uint8_t*)sfa;
    p.sfb = (const uint8_t*)sfb;
    p.scale_format = fp8 ? scale_format : kgw::kScalesU8;
    p.offsets = offsets;
    p.out = out;
    p.out_ptrs = out_ptrs;
    p.ragged = (layout & KGW_RAGGED) ? 1 : 0;
    p.hidden = hidden;
    p.n = n;
    p.tokens_sum = tokens_sum;
    p.num_experts = num_experts;
    p.tiles_m = (int32_t)((hidden + bm - 1) / bm);
    p.tiles_n = (int32_t)((n + bn - 1) / bn);
    p.num_items = p.tiles_m * p.tiles_n * num_experts;
    p.accumulate = accumulate;
    p.num_xcds = d.num_xcds;
    p.split = 1;
    // bf16 tile order: columns of four M tiles, so one XCD's 32 concurrent tiles are a
    // 4 x 8 block; with short experts (under 1024 tokens on average: a few K steps per
    // tile, the output stores dominate) columns of eight.  Measured on one box, one
    // process: E=256 / hidden 7168 / N 2048 / 256 tokens per expert 4.07 -> 3.90 ms with
    // eight, while E=8 / 4096 / 2048 / ~4448 tokens went 0.482 -> 0.494 ms.
    const bool short_experts = tokens_sum < (int64_t)kShortExpertTokens * num_experts;
    p.group_m = short_experts ? 8 : 4;
    // Long experts: odd rounds of the persistent stride take the slots in reverse.  The
    // workgroups that drew the shorter experts in one round draw the longer ones in the
    // next, which evens out the per-CU token sums (balanced E=8: 0.4895 -> 0.4829 ms and
    // 0.4924 -> 0.4847 ms, one box, one process).  With short experts it lost 2.8% on the
    // E=256 workload (stores, not K sums, set its time), so it is off there.
    p.snake = short_experts ? 0 : 1;
    // Short experts, bf16 kernel: no XCD remapping either.  Consecutive tiles then go to
    // different XCDs, which gives up panel sharing in each XCD's L2 (small operands there)
    // for a finer interleave of the output stores: E=256 / 256-token experts 4.02 -> 3.85 ms
    // and 4.01 -> 3.84 ms (one process, two passes), with eight-tile columns still better
    // than four (3.71 vs 3.91 ms).
    if (short_experts && kernel == Kernel::kBf16) p.num_xcds = 1;
    int out_kind = out_dtype;              // KGW_OUT_* values are the kernels' output kinds

    // Split-K when planned and the caller's workspace holds the partials;
    // otherwise one pass (same result up to the order of the fp32 additions).
    const SplitPlan plan = split_plan(num_experts, hidden, n, tokens_sum, fp8, d.num_cus);
    const bool split = plan.split > 1 && workspace && workspace_bytes >= plan.bytes && aligned16(workspace);
    if (split) {
        p.split = plan.split;
        p.num_items *= plan.split;
        p.out = workspace;
        p.out_ptrs = nullptr;
        p.accumulate = 0;
        out_kind = kgw::kOutF32;
    }
    p.sched = nullptr;
    const int grid = p.num_items < d.num_cus ? p.num_items : d.num_cus;
    hipError_t err = hipSuccess;
    if (kernel == Kernel::kBf16 && !split && dynamic_plan(num_experts, hidden, n, tokens_sum, d.num_cus) &&
        workspace && workspace_bytes >= kgw::kSchedWords * sizeof(int32_t) && aligned16(workspace) &&
        grid % d.num_xcds == 0) {
        p.sched = (int32_t*)workspace;
        p.snake = 0;
        err = kgw::launch_sched_reset(p.sched, (hipStream_t)stream);
        if (err != hipSuccess) return KGW_ERROR_DEVICE;
    }
    switch (kernel) {
        case Kernel::kBf16:
            err = layout ? kgw::launch_wgrad_bf16_layout(p, (layout & KGW_A_M_MAJOR) != 0,
                                                         (layout & KGW_B_K_MAJOR) != 0, out_kind, grid,
                                                         (hipStream_t)stream)
                         : kgw::launch_wgrad_bf16(p, out_kind, grid, (hipStream_t)stream);
            break;
        case Kernel::kFp8:
            err = layout ? kgw::launch_wgrad_fp8_layout(p, (layout & KGW_A_M_MAJOR) != 0,
                                                        (layout & KGW_B_K_MAJOR) != 0, out_kind, grid,
                                                        (hipStream_t)stream)
                         : kgw::launch_wgrad_fp8(p, out_kind, grid, (hipStream_t)stream);
            break;
        case Kernel::kFp4: err = kgw::launch_wgrad_fp4(p, out_kind, grid, (hipStream_t)stream); break;
        default: err = kgw::launch_wgrad_fp8_native(p, out_kind, grid, (hipStream_t)stream); break;
    }
    if (err == hipSuccess && split)
        err = kgw::launch_splitk_reduce((const float*)workspace, offsets, num_experts, hidden, n, tokens_sum,
                                        plan.split, out, out_ptrs, out_dtype, accumulate, d.num_cus,
                                        (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

}  // namespace

extern "C" {

kgw_status_t kgw_wgrad_bf16(const void* A, const void* B, const int32_t* offsets, int32_t num_experts,
                            int64_t hidden, int64_t n, int64_t tokens_sum, void* out, int32_t out_dtype,
                            int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream) {
    return run(Kernel::kBf16, A, nullptr, B, nullptr, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum,
               out, nullptr, out_dtype, accumulate, workspace, workspace_bytes, stream);
}

kgw_status_t kgw_wgrad_bf16_noalloc(const void* A, const void* B, const int32_t* offsets, int32_t num_experts,
                                    int64_t hidden, int64_t n, int64_t tokens_sum, void* out, int32_t out_dtype,
                                    int32_t accumulate, void* stream) {
    // Same checks and kernels as kgw_wgrad_bf16; the split-K partials (when the plan splits and
    // they fit) go to this device's scratch, so nothing is allocated.  Checked before the
    // device is touched, like every other argument error.
    DeviceProps d;
    const kgw_status_t st = current_props(&d);
    if (st == KGW_SUCCESS && d.is_gfx950) {
        void* ws = device_scratch();
        if (!ws) return KGW_ERROR_DEVICE;
        return run(Kernel::kBf16, A, nullptr, B, nullptr, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum,
                   out, nullptr, out_dtype, accumulate, ws, kScratchBytes, stream);
    }
    // no usable device: let run() report the argument errors first, then the device error
    return run(Kernel::kBf16, A, nullptr, B, nullptr, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum, out,
               nullptr, out_dtype, accumulate, nullptr, 0, stream);
}

kgw_status_t kgw_wgrad_bf16_ex(const void* A, const void* B, int32_t layout, const int32_t* offsets,
                               int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, void* out,
                               void* const* out_ptrs, int32_t out_dtype, int32_t accumulate, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return run(Kernel::kBf16, A, nullptr, B, nullptr, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum,
               out, out_ptrs, out_dtype, accumulate, workspace, workspace_bytes, stream, layout);
}

kgw_status_t kgw_wgrad_fp8(const void* A, const uint8_t* sfa, const void* B, const uint8_t* sfb,
                           const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                           int64_t tokens_sum, void* out, int32_t out_dtype, int32_t accumulate,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return run(Kernel::kFp8, A, sfa, B, sfb, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum, out,
               nullptr, out_dtype, accumulate, workspace, workspace_bytes, stream);
}

kgw_status_t kgw_wgrad_fp8_native(const void* A, const uint8_t* sfa, const void* B, const uint8_t* sfb,
                                  const int32_t* offsets, int32_t num_experts, int64_t hidden, int64_t n,
                                  int64_t tokens_sum, void* out, int32_t out_dtype, int32_t accumulate,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return run(Kernel::kFp8Native, A, sfa, B, sfb, KGW_SCALES_U8, offsets, num_experts, hidden, n, tokens_sum,
               out, nullptr, out_dtype, accumulate, workspace, workspace_bytes, stream);
}

kgw_status_t kgw_wgrad_fp8_ex(const void* A, const void* sfa, const void* B, const void* sfb, int32_t scale_format,
                              int32_t native, int32_t layout, const int32_t* offsets, int32_t num_experts,
                              int64_t hidden, int64_t n, int64_t tokens_sum, void* out, void* const* out_ptrs,
                              int32_t out_dtype, int32_t accumulate, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (native != 0 && native != 1) return KGW_ERROR_INVALID_VALUE;
    return run(native ? Kernel::kFp8Native : Kernel::kFp8, A, sfa, B, sfb, scale_format, offsets, num_experts,
               hidden, n, tokens_sum, out, out_ptrs, out_dtype, accumulate, workspace, workspace_bytes, stream,
               layout);
}

kgw_status_t kgw_wgrad_fp4(const void* A, const void* sfa, const void* B, const void* sfb, const int32_t* offsets,
                           int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, void* out,
                           void* const* out_ptrs, int32_t out_dtype, int32_t accumulate, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return run(Kernel::kFp4, A, sfa, B, sfb, KGW_SCALES_PACKED_32, offsets, num_experts, hidden, n, tokens_sum, out,
               out_ptrs, out_dtype, accumulate, workspace, workspace_bytes, stream);
}

kgw_status_t kgw_quantize_fp8(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                              void* q, void* scales, void* stream) {
    if (token_axis != 0 && token_axis != 1) return KGW_ERROR_INVALID_VALUE;
    if (scale_format != KGW_SCALES_U8 && scale_format != KGW_SCALES_PACKED && scale_format != KGW_SCALES_PACKED_32)
        return KGW_ERROR_INVALID_VALUE;
    if (rows < 0 || cols < 0) return KGW_ERROR_INVALID_VALUE;
    const int64_t tokens = token_axis ? cols : rows;
    if (tokens % 128 != 0) return KGW_ERROR_INVALID_VALUE;
    if (rows == 0 || cols == 0) return KGW_SUCCESS;
    if (!x || !q || !scales) return KGW_ERROR_INVALID_VALUE;
    if (cols % 8 != 0 || !aligned16(x) || !aligned16(q)) return KGW_ERROR_MISALIGNED;
    if (scale_format == KGW_SCALES_U8 && !token_axis && ((uintptr_t)scales & 7u)) return KGW_ERROR_MISALIGNED;
    if (scale_format == KGW_SCALES_PACKED_32 && !aligned16(scales)) return KGW_ERROR_MISALIGNED;
    if (rows * cols >= ((int64_t)1 << 40)) return KGW_ERROR_UNSUPPORTED;
    DeviceProps d;
    kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    const hipError_t err = kgw::launch_quantize_fp8(x, rows, cols, token_axis, scale_format, q, scales, d.num_cus,
                                                    (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

kgw_status_t kgw_quantize_fp4(const void* x, int64_t rows, int64_t cols, int32_t token_axis, int32_t scale_format,
                              void* q, void* scales, void* stream) {
    if (token_axis != 0 && token_axis != 1) return KGW_ERROR_INVALID_VALUE;
    if (scale_format != KGW_SCALES_U8 && scale_format != KGW_SCALES_PACKED_32) return KGW_ERROR_INVALID_VALUE;
    if (rows < 0 || cols < 0) return KGW_ERROR_INVALID_VALUE;
    const int64_t tokens = token_axis ? cols : rows;
    if (tokens % 128 != 0) return KGW_ERROR_INVALID_VALUE;
    if (rows == 0 || cols == 0) return KGW_SUCCESS;
    if (!x || !q || !scales) return KGW_ERROR_INVALID_VALUE;
    if (cols % 8 != 0 || !aligned16(x) || !aligned16(q)) return KGW_ERROR_MISALIGNED;
    if (scale_format == KGW_SCALES_U8 && !token_axis && ((uintptr_t)scales & 7u)) return KGW_ERROR_MISALIGNED;
    if (scale_format == KGW_SCALES_PACKED_32 && !aligned16(scales)) return KGW_ERROR_MISALIGNED;
    if (rows * cols >= ((int64_t)1 << 40)) return KGW_ERROR_UNSUPPORTED;
    DeviceProps d;
    kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    const hipError_t err = kgw::launch_quantize_fp4(x, rows, cols, token_axis, scale_format, q, scales, d.num_cus,
                                                    (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

kgw_status_t kgw_mgrouped_bf16(const void* A, const void* W, int32_t layout, const int32_t* offsets,
                               const int32_t* m_indices, int32_t num_groups, int64_t m, int64_t k, int64_t n,
                               void* out, int32_t out_dtype, int32_t accumulate, void* stream) {
    if (num_groups < 1 || m < 0 || k < 0 || n < 0) return KGW_ERROR_INVALID_VALUE;
    if (layout != KGW_LAYOUT_NT && layout != KGW_LAYOUT_NN) return KGW_ERROR_INVALID_VALUE;
    if (out_dtype != KGW_OUT_FP32 && out_dtype != KGW_OUT_BF16 && out_dtype != KGW_OUT_FP16)
        return KGW_ERROR_INVALID_VALUE;
    if (accumulate != 0 && accumulate != 1) return KGW_ERROR_INVALID_VALUE;
    if ((offsets != nullptr) == (m_indices != nullptr)) return KGW_ERROR_INVALID_VALUE;
    if (num_groups > kgw::kMaxExperts) return KGW_ERROR_UNSUPPORTED;
    if (m > INT32_MAX || k >= ((int64_t)1 << 22) || n >= ((int64_t)1 << 24)) return KGW_ERROR_UNSUPPORTED;
    if (k % 64 != 0 || n % 8 != 0) return KGW_ERROR_MISALIGNED;
    if (m == 0 || n == 0) return KGW_SUCCESS;
    if (!out || (k > 0 && (!A || !W))) return KGW_ERROR_INVALID_VALUE;
    if (!aligned16(A) || !aligned16(W) || !aligned16(out) || (((uintptr_t)offsets | (uintptr_t)m_indices) & 3u))
        return KGW_ERROR_MISALIGNED;
    if (accumulate && k == 0) return KGW_SUCCESS;
    DeviceProps d;
    kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    kgw::MGroupedParams p;
    p.A = A;
    p.W = W;
    p.sa = nullptr;
    p.sw = nullptr;
    p.offsets = offsets;
    p.m_indices = m_indices;
    p.out = out;
    p.out_ptrs = nullptr;
    p.hidden = m;
    p.n = n;
    p.k = k;
    p.num_groups = num_groups;
    p.tiles_m = (int32_t)((m + 255) / 256);
    p.tiles_n = (int32_t)((n + 255) / 256);
    if (2 * (int64_t)p.tiles_m * p.tiles_n >= INT32_MAX) return KGW_ERROR_UNSUPPORTED;
    p.num_tiles = p.tiles_m * p.tiles_n;
    p.num_items = 2 * p.num_tiles;
    p.accumulate = accumulate;
    p.num_xcds = d.num_xcds;
    const int grid = p.num_items < d.num_cus ? p.num_items : d.num_cus;
    const hipError_t err = kgw::launch_mgrouped_bf16(p, layout == KGW_LAYOUT_NT, out_dtype, grid, (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

kgw_status_t kgw_mgrouped_fp8(const void* A, const uint8_t* sa, const void* W, const uint8_t* sw, int32_t layout,
                              const int32_t* offsets, const int32_t* m_indices, int32_t num_groups, int64_t m,
                              int64_t k, int64_t n, void* out, int32_t out_dtype, int32_t accumulate, void* stream) {
    if (num_groups < 1 || m < 0 || k < 0 || n < 0) return KGW_ERROR_INVALID_VALUE;
    if (layout != KGW_LAYOUT_NT && layout != KGW_LAYOUT_NN) return KGW_ERROR_INVALID_VALUE;
    if (out_dtype != KGW_OUT_FP32 && out_dtype != KGW_OUT_BF16 && out_dtype != KGW_OUT_FP16)
        return KGW_ERROR_INVALID_VALUE;
    if (accumulate != 0 && accumulate != 1) return KGW_ERROR_INVALID_VALUE;
    if ((offsets != nullptr) == (m_indices != nullptr)) return KGW_ERROR_INVALID_VALUE;
    if (num_groups > kgw::kMaxExperts) return KGW_ERROR_UNSUPPORTED;
    if (m > INT32_MAX || k >= ((int64_t)1 << 22) || n >= ((int64_t)1 << 24)) return KGW_ERROR_UNSUPPORTED;
    // nn: W's rows of N values move in 16-byte pieces
    if (k % 128 != 0 || n % (layout == KGW_LAYOUT_NN ? 16 : 8) != 0) return KGW_ERROR_MISALIGNED;
    if (m == 0 || n == 0) return KGW_SUCCESS;
    if (!out || (k > 0 && (!A || !W || !sa || !sw))) return KGW_ERROR_INVALID_VALUE;
    if (!aligned16(A) || !aligned16(W) || !aligned16(out) || (((uintptr_t)offsets | (uintptr_t)m_indices) & 3u))
        return KGW_ERROR_MISALIGNED;
    if (accumulate && k == 0) return KGW_SUCCESS;
    DeviceProps d;
    kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    kgw::MGroupedParams p;
    p.A = A;
    p.W = W;
    p.sa = sa;
    p.sw = sw;
    p.offsets = offsets;
    p.m_indices = m_indices;
    p.out = out;
    p.out_ptrs = nullptr;
    p.hidden = m;
    p.n = n;
    p.k = k;
    p.num_groups = num_groups;
    p.tiles_m = (int32_t)((m + 255) / 256);
    p.tiles_n = (int32_t)((n + 255) / 256);
    if (2 * (int64_t)p.tiles_m * p.tiles_n >= INT32_MAX) return KGW_ERROR_UNSUPPORTED;
    p.num_tiles = p.tiles_m * p.tiles_n;
    p.num_items = 2 * p.num_tiles;
    p.accumulate = accumulate;
    p.num_xcds = d.num_xcds;
    const int grid = p.num_items < d.num_cus ? p.num_items : d.num_cus;
    const hipError_t err = kgw::launch_mgrouped_fp8(p, layout == KGW_LAYOUT_NT, out_dtype, grid, (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

size_t kgw_workspace_bytes(int32_t num_experts, int64_t hidden, int64_t n, int64_t tokens_sum, int32_t fp8) {
    DeviceProps d;
    const int cus = current_props(&d) == KGW_SUCCESS ? d.num_cus : kDefaultCus;
    const size_t split = split_plan(num_experts, hidden, n, tokens_sum, fp8 != 0, cus).bytes;
    if (split) return split;
    if (!fp8 && dynamic_plan(num_experts, hidden, n, tokens_sum, cus)) return kgw::kSchedWords * sizeof(int32_t);
    return 0;
}

kgw_status_t kgw_validate_offsets_host(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                                       int32_t alignment, int32_t* bad_expert) {
    if (bad_expert) *bad_expert = -1;
    if (!offsets || num_experts < 1 || alignment < 1) return KGW_ERROR_INVALID_VALUE;
    int64_t prev = 0;
    for (int32_t e = 0; e < num_experts; ++e) {
        const int64_t cur = offsets[e];
        const int64_t count = cur - prev;
        if (count < 0 || count % alignment != 0) {
            if (bad_expert) *bad_expert = e;
            return KGW_ERROR_BAD_OFFSETS;
        }
        prev = cur;
    }
    if (prev != tokens_sum) {
        if (bad_expert) *bad_expert = num_experts - 1;
        return KGW_ERROR_BAD_OFFSETS;
    }
    return KGW_SUCCESS;
}

kgw_status_t kgw_validate_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                                  int32_t alignment, int32_t* bad_expert, void* stream) {
    if (bad_expert) *bad_expert = -1;
    if (!offsets || num_experts < 1 || alignment < 1) return KGW_ERROR_INVALID_VALUE;
    std::vector<int32_t> host((size_t)num_experts);
    if (hipMemcpyAsync(host.data(), offsets, sizeof(int32_t) * (size_t)num_experts, hipMemcpyDeviceToHost,
                       (hipStream_t)stream) != hipSuccess)
        return KGW_ERROR_DEVICE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KGW_ERROR_DEVICE;
    return kgw_validate_offsets_host(host.data(), num_experts, tokens_sum, alignment, bad_expert);
}

kgw_status_t kgw_check_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                               int32_t alignment, int32_t* result, void* stream) {
    if (!offsets || !result || num_experts < 1 || alignment < 1 || tokens_sum < 0) return KGW_ERROR_INVALID_VALUE;
    if (num_experts > kgw::kMaxExperts) return KGW_ERROR_UNSUPPORTED;
    if (((uintptr_t)offsets | (uintptr_t)result) & 3u) return KGW_ERROR_MISALIGNED;
    DeviceProps d;
    const kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    const hipError_t err = kgw::launch_check_offsets(offsets, num_experts, tokens_sum, alignment, result,
                                                     (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

kgw_status_t kgw_mfma_ceiling(const void* src, int64_t src_bytes, int32_t kind, int32_t iters, int32_t workgroups,
                              uint64_t* cycles, void* stream) {
    if (!src || !cycles || src_bytes < 4096 || kind < 0 || kind > 3 || iters < 1 || iters > 10000000 ||
        workgroups < 1 || workgroups > 65536)
        return KGW_ERROR_INVALID_VALUE;
    if (src_bytes >= ((int64_t)1 << 34)) return KGW_ERROR_UNSUPPORTED;
    if (((uintptr_t)src & 3u) || ((uintptr_t)cycles & 7u)) return KGW_ERROR_MISALIGNED;
    DeviceProps d;
    const kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (!d.is_gfx950) return KGW_ERROR_DEVICE;
    const hipError_t err = kgw::launch_mfma_ceiling(src, src_bytes, kind, iters, workgroups, cycles, (hipStream_t)stream);
    return err == hipSuccess ? KGW_SUCCESS : KGW_ERROR_DEVICE;
}

const char* kgw_status_string(kgw_status_t status) {
    switch (status) {
        case KGW_SUCCESS: return "success";
        case KGW_ERROR_INVALID_VALUE: return "invalid value (null pointer, bad size, dtype or flag)";
        case KGW_ERROR_MISALIGNED: return "misaligned pointer or n not a multiple of the vector width";
        case KGW_ERROR_BAD_OFFSETS: return "malformed or unaligned offsets / tokens_sum";
        case KGW_ERROR_UNSUPPORTED: return "size outside what the kernels support";
        case KGW_ERROR_DEVICE: return "no usable gfx950 device or a HIP error";
    }
    return "unknown status";
}

kgw_status_t kgw_device_info(int32_t* num_cus, int32_t* is_gfx950, int32_t* num_xcds) {
    DeviceProps d;
    kgw_status_t st = current_props(&d);
    if (st != KGW_SUCCESS) return st;
    if (num_cus) *num_cus = d.num_cus;
    if (is_gfx950) *is_gfx950 = d.is_gfx950;
    if (num_xcds) *num_xcds = d.num_xcds;
    return KGW_SUCCESS;
}

}  // extern "C"
