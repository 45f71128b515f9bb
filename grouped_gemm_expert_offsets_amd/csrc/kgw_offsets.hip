// Device-side check of the offsets contract (cuDNN "Grouped GEMM + WGrad
// (Unified)", section "BF16 contract"): the inclusive cumulative counts must be
// non-decreasing, every count a multiple of the alignment, and the last value
// equal to tokens_sum.  One workgroup scans the offsets and writes the first
// offending expert (or -1) to a device word, so the check stays on the stream:
// no copy to the host, no synchronisation, nothing for the caller to allocate
// beyond that word.  The GEMM kernels clamp malformed ranges on their own; this
// is the flag that says it happened.  (Also here: the reset of the bf16 kernel's
// dynamic-schedule counters, another one-workgroup bookkeeping kernel.)
#include "kgw_internal.h"

namespace kgw {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_offsets_kernel(const int32_t* __restrict__ offsets,
                                                                      int32_t num_experts, int64_t tokens_sum,
                                                                      int32_t alignment, int32_t* __restrict__ result) {
    __shared__ int first_bad;
    if (threadIdx.x == 0) first_bad = num_experts;
    __syncthreads();
    int mine = num_experts;
    for (int e = threadIdx.x; e < num_experts; e += kCheckThreads) {
        const int64_t cur = offsets[e];
        const int64_t prev = e ? (int64_t)offsets[e - 1] : 0;
        const int64_t count = cur - prev;
        const bool bad = count < 0 || count % alignment != 0 || (e == num_experts - 1 && cur != tokens_sum);
        if (bad) {
            mine = e;      // experts are visited in increasing order: the first one is this thread's smallest
            break;
        }
    }
    if (mine < num_experts) atomicMin(&first_bad, mine);
    __syncthreads();
    if (threadIdx.x == 0) result[0] = first_bad < num_experts ? first_bad : -1;
}

__global__ void sched_reset_kernel(int32_t* __restrict__ sched) {
    if (threadIdx.x < kSchedWords) sched[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_sched_reset(int32_t* sched, hipStream_t stream) {
    hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(kSchedWords), 0, stream, sched);
    return hipGetLastError();
}

hipError_t launch_check_offsets(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum, int32_t alignment,
                                int32_t* result, hipStream_t stream) {
    hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(kCheckThreads), 0, stream, offsets, num_experts,
                       tokens_sum, alignment, result);
    return hipGetLastError();
}

}  // namespace kgw
