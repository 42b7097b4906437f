// gg_prologue.hip -- per-call set-up and finalisation kernels.
//
// Set-up runs before every grouped GEMM on the same stream: it clears the
// workspace's error word and accumulators (a fill kernel rather than a
// memset node, so that the sequence can be captured into a HIP graph), checks
// the group offsets against the pages' rules (non-decreasing cumulative
// ends, every group a multiple of 256, last end == total / <= rows), and for
// wgrad ranks the experts by token count, largest first, so that the longest
// reductions are dispatched first (a table of (expert, begin, end) by rank),
// and clears the work-queue counters.
#include "gg_internal.hpp"
#include "gg_moe.h"

namespace gg {

constexpr int kPrologueThreads = 1024;

__global__ void __launch_bounds__(kPrologueThreads)
prologue_kernel(const int32_t* __restrict__ offsets, int n, int64_t total, int dgrad,
                int32_t* __restrict__ err, int32_t* __restrict__ order,
                float* __restrict__ clear, int64_t nclear, float* __restrict__ clear2,
                int64_t nclear2) {
    const int t = threadIdx.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + t; i < nclear + nclear2;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nclear)
            clear[i] = 0.0f;
        else
            clear2[i - nclear] = 0.0f;
    }
    if (blockIdx.x != 0)
        return;
    __shared__ int32_t cnt[1024];
    __shared__ int flags;
    if (t == 0)
        flags = 0;
    __syncthreads();
    int f = 0;
    for (int i = t; i < n; i += blockDim.x) {
        int32_t prev = i ? offsets[i - 1] : 0;
        int32_t cur = offsets[i];
        if (cur < prev)
            f |= GG_DEVERR_DECREASING;
        else if ((cur - prev) % 256 != 0)
            f |= GG_DEVERR_GRANULE;
        if (i == n - 1 && (dgrad ? (int64_t)cur > total : (int64_t)cur != total))
            f |= GG_DEVERR_LAST;
        cnt[i] = cur > prev ? cur - prev : 0;
    }
    if (f)
        atomicOr(&flags, f);
    __syncthreads();
    if (t == 0)
        err[0] = flags;
    if (t < 8)
        err[kWsQueue + t] = 0;
    if (order) {
        // rank r's entry: the expert and its raw bounds (offsets[e-1] or 0,
        // offsets[e]), so that a work item needs one 16-byte load to find
        // its token range
        for (int i = t; i < n; i += blockDim.x) {
            int ci = cnt[i], rank = 0;
            for (int j = 0; j < n; j++) {
                int cj = cnt[j];
                rank += (cj > ci) | ((cj == ci) & (j < i));
            }
            order[4 * rank] = i;
            order[4 * rank + 1] = i ? offsets[i - 1] : 0;
            order[4 * rank + 2] = offsets[i];
            order[4 * rank + 3] = 0;
        }
    }
}

hipError_t launch_prologue(const int32_t* offsets, int n, int64_t total, int dgrad,
                           int32_t* err, int32_t* order, float* clear, int64_t nclear,
                           float* clear2, int64_t nclear2, hipStream_t s) {
    int64_t blocks = (nclear + nclear2 + kPrologueThreads * 4 - 1) / (kPrologueThreads * 4);
    if (blocks < 1)
        blocks = 1;
    if (blocks > 256)
        blocks = 256;
    hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)blocks), dim3(kPrologueThreads), 0, s,
                       offsets, n, total, dgrad, err, order, clear, nclear, clear2, nclear2);
    return hipGetLastError();
}

__device__ __forceinline__ uint16_t rne_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ void __launch_bounds__(256)
dbias_finalize_kernel(uint16_t* __restrict__ dbias, const float* __restrict__ acc, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float old = __builtin_bit_cast(float, (uint32_t)dbias[i] << 16);
        dbias[i] = rne_bf16(old + acc[i]);
    }
}

hipError_t launch_dbias_finalize(uint16_t* dbias, const float* acc, int64_t n, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048)
        blocks = 2048;
    if (blocks < 1)
        return hipSuccess;
    hipLaunchKernelGGL(dbias_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dbias, acc, n);
    return hipGetLastError();
}

}  // namespace gg
