// gg_peak.hip -- measurement support, built as its own library (libgg_peak.so)
// and loaded by the benchmark only: the sustained dense MFMA rate of the
// chip, the denominator of "% of the measured MFMA peak" beside the
// published one.
//
// Every wave of a grid that fills the chip issues rounds of four independent
// MFMAs on register operands (no memory traffic inside the loop), bf16
// v_mfma_f32_32x32x16_bf16 or MXFP8 v_mfma_scale_f32_32x32x64_f8f6f4.  Four
// accumulators per wave and two waves per SIMD keep the pipe issuing back
// to back.  The sums are folded into one value per workgroup, stored only
// when it equals an impossible sentinel, so the compiler keeps every MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;             // 8 waves: two per SIMD

__device__ __forceinline__ float fold(const f32x16& c) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++)
        s += c[i];
    return s;
}

__global__ void __launch_bounds__(kThreads) mfma_bf16_probe(int iters, float* out) {
    const float t = (float)(threadIdx.x & 7) * 0.125f;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(t + (float)i);
        b[i] = (__bf16)(t - (float)i);
    }
    f32x16 c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
#pragma unroll 4
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    const float s = fold(c0) + fold(c1) + fold(c2) + fold(c3);
    if (s == -1234.5f)
        out[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kThreads) mfma_mx8_probe(int iters, float* out) {
    const int t = (int)(threadIdx.x & 7);
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = 0x38383838 + t + i;               // E4M3 codes near 1
        b[i] = 0x30303030 + t - i;
    }
    const int sa = 127, sb = 127;               // E8M0 scales 2^0
    f32x16 c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
#pragma unroll 4
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, sa, 0, sb);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, sa, 0, sb);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, sa, 0, sb);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, sa, 0, sb);
    }
    const float s = fold(c0) + fold(c1) + fold(c2) + fold(c3);
    if (s == -1234.5f)
        out[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Queues one probe launch on `stream`: kind 0 bf16, 1 MXFP8; `blocks`
// workgroups of 512 threads, `iters` rounds of four MFMAs per wave; `out`
// holds at least `blocks` floats (never written in practice).  Returns the
// FLOPs the launch performs, or -1 for an invalid argument or launch error.
double gg_peak_mfma(int kind, int blocks, int iters, float* out, void* stream) {
    if ((kind != 0 && kind != 1) || blocks < 1 || iters < 1 || !out)
        return -1.0;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(mfma_bf16_probe, dim3(blocks), dim3(kThreads), 0, s, iters, out);
    else
        hipLaunchKernelGGL(mfma_mx8_probe, dim3(blocks), dim3(kThreads), 0, s, iters, out);
    if (hipGetLastError() != hipSuccess)
        return -1.0;
    const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
    return per * 4.0 * iters * (kThreads / 64) * (double)blocks;
}

}  // extern "C"
