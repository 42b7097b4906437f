// gg_wgrad_mx.hip -- block-scaled (MXFP8) grouped weight gradient on gfx950.
//
// Computes Wgrad[e] = deq(A)[:, begin:end] @ deq(B)[begin:end, :] for every
// expert ("Grouped GEMM + WGrad (Unified)", "Operation", on the operands of
// its "Block-scaled contract"): FP8 codes (E4M3, or E5M2 for both operands:
// the FP8 formats the dGLU page's data-type table lists) with one E8M0 scale per 32 tokens
// of a row, A (hidden, T) and B stored K-major as (inter, T), so that the
// reduction axis is contiguous in both, as the scaled MFMA consumes it.
// Either operand is a tensor2d (rows T tokens apart) or tensor_ragged (each
// expert's (rows, count) block stored contiguously, blocks in expert order).
//
// Design: the work order of the bf16 wgrad kernel (experts ranked by token
// count on the device, largest first; XCD-banded tiles within an expert) on
// the block-scaled main loop of gg_mx.hpp (4 waves of 128x128
// accumulators), with the wgrad output epilogue of gg_wgrad_epi.hpp.  The
// main loop moves whole load units of 128 tokens, so an expert's token count
// must be a multiple of 128 (the pages require 256): other counts are
// skipped and flagged in the device error word.
#include "gg_mx.hpp"
#include "gg_wgrad_epi.hpp"
#include "gg_moe.h"

namespace gg {

using WgradMxCfg = Cfg<256, 256, 2, 2>;

// AB: the codes' FP8 format (0 E4M3, 1 E5M2).
template <class C, int AB>
__global__ void __launch_bounds__(C::kThreads, 1) wgrad_mx_kernel(WgradArgs p) {
    constexpr int TM = C::TM, TN = C::TN;
    __shared__ __attribute__((aligned(1024))) char smem[ScaleLds<C>::kSmem];

    const int tiles_m = (p.hidden + TM - 1) / TM;
    const int tiles_n = (p.inter + TN - 1) / TN;
    const int P = tiles_m * tiles_n;
    const int rank = uniform(blockIdx.x / P);
    int mt_, nt_;
    xcd_remap2d(blockIdx.x % P, tiles_m, tiles_n, p.xcd_gm, mt_, nt_);
    const int mt = uniform(mt_), nt = uniform(nt_);
    const u32x4 ent = *reinterpret_cast<const u32x4*>(p.ws + kWsHeader / 4 + 4 * rank);
    const int e = uniform((int)ent.x);

    int64_t begin = uniform((int)ent.y);
    int64_t end = uniform((int)ent.z);
    begin = begin < 0 ? 0 : (begin > p.T ? p.T : begin);
    end = end < begin ? begin : (end > p.T ? p.T : end);
    if (((begin | end) & 127) != 0) {     // not whole load units
        if (threadIdx.x == 0)
            atomicOr(p.ws, GG_DEVERR_SKIPPED);
        end = begin;
    }
    const int64_t cnt = end - begin;
    if (cnt == 0 && p.accumulate)
        return;                            // nothing to add: output untouched

    const int w = threadIdx.x >> 6;
    const int wm = w / C::WN, wn = w % C::WN;
    const int m0 = mt * TM, n0 = nt * TN;
    const int am0 = uniform(wm * (TM / C::WM)), bn0 = uniform(wn * (TN / C::WN));

    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; i++)
#pragma unroll
        for (int j = 0; j < C::NB; j++)
            acc[i][j] = f32x16{0};

    // the expert's first token of row 0, and the row pitch, in codes (one
    // byte per value) and in scales (one byte per 32 values)
    const int64_t ld = p.ragged ? cnt : p.T;
    const int64_t a0 = p.ragged ? (int64_t)p.hidden * begin : begin;
    const int64_t b0 = p.ragged ? (int64_t)p.inter * begin : begin;
    const char* a = (const char*)p.a + a0 + (int64_t)m0 * ld;
    const char* b = (const char*)p.b + b0 + (int64_t)n0 * ld;
    const char* sfa = (const char*)p.sfa + (a0 + (int64_t)m0 * ld) / 32;
    const char* sfb = (const char*)p.sfb + (b0 + (int64_t)n0 * ld) / 32;
    if (cnt > 0)
        mx_mainloop<C, AB>(smem, a, sfa, b, sfb, ld, cnt, p.hidden - m0, p.inter - n0, am0, bn0,
                           acc);

    void* out = p.out_dense
        ? (void*)((char*)p.out_dense +
                  (int64_t)e * p.hidden * p.inter * (p.out_dtype == kF32 ? 4 : 2))
        : (void*)p.out_ptrs[e];
    out = uniform_ptr(out);
    const int accumulate = cnt > 0 ? p.accumulate : 0;
    wgrad_epilogue<C>(acc, (float*)(smem + w * kEpiWaveBytes), out, p.out_dtype, p.hidden,
                      p.inter, m0 + am0, n0 + bn0, accumulate);
}

hipError_t launch_wgrad_mx(const WgradArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = WgradMxCfg;
    const int tiles = ((p.hidden + C::TM - 1) / C::TM) * ((p.inter + C::TN - 1) / C::TN);
    if (info) {
        snprintf(info->kernel, sizeof(info->kernel), "wgrad_mx_kernel<A/B %s> (one tile per workgroup)",
                 p.ab_e5m2 ? "e5m2" : "e4m3");
        info->tm = C::TM;
        info->tn = C::TN;
        info->waves = C::kWaves;
        info->grid = (int64_t)tiles * p.E;
    }
    if (p.ab_e5m2)
        hipLaunchKernelGGL((wgrad_mx_kernel<C, 1>), dim3((unsigned)(tiles * p.E)), dim3(C::kThreads),
                           0, s, p);
    else
        hipLaunchKernelGGL((wgrad_mx_kernel<C, 0>), dim3((unsigned)(tiles * p.E)), dim3(C::kThreads),
                           0, s, p);
    return hipGetLastError();
}

}  // namespace gg
