// gg_wgrad.hip -- grouped weight gradient on gfx950.
//
// Computes Wgrad[e] = A[:, begin:end] @ B[begin:end, :] for every expert,
// where [begin, end) is expert e's token slice (begin = offsets[e-1], or 0
// for the first expert; end = offsets[e]), as the "Operation" section of the
// "Grouped GEMM + WGrad (Unified)" page defines it; accumulate or overwrite,
// an empty expert giving zero.
//
// Design: one workgroup per (expert, M tile, N tile) work item.  The grid is
// ordered by the prologue's ranking (largest token count first) so that the
// hardware dispatcher, which starts workgroups in index order as CUs free up,
// acts as a longest-first greedy scheduler over the Zipf-skewed experts.
// Within an expert the items are remapped so each XCD owns a band of M
// tiles.  The reduction runs over the expert's tokens in K steps of 64:
// global loads for step k+1 are issued before the MFMAs of step k, then
// written to the other LDS buffer (one barrier per step).  K-major operands
// are copied chunk-wise; M-/N-major operands (the natural layouts of X and
// dY) are transposed 8x8 in registers on their way to LDS.
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "../../include/gg_moe.h"

namespace gg {

template <int TM, int TN>
struct WgradCfg {
    static constexpr int MB = TM / 64;  // 32-row MFMA blocks per wave (2 waves in M)
    static constexpr int NB = TN / 64;
    static constexpr int kBufBytes = (TM + TN) * kRowBytes;
    static constexpr int kLdsBytes = 2 * kBufBytes;
};

template <int DT, int MB, int NB>
__device__ __forceinline__ void wgrad_epilogue(const f32x16 (&acc)[MB][NB], void* out, int hidden,
                                               int inter, int row0, int col0, int accumulate) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int col = col0 + 32 * j + (l & 31);
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = row0 + 32 * i + acc_row(r, l);
                if (row < hidden && col < inter) {
                    const int64_t idx = (int64_t)row * inter + col;
                    float v = acc[i][j][r];
                    if (accumulate)
                        v += load_elem(out, DT, idx);
                    store_elem(out, DT, idx, v);
                }
            }
        }
}

template <int TM, int TN, bool A_K, bool B_K>
__global__ void __launch_bounds__(kThreads, 1) wgrad_kernel(WgradArgs p) {
    using Cfg = WgradCfg<TM, TN>;
    constexpr int MB = Cfg::MB, NB = Cfg::NB;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];

    const int tiles_m = (p.hidden + TM - 1) / TM;
    const int tiles_n = (p.inter + TN - 1) / TN;
    const int P = tiles_m * tiles_n;
    const int rank = uniform(blockIdx.x / P);
    const int q = uniform(xcd_remap(blockIdx.x % P, P));
    const int mt = uniform(q / tiles_n), nt = uniform(q % tiles_n);
    const int32_t* order = p.ws + kWsHeader / 4;
    const int e = uniform(order[rank]);

    int64_t begin = e ? (int64_t)uniform(p.offsets[e - 1]) : 0;
    int64_t end = uniform(p.offsets[e]);
    begin = begin < 0 ? 0 : (begin > p.T ? p.T : begin);
    end = end < begin ? begin : (end > p.T ? p.T : end);
    if (((begin | end) & 7) != 0) {       // not expressible in 16-byte chunks
        if (threadIdx.x == 0)
            atomicOr(p.ws, GG_DEVERR_SKIPPED);
        end = begin;
    }
    const int64_t cnt = end - begin;
    if (cnt == 0 && p.accumulate)
        return;                            // nothing to add: output untouched

    const int w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int m0 = mt * TM, n0 = nt * TN;

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
            acc[i][j] = f32x16{0};

    const int nk = (int)((cnt + 63) / 64);
    if (nk > 0) {
        const char* a = (const char*)p.a;
        const char* b = (const char*)p.b;
        // A: tile rows are hidden rows; B: tile rows are intermediate columns.
        typename std::conditional<A_K, KLoader<TM>, MNLoader16<TM>>::type la;
        typename std::conditional<B_K, KLoader<TN>, MNLoader16<TN>>::type lb;
        auto load = [&](int kt) {
            const int64_t k0 = begin + (int64_t)kt * 64;
            if constexpr (A_K)
                la.load(a + (int64_t)m0 * p.T * 2, p.T * 2, p.hidden - m0, k0 * 2, end * 2);
            else
                la.load(a + (k0 * p.hidden + m0) * 2, (int64_t)p.hidden * 2, p.hidden - m0, end - k0);
            if constexpr (B_K)
                lb.load(b + (int64_t)n0 * p.T * 2, p.T * 2, p.inter - n0, k0 * 2, end * 2);
            else
                lb.load(b + (k0 * p.inter + n0) * 2, (int64_t)p.inter * 2, p.inter - n0, end - k0);
        };
        load(0);
        la.store(smem);
        lb.store(smem + TM * kRowBytes);
        __syncthreads();
        for (int kt = 0; kt < nk; kt++) {
            char* cur = smem + (kt & 1) * Cfg::kBufBytes;
            char* nxt = smem + ((kt + 1) & 1) * Cfg::kBufBytes;
            const bool more = kt + 1 < nk;
            if (more)
                load(kt + 1);
            mfma_step_bf16<MB, NB>(cur, cur + TM * kRowBytes, wm * (TM / 2), wn * (TN / 2), acc);
            if (more) {
                la.store(nxt);
                lb.store(nxt + TM * kRowBytes);
            }
            __syncthreads();
        }
    }

    void* out = p.out_dense
        ? (void*)((char*)p.out_dense +
                  (int64_t)e * p.hidden * p.inter * (p.out_dtype == kF32 ? 4 : 2))
        : (void*)p.out_ptrs[e];
    const int row0 = m0 + wm * (TM / 2), col0 = n0 + wn * (TN / 2);
    const int accumulate = cnt > 0 ? p.accumulate : 0;
    if (p.out_dtype == kBF16)
        wgrad_epilogue<kBF16>(acc, out, p.hidden, p.inter, row0, col0, accumulate);
    else if (p.out_dtype == kF16)
        wgrad_epilogue<kF16>(acc, out, p.hidden, p.inter, row0, col0, accumulate);
    else
        wgrad_epilogue<kF32>(acc, out, p.hidden, p.inter, row0, col0, accumulate);
}

template <int TM, int TN>
static hipError_t launch_wgrad_t(const WgradArgs& p, hipStream_t s) {
    const int tiles = ((p.hidden + TM - 1) / TM) * ((p.inter + TN - 1) / TN);
    const dim3 grid((unsigned)(tiles * p.E)), block(kThreads);
    if (p.a_kmajor && p.b_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<TM, TN, true, true>), grid, block, 0, s, p);
    else if (p.a_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<TM, TN, true, false>), grid, block, 0, s, p);
    else if (p.b_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<TM, TN, false, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((wgrad_kernel<TM, TN, false, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_wgrad(const WgradArgs& p, hipStream_t s) {
    return launch_wgrad_t<256, 256>(p, s);
}

}  // namespace gg
