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
// acts as a longest-first greedy scheduler over skewed experts.  Within an
// expert the items are remapped so each XCD owns a band of M tiles.  The
// reduction runs over the expert's tokens, 32 per stage and 64 per load
// unit, through the pipelined main loop of gg_tile.hpp: K-major operands
// are staged in the K
// layout, M-/N-major operands (the natural layouts of X and dY) are staged
// untransposed in the MN layout and transposed by the LDS transpose reads.
#include "gg_wgrad_epi.hpp"
#include "gg_moe.h"

namespace gg {

using WgradCfg = Cfg<256, 256, 4, 2>;
// main loop of gg_tile.hpp: 0 two unit buffers, 1 five slots, 2 five slots
// with the two wave groups in ping-pong
constexpr int kWgradPipe = 2;

template <class C, bool A_K, bool B_K>
__global__ void __launch_bounds__(C::kThreads, 1) wgrad_kernel(WgradArgs p) {
    constexpr int TM = C::TM, TN = C::TN;
    __shared__ __attribute__((aligned(1024))) char smem[kWgradPipe ? Slots5<C>::kLds : C::kLds];

    const int tiles_m = (p.hidden + TM - 1) / TM;
    const int tiles_n = (p.inter + TN - 1) / TN;
    const int P = tiles_m * tiles_n;
    const int rank = uniform(blockIdx.x / P);
    int mt_, nt_;
    xcd_remap2d(blockIdx.x % P, tiles_m, tiles_n, p.xcd_gm, mt_, nt_);
    const int mt = uniform(mt_), nt = uniform(nt_);
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
    const int wm = w / C::WN, wn = w % C::WN;
    const int m0 = mt * TM, n0 = nt * TN;
    const int am0 = uniform(wm * (TM / C::WM)), bn0 = uniform(wn * (TN / C::WN));   // wave offsets in the tile

    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; i++)
#pragma unroll
        for (int j = 0; j < C::NB; j++)
            acc[i][j] = f32x16{0};

    // K-major operands: the expert's slice starts at token `begin` of rows T
    // tokens apart (tensor2d), or is its own (rows, cnt) block stored at
    // element rows * begin (tensor_ragged).  M-/N-major operands hold each
    // token's row contiguously either way.
    const int64_t ldk = (p.ragged ? cnt : p.T) * 2;
    const char* a = (const char*)p.a;
    const char* b = (const char*)p.b;
    const char* ak = a + (p.ragged ? (int64_t)p.hidden * begin : begin) * 2;
    const char* bk = b + (p.ragged ? (int64_t)p.inter * begin : begin) * 2;
    std::conditional_t<A_K, LoadK<C, TM>, LoadMN<C>> la;
    std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>> lb;
    if constexpr (A_K)
        la.init(ldk, p.hidden - m0);
    else
        la.init((int64_t)p.hidden * 2, p.hidden - m0);
    if constexpr (B_K)
        lb.init(ldk, p.inter - n0);
    else
        lb.init((int64_t)p.inter * 2, p.inter - n0);
    using LA = std::conditional_t<A_K, LoadK<C, TM>, LoadMN<C>>;
    using LB = std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>>;
    auto issue2 = [&](uint32_t sa, uint32_t sb, int u, int i) {
        const int64_t k0 = begin + (int64_t)u * 64;
        if (i < LA::kN) {
            if constexpr (A_K)
                la.template issue<true>(sa, ak + (int64_t)m0 * ldk + (int64_t)u * 128, (end - k0) * 2, i);
            else
                la.issue(sa, a + (k0 * p.hidden + m0) * 2, end - k0, i);
        } else {
            if constexpr (B_K)
                lb.template issue<true>(sb, bk + (int64_t)n0 * ldk + (int64_t)u * 128,
                                        (end - k0) * 2, i - LA::kN);
            else
                lb.issue(sb, b + (k0 * p.inter + n0) * 2, end - k0, i - LA::kN);
        }
    };
    auto read2 = [&](const char* sa, const char* sb, int kt, FragBf16<C>& f, int g) {
        read_bf16<C, A_K, B_K>(sa, sb, am0, bn0, kt & 1, f, g);
    };
    auto mma = [&](const FragBf16<C>& f, int m0_, int m1_) { mma_bf16<C>(f, acc, m0_, m1_); };
    FragBf16<C> frag[2];
    const int nk = (int)((cnt + 31) / 32);
    if constexpr (kWgradPipe == 2) {
        pipeline_pp<C, LA::kN, LA::kN + LB::kN, 2 * C::MB * C::NB, C::MB + C::NB>(smem, nk, frag[0],
                                                                                  issue2, read2, mma);
    } else if constexpr (kWgradPipe == 1) {
        pipeline5<C, LA::kN, LA::kN + LB::kN, 2 * C::MB * C::NB, C::MB + C::NB>(smem, nk, frag, issue2,
                                                                                read2, mma);
    } else {
        auto issue = [&](uint32_t st, int u, int i) { issue2(st, st + TM * kRowBytes, u, i); };
        auto read = [&](const char* st, int kt, FragBf16<C>& f, int g) {
            read2(st, st + TM * kRowBytes, kt, f, g);
        };
        pipeline<C, LA::kN + LB::kN, 2 * C::MB * C::NB, C::MB + C::NB>(smem, nk, frag, issue, read, mma);
    }

    void* out = p.out_dense
        ? (void*)((char*)p.out_dense +
                  (int64_t)e * p.hidden * p.inter * (p.out_dtype == kF32 ? 4 : 2))
        : (void*)p.out_ptrs[e];
    out = uniform_ptr(out);
    const int accumulate = cnt > 0 ? p.accumulate : 0;
    wgrad_epilogue<C>(acc, (float*)(smem + w * kEpiWaveBytes), out, p.out_dtype, p.hidden,
                      p.inter, m0 + am0, n0 + bn0, accumulate);
}

hipError_t launch_wgrad(const WgradArgs& p, hipStream_t s) {
    using C = WgradCfg;
    const int tiles = ((p.hidden + C::TM - 1) / C::TM) * ((p.inter + C::TN - 1) / C::TN);
    const dim3 grid((unsigned)(tiles * p.E)), block(C::kThreads);
    if (p.a_kmajor && p.b_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<C, true, true>), grid, block, 0, s, p);
    else if (p.a_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<C, true, false>), grid, block, 0, s, p);
    else if (p.b_kmajor)
        hipLaunchKernelGGL((wgrad_kernel<C, false, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((wgrad_kernel<C, false, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
