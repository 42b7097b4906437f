// gg_wgrad.hip -- grouped weight gradient on gfx950.
//
// Computes Wgrad[e] = A[:, begin:end] @ B[begin:end, :] for every expert,
// where [begin, end) is expert e's token slice (begin = offsets[e-1], or 0
// for the first expert; end = offsets[e]), as the "Operation" section of the
// "Grouped GEMM + WGrad (Unified)" page defines it; accumulate or overwrite,
// an empty expert giving zero.
//
// Design: a persistent kernel, one workgroup per CU, over the (expert, M
// tile, N tile) work items.  Items are numbered expert rank-major (the
// prologue ranks the experts by token count, largest first) and, within an
// expert, remapped so that each XCD owns one block of the expert's tile grid
// (xcd_remap2d): item t belongs to XCD t % 8.  Each XCD has a work queue --
// an atomic counter in the workspace, cleared by the set-up kernel -- over
// its items, and the workgroups dispatched to that XCD (blockIdx % 8, the
// dispatcher's round-robin order) take items from it in order: a
// longest-first greedy schedule per XCD, with every expert spread evenly
// over the XCDs.  A workgroup asks for its next item when its main loop
// ends, and loads the next item's first K unit while it writes the current
// one's output, so that the fill of the next main loop overlaps the
// epilogue.
//
// The reduction runs over the expert's tokens, 32 per stage and 64 per load
// unit, through the ping-pong main loop of gg_tile.hpp: K-major operands are
// staged in the K layout, M-/N-major operands (the natural layouts of X and
// dY) untransposed in the MN layout and transposed by the LDS transpose
// reads.
#include <hip/hip_runtime.h>

#include "gg_wgrad_epi.hpp"
#include "gg_moe.h"

namespace gg {

using WgradCfg = Cfg<256, 256, 4, 2>;

// LDS: five 32 KiB slots for the main loop.  After it, the next item's first
// unit is loaded into slots 0 and 1 while the epilogue stages its output
// through 32-row pieces in slots 2 .. 4; the last word broadcasts the next
// item's queue position.
constexpr int kWgradEpiBase = 2 * Slots5<WgradCfg>::kSlot;
constexpr int kWgradBcast = Slots5<WgradCfg>::kLds - 16;
static_assert(kWgradEpiBase + WgradCfg::kWaves * kEpiHalfBytes <= kWgradBcast,
              "epilogue staging must leave slots 0, 1 and the broadcast word alone");

template <class C, bool A_K, bool B_K>
__global__ void __launch_bounds__(C::kThreads, 1) wgrad_kernel(WgradArgs p) {
    constexpr int TM = C::TM, TN = C::TN;
    constexpr int kSlot = Slots5<C>::kSlot;
    __shared__ __attribute__((aligned(1024))) char smem[Slots5<C>::kLds];

    const int tiles_m = (p.hidden + TM - 1) / TM;
    const int tiles_n = (p.inter + TN - 1) / TN;
    const int P = tiles_m * tiles_n;
    const int total = P * p.E;
    const int x = blockIdx.x & 7;                       // this workgroup's queue
    int32_t* queue = p.ws + kWsQueue + x;
    const int32_t* order = p.ws + kWsHeader / 4;
    int* bcast = (int*)(smem + kWgradBcast);

    const int w = threadIdx.x >> 6;
    const int wm = w / C::WN, wn = w % C::WN;
    const int am0 = uniform(wm * (TM / C::WM)), bn0 = uniform(wn * (TN / C::WN));   // wave offsets in the tile

    using LA = std::conditional_t<A_K, LoadK<C, TM>, LoadMN<C>>;
    using LB = std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>>;
    LA la;
    LB lb;
    const char* a = (const char*)p.a;
    const char* b = (const char*)p.b;

    // State of the item being loaded.  K-major operands: the expert's slice
    // starts at token `begin` of rows T tokens apart (tensor2d), or is its
    // own (rows, cnt) block stored at element rows * begin (tensor_ragged).
    // M-/N-major operands hold each token's row contiguously either way.
    int e = 0, m0 = 0, n0 = 0;
    int64_t begin = 0, end = 0, cnt = 0, ldk = 0;
    const char* ak = a;
    const char* bk = b;
    auto decode = [&](int t) {
        const int rank = uniform(t / P);
        int mt_, nt_;
        xcd_remap2d(t % P, tiles_m, tiles_n, p.xcd_gm, mt_, nt_);
        m0 = uniform(mt_) * TM;
        n0 = uniform(nt_) * TN;
        e = uniform(order[rank]);
        int64_t bg = e ? (int64_t)uniform(p.offsets[e - 1]) : 0;
        int64_t en = uniform(p.offsets[e]);
        bg = bg < 0 ? 0 : (bg > p.T ? p.T : bg);
        en = en < bg ? bg : (en > p.T ? p.T : en);
        if (((bg | en) & 7) != 0) {       // not expressible in 16-byte chunks
            if (threadIdx.x == 0)
                atomicOr(p.ws, GG_DEVERR_SKIPPED);
            en = bg;
        }
        begin = bg;
        end = en;
        cnt = en - bg;
        ldk = (p.ragged ? cnt : p.T) * 2;
        ak = a + (p.ragged ? (int64_t)p.hidden * bg : bg) * 2;
        bk = b + (p.ragged ? (int64_t)p.inter * bg : bg) * 2;
        if constexpr (A_K)
            la.init(ldk, p.hidden - m0);
        else
            la.init((int64_t)p.hidden * 2, p.hidden - m0);
        if constexpr (B_K)
            lb.init(ldk, p.inter - n0);
        else
            lb.init((int64_t)p.inter * 2, p.inter - n0);
    };
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
    const uint32_t lds0 = lds_addr(smem);
    auto prefetch = [&]() {                             // unit 0 into slots 0 and 1
#pragma unroll
        for (int i = 0; i < LA::kN + LB::kN; i++)
            issue2(lds0, lds0 + kSlot, 0, i);
    };
    auto read2 = [&](const char* sa, const char* sb, int kt, FragBf16<C>& f, int g) {
        read_bf16<C, A_K, B_K>(sa, sb, am0, bn0, kt & 1, f, g);
    };
    f32x16 acc[C::MB][C::NB];
    auto mma = [&](const FragBf16<C>& f, int m0_, int m1_) { mma_bf16<C>(f, acc, m0_, m1_); };
    FragBf16<C> frag;

    if (threadIdx.x == 0)
        *bcast = atomicAdd(queue, 1);
    __syncthreads();
    const int t0 = 8 * uniform(*bcast) + x;
    if (t0 >= total)
        return;
    decode(t0);
    prefetch();
    for (;;) {
        const bool skip = cnt == 0 && p.accumulate;     // nothing to add: output untouched
#pragma unroll
        for (int i = 0; i < C::MB; i++)
#pragma unroll
            for (int j = 0; j < C::NB; j++)
                acc[i][j] = f32x16{0};
        const int nk = skip ? 0 : (int)((cnt + 31) / 32);
        pipeline_pp<C, LA::kN, LA::kN + LB::kN, 2 * C::MB * C::NB, C::MB + C::NB, true>(
            smem, nk, frag, issue2, read2, mma);

        // this item's output
        void* out = p.out_dense
            ? (void*)((char*)p.out_dense +
                      (int64_t)e * p.hidden * p.inter * (p.out_dtype == kF32 ? 4 : 2))
            : (void*)p.out_ptrs[e];
        out = uniform_ptr(out);
        const int accumulate = cnt > 0 ? p.accumulate : 0;
        const int row0 = m0 + am0, col0 = n0 + bn0;

        // the next item, asked for once this one's main loop is done (asking
        // earlier hands the queue out in start order rather than finish
        // order, which scatters the tiles that share operand panels and
        // measured 20% more HBM fetch); its first unit loads while this
        // one's output is written
        if (threadIdx.x == 0)
            *bcast = atomicAdd(queue, 1);
        __syncthreads();
        const int tn = 8 * uniform(*bcast) + x;
        if (tn < total) {
            decode(tn);
            prefetch();
        }
        if (!skip)
            wgrad_epilogue<C, 32>(acc, (float*)(smem + kWgradEpiBase + w * kEpiHalfBytes), out,
                                  p.out_dtype, p.hidden, p.inter, row0, col0, accumulate);
        if (tn >= total)
            break;
        // every wave's staging reads are done before slot 2 is loaded again;
        // the stores and the prefetch stay in flight
        lds_wait();
        unit_barrier();
    }
}

hipError_t launch_wgrad(const WgradArgs& p, hipStream_t s) {
    using C = WgradCfg;
    const int64_t total = (int64_t)((p.hidden + C::TM - 1) / C::TM) *
                          ((p.inter + C::TN - 1) / C::TN) * p.E;
    if (total == 0)
        return hipSuccess;
    if (total > (1 << 28))              // item numbers and queue positions stay in int32
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)persistent_grid(total)), block(C::kThreads);
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
