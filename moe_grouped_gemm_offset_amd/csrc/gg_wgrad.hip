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
// over the XCDs.  A workgroup holds one item in reserve: when a main loop
// ends it asks for the item after the reserve, and one wave looks that up
// (rank table, tile coordinates) at the end of the item and hands it to the
// others through LDS, so that neither the request nor the look-up is
// waited for.  With a bf16 output the reserve's first K unit is issued
// before the output is written, and the next main loop leaves the output
// stores in flight at its first wait, so that they drain under its first
// MFMAs; otherwise the unit loads between the two halves of the output.
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

// OUT: the output format and mode, known at compile time for the common
// cases (the epilogue is then straight-line code): kOutBf16 (bf16,
// overwritten), kOutF32Acc (fp32, accumulated into); kOutAny reads dtype
// and mode at run time.
constexpr int kOutAny = 0, kOutBf16 = 1, kOutF32Acc = 2;

template <class C, bool A_K, bool B_K, int OUT>
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
    const int32_t* ranks = p.ws + kWsHeader / 4;
    int* bcast = (int*)(smem + kWgradBcast);

    const int w = threadIdx.x >> 6;
    const int wm = w / C::WN, wn = w % C::WN;
    const int am0 = uniform(wm * (TM / C::WM)), bn0 = uniform(wn * (TN / C::WN));   // wave offsets in the tile

    constexpr int kHalf = 4 * (C::MB / 2) * (C::NB / 2);   // half of the row walk's items
    constexpr bool kSplit = OUT != kOutAny;
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
    // Item t located: {expert, M tile | N tile << 16, first token, end
    // token} from its rank-table entry, or {-1, ...} past the last item.
    // (Scalar divisions: done by one wave, the others read the result.)
    auto locate = [&](int t) {
        if (t >= total)
            return u32x4{~0u, 0u, 0u, 0u};
        const int rank = t / P;
        const u32x4 ent = scalar_read(reinterpret_cast<const u32x4*>(ranks + 4 * rank));
        int mt_, nt_;
        xcd_remap2d(t - rank * P, tiles_m, tiles_n, p.xcd_gm, mt_, nt_);
        int64_t bg = (int)ent.y;
        int64_t en = (int)ent.z;
        bg = bg < 0 ? 0 : (bg > p.T ? p.T : bg);
        en = en < bg ? bg : (en > p.T ? p.T : en);
        if (((bg | en) & 7) != 0) {       // not expressible in 16-byte chunks
            if (threadIdx.x == 0)
                atomicOr(p.ws, GG_DEVERR_SKIPPED);
            en = bg;
        }
        return u32x4{ent.x, (uint32_t)mt_ | ((uint32_t)nt_ << 16), (uint32_t)bg, (uint32_t)en};
    };
    auto decode = [&](u32x4 loc) {
        e = uniform((int)loc.x);
        const int mn = uniform((int)loc.y);
        m0 = (mn & 0xffff) * TM;
        n0 = (mn >> 16) * TN;
        // token positions come from int32 offsets: kept workgroup-uniform,
        // so that every branch on them is a scalar one
        begin = uniform((int)loc.z);
        end = uniform((int)loc.w);
        const int64_t bg = begin;
        cnt = end - begin;
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
    // bf16 overwrite: transposed accumulators for the bf16-staged epilogue
    auto mma = [&](const FragBf16<C>& f, int m0_, int m1_) {
        mma_bf16<C, OUT == kOutBf16>(f, acc, m0_, m1_);
    };
    FragBf16<C> frag;

    // Static scheduling: workgroup j of the W that serve queue x takes its
    // positions j, j + W, j + 2W, ... without the queue.  W = grid / 8 (the
    // grid is a multiple of 8), or 1 when the grid has fewer than 8
    // workgroups (one per item); W >= 1, so every workgroup's walk ends.
    const int spos0 = blockIdx.x >> 3;
    const int sstep = gridDim.x >= 8 ? (int)(gridDim.x >> 3) : 1;
    if (threadIdx.x == 0)
        *bcast = p.static_sched ? spos0 : atomicAdd(queue, 1);
    __syncthreads();
    const int t0 = 8 * uniform(*bcast) + x;
    if (t0 >= total)
        return;
    decode(locate(t0));
    prefetch();
    // The workgroup holds one item in reserve: the item after the one being
    // computed is asked for and looked up one whole item ahead, so that the
    // queue request and the rank-table read are never waited for.  Wave 0
    // looks it up and hands it to the others through LDS; the barrier that
    // ends each item publishes it.
    int spos = spos0 + sstep;                         // static position of the reserve
    int qpos = 0;
    if (threadIdx.x == 0)
        qpos = p.static_sched ? spos : atomicAdd(queue, 1);
    auto lookup = [&]() {                             // wave 0: qpos -> bcast
        if (uniform(w) == 0) {
            qpos = __builtin_amdgcn_readfirstlane(qpos);
            const u32x4 loc = locate(8 * qpos + x);
            if (threadIdx.x == 0)
                *reinterpret_cast<u32x4*>(bcast) = loc;
        }
    };
    unit_barrier();                   // every wave has read the first item
    lookup();
    wait_all();                       // later items: see the end of the loop
    unit_barrier();
    u32x4 nxt = *reinterpret_cast<const u32x4*>(bcast);
    for (;;) {
        // nothing to add: output untouched (a uniform branch)
        const bool skip = uniform(cnt == 0 && p.accumulate) != 0;
#pragma unroll
        for (int i = 0; i < C::MB; i++)
#pragma unroll
            for (int j = 0; j < C::NB; j++)
                acc[i][j] = f32x16{0};
        const int nk = skip ? 0 : uniform((int)((cnt + 31) / 32));
        pipeline_pp<C, LA::kN, LA::kN + LB::kN, 2 * C::MB * C::NB, C::MB + C::NB, true,
                    OUT == kOutBf16 ? 2 * kHalf : kHalf>(smem, nk, frag, issue2, read2, mma);

        // The new reserve is asked for once this item's main loop is done
        // (asking earlier hands the queue out in start order rather than
        // finish order, which scatters the tiles that share operand panels
        // and measured 20% more HBM fetch).
        spos += sstep;
        if (threadIdx.x == 0)
            qpos = p.static_sched ? spos : atomicAdd(queue, 1);
        __builtin_amdgcn_sched_barrier(0);

        // this item's output
        void* out = p.out_dense
            ? (void*)((char*)p.out_dense +
                      (int64_t)e * p.hidden * p.inter * (p.out_dtype == kF32 ? 4 : 2))
            : (void*)scalar_read(p.out_ptrs + e);
        out = uniform_ptr(out);
        const int accumulate = uniform(cnt > 0 ? p.accumulate : 0);
        const int row0 = m0 + am0, col0 = n0 + bn0;
        float* const stage = (float*)(smem + kWgradEpiBase + w * kEpiHalfBytes);
        // A skipped item runs the same epilogue with every row masked (no
        // access reaches memory), so that no branch goes around its stores.
        const int rows = skip ? 0 : p.hidden;
        // the reserve becomes the next item: its first unit is issued
        const bool more = uniform((int)nxt.x) >= 0;
        auto next_item = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            if (more) {
                decode(nxt);
                prefetch();
            }
        };
        // bf16 output: the next item's first unit is issued before the
        // output, whose 2 kHalf stores the next main loop leaves in flight at
        // its first wait (issued before the stores, the unit lands under
        // them: 2.4% on the MoE shape).  fp32 accumulate: the unit loads
        // between the two halves of the output, after whose loads of the old
        // values, awaited there, only the second half's stores remain in
        // flight.  Run-time format: the unit comes before the output, written
        // in one walk (the registers of the run-time dispatch, twice, would
        // spill inside the main loop).
        if constexpr (OUT == kOutBf16) {
            next_item();
            wgrad_epilogue_bf16t<C, 0>(acc, (char*)stage, out, rows, p.inter, row0, col0);
            wgrad_epilogue_bf16t<C, 1>(acc, (char*)stage, out, rows, p.inter, row0, col0);
        } else if constexpr (kSplit) {
            wgrad_epilogue_t<C, 32, kF32, true, 0, kHalf>(acc, stage, out, rows, p.inter,
                                                          row0, col0);
            next_item();
            wgrad_epilogue_t<C, 32, kF32, true, kHalf, 2 * kHalf>(acc, stage, out, rows,
                                                                  p.inter, row0, col0);
        } else {
            next_item();
            wgrad_epilogue<C, 32>(acc, stage, out, p.out_dtype, rows, p.inter, row0, col0,
                                  accumulate);
        }
        if (!more)
            break;
        lookup();
        // every wave's staging reads are done before slot 2 is loaded again,
        // and the new reserve is published; the stores and the prefetch stay
        // in flight
        lds_wait();
        unit_barrier();
        nxt = *reinterpret_cast<const u32x4*>(bcast);
    }
}

hipError_t launch_wgrad(const WgradArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = WgradCfg;
    const int64_t total = (int64_t)((p.hidden + C::TM - 1) / C::TM) *
                          ((p.inter + C::TN - 1) / C::TN) * p.E;
    if (total == 0)
        return hipSuccess;
    if (total > (1 << 28))              // item numbers and queue positions stay in int32
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)persistent_grid(total)), block(C::kThreads);
    auto go = [&](auto AK, auto BK) {
        constexpr bool ak = decltype(AK)::value, bk = decltype(BK)::value;
        if (info) {
            const int out = p.out_dtype == kBF16 && !p.accumulate ? kOutBf16
                          : p.out_dtype == kF32 && p.accumulate   ? kOutF32Acc
                                                                  : kOutAny;
            snprintf(info->kernel, sizeof(info->kernel),
                     "wgrad_kernel<A %s-major, B %s-major, out %s> (%s scheduling)",
                     ak ? "K" : "M", bk ? "K" : "N",
                     out == kOutBf16 ? "bf16" : out == kOutF32Acc ? "fp32 +=" : "run-time",
                     p.static_sched ? "static" : "dynamic");
            info->tm = C::TM;
            info->tn = C::TN;
            info->waves = C::kWaves;
            info->grid = grid.x;
        }
        if (p.out_dtype == kBF16 && !p.accumulate)
            hipLaunchKernelGGL((wgrad_kernel<C, ak, bk, kOutBf16>), grid, block, 0, s, p);
        else if (p.out_dtype == kF32 && p.accumulate)
            hipLaunchKernelGGL((wgrad_kernel<C, ak, bk, kOutF32Acc>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((wgrad_kernel<C, ak, bk, kOutAny>), grid, block, 0, s, p);
    };
    const std::true_type yes;
    const std::false_type no;
    if (p.a_kmajor && p.b_kmajor)
        go(yes, yes);
    else if (p.a_kmajor)
        go(yes, no);
    else if (p.b_kmajor)
        go(no, yes);
    else
        go(no, no);
    return hipGetLastError();
}

}  // namespace gg
