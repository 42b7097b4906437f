// gg_dglu.hip -- M-grouped dgrad fused with the dSwiGLU / dGeGLU backward on
// gfx950.
//
// For the rows of group g (padded_offsets[g-1] <= m < padded_offsets[g]):
// R = alpha_g^2 A_g B_g^T, X = beta_g C, and the 32-wide interleaved
// input/gate blocks of X feed the activation backward; D, dprob and dbias are
// produced in the epilogue ("Grouped GEMM + dGLU (SM100)", "BF16 contract /
// Tensors, layouts, and equation").
//
// Design: one workgroup per (M tile, N tile) of the compact R.  Groups are
// multiples of 256 rows, so a 256-row tile never straddles two groups and
// the tile's expert is found by a binary search over padded_offsets.  The
// main loop is the pipelined bf16 loop of gg_tile.hpp (A and K-major B in the
// K layout, N-major discrete B in the MN layout); the epilogue is the fused
// activation backward of gg_dglu_epi.hpp.
#include "gg_dglu_epi.hpp"
#include "gg_moe.h"

namespace gg {

using DgluCfg = Cfg<256, 256, 4, 2>;
// main loop of gg_tile.hpp: 0 two unit buffers, 1 five slots, 2 five slots
// with the two wave groups in ping-pong
constexpr int kDgluPipe = 2;

// W32: C is fp32 (else bf16 / fp16); ACT: 0 dSwiGLU, 1 dGeGLU; BF: C and D
// both bf16; DB: dbias requested; FILT: dGeGLU's value (0) or mask (1)
// filters.  Each combination is its own kernel so the register allocation
// and arithmetic of one epilogue do not burden the others.
template <class C, bool B_K, bool W32, int ACT, bool BF, bool DB, int FILT>
__global__ void __launch_bounds__(C::kThreads, 1) dglu_kernel(DgluArgs p) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    __shared__ __attribute__((aligned(1024))) char smem[kDgluPipe ? Slots5<C>::kLds : C::kLds];

    const int tiles_n = (p.N + TN - 1) / TN;
    const int tiles_m = (int)((p.m_rows + TM - 1) / TM);
    const int P = tiles_m * tiles_n;
    const int q = uniform(xcd_remap(blockIdx.x, P));
    const int mt = uniform(q / tiles_n), nt = uniform(q % tiles_n);

    int64_t valid_m = uniform(p.po[p.L - 1]);
    valid_m = valid_m < 0 ? 0 : (valid_m > p.m_rows ? p.m_rows : valid_m);
    const int64_t m0 = (int64_t)mt * TM;
    if (m0 >= valid_m)
        return;
    const int g = uniform(group_of(p.po, p.L, m0));
    if (g >= p.L)
        return;
    const int n0 = nt * TN;
    const int rows_valid = (int)(valid_m - m0 < TM ? valid_m - m0 : TM);

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int wm = w / C::WN, wn = w % C::WN;
    const int am0 = wm * (TM / C::WM), bn0 = wn * (TN / C::WN);

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
            acc[i][j] = f32x16{0};

    const char* a = (const char*)p.a + m0 * p.K * 2;
    const char* bg = p.b_dense ? (const char*)p.b_dense + (int64_t)g * p.N * p.K * 2
                               : (const char*)p.b_ptrs[g];
    const int64_t lda = (int64_t)p.K * 2;
    LoadK<C, TM> la;
    std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>> lb;
    la.init(lda, rows_valid);
    if constexpr (B_K)
        lb.init(lda, p.N - n0);
    else
        lb.init((int64_t)p.N * 2, p.N - n0);
    using LB = std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>>;
    constexpr int kLA = LoadK<C, TM>::kN;
    auto issue2 = [&](uint32_t sa, uint32_t sb, int u, int i) {
        const int64_t kb = (int64_t)u * 128;
        if (i < kLA) {
            la.template issue<false>(sa, a + kb, lda - kb, i);
        } else {
            if constexpr (B_K)
                lb.template issue<false>(sb, bg + (int64_t)n0 * lda + kb, lda - kb, i - kLA);
            else
                lb.issue(sb, bg + ((int64_t)u * 64 * p.N + n0) * 2, (int64_t)p.K - u * 64, i - kLA);
        }
    };
    auto read2 = [&](const char* sa, const char* sb, int kt, FragBf16<C>& f, int g) {
        read_bf16<C, true, B_K>(sa, sb, am0, bn0, kt & 1, f, g);
    };
    auto mma = [&](const FragBf16<C>& f, int m0_, int m1_) { mma_bf16<C>(f, acc, m0_, m1_); };
    FragBf16<C> frag[2];
    if constexpr (kDgluPipe == 2) {
        pipeline_pp<C, kLA, kLA + LB::kN, 2 * MB * NB, MB + NB>(smem, p.K / 32, frag[0], issue2, read2,
                                                                mma);
    } else if constexpr (kDgluPipe == 1) {
        pipeline5<C, kLA, kLA + LB::kN, 2 * MB * NB, MB + NB>(smem, p.K / 32, frag, issue2, read2, mma);
    } else {
        auto issue = [&](uint32_t st, int u, int i) { issue2(st, st + TM * kRowBytes, u, i); };
        auto read = [&](const char* st, int kt, FragBf16<C>& f, int g) {
            read2(st, st + TM * kRowBytes, kt, f, g);
        };
        pipeline<C, kLA + LB::kN, 2 * MB * NB, MB + NB>(smem, p.K / 32, frag, issue, read, mma);
    }

    // C of the items 6 ahead (3 for fp32 C) in flight in the epilogue: deeper
    // prefetch spilled registers and measured slower
    dglu_epilogue<C, W32 ? 4 : 2, ACT, false, W32 ? 3 : 6, 0, BF, DB, FILT>(p, acc, smem, m0, n0, g,
                                                                       rows_valid, am0, bn0);
}

hipError_t launch_dglu(const DgluArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = DgluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    if (info) {
        static const char* const kAct[] = {"dSwiGLU", "dGeGLU", "dSiTU-GLU"};
        snprintf(info->kernel, sizeof(info->kernel),
                 "dglu_kernel<%s, B %s-major, C %s, D %s%s%s>", kAct[p.act], p.b_kmajor ? "K" : "N",
                 dtype_name(p.c_dtype), dtype_name(p.d_dtype), p.dbias ? ", dbias" : "", p.act == 1 && p.mask_filter ? ", mask filter" : "");
        info->tm = C::TM;
        info->tn = C::TN;
        info->waves = C::kWaves;
        info->grid = tiles;
    }
    auto go_act = [&](auto BK, auto W32, auto BF, auto DB) {
        constexpr bool bk = decltype(BK)::value, w32 = decltype(W32)::value;
        constexpr bool bf = decltype(BF)::value, db = decltype(DB)::value;
        if (p.act == 0)
            hipLaunchKernelGGL((dglu_kernel<C, bk, w32, 0, bf, db, 0>), grid, block, 0, s, p);
        else if (p.mask_filter)
            hipLaunchKernelGGL((dglu_kernel<C, bk, w32, 1, bf, db, 1>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((dglu_kernel<C, bk, w32, 1, bf, db, 0>), grid, block, 0, s, p);
    };
    auto go = [&](auto BK, auto W32, auto BF) {
        if (p.dbias)
            go_act(BK, W32, BF, std::true_type());
        else
            go_act(BK, W32, BF, std::false_type());
    };
    auto go_bk = [&](auto BK) {
        if (p.c_dtype == kF32)
            go(BK, std::true_type(), std::false_type());
        else if (p.c_dtype == kBF16 && p.d_dtype == kBF16)
            go(BK, std::false_type(), std::true_type());
        else
            go(BK, std::false_type(), std::false_type());
    };
    if (p.b_kmajor)
        go_bk(std::true_type());
    else
        go_bk(std::false_type());
    return hipGetLastError();
}

}  // namespace gg
