// gg_dglu_mx.hip -- M-grouped block-scaled (MXFP8) dgrad fused with the
// dSwiGLU / dGeGLU / dSiTU-GLU backward on gfx950.
//
// For the rows of group g ("Grouped GEMM + dGLU (SM100)", "Block-scaled
// contract / Equations"):
//   R = alpha_g^2 * sum_k deq(A) deq(B_g)   (E4M3 values, one E8M0 scale per
//                                            32 K values of a row)
// followed by the activation backward on X = beta_g C (the BF16 contract's
// dSwiGLU and dGeGLU, or the block-scaled contract's dSiTU-GLU), which
// yields D, dprob and the optional dbias, and by the per-expert amax of the
// input-gradient and gate-gradient halves of D ("Shapes": (L, 2, 1)).  Each expert's codes
// and scales may sit at their own addresses (pointer arrays), as well as in
// one dense (L, N, K) tensor.
//
// Design: the tiling of the dsReLU kernel -- the block-scaled main loop of
// gg_mx.hpp with 4 waves of 128x128 accumulators -- followed by the fused
// epilogue of gg_dglu_epi.hpp.
#include "gg_dglu_epi.hpp"
#include "gg_mx.hpp"
#include "gg_moe.h"

namespace gg {

using DgluMxCfg = Cfg<256, 256, 2, 2>;

// W32: C is fp32 (else bf16 / fp16); ACT: 0 dSwiGLU, 1 dGeGLU, 2 dSiTU-GLU;
// Q: FP8 D_row / D_col with E8M0 scales; BF: C bf16 and, unless Q, D bf16.
template <class C, bool W32, int ACT, bool Q, bool BF>
__global__ void __launch_bounds__(C::kThreads, 1) dglu_mx_kernel(DgluArgs p) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    __shared__ __attribute__((aligned(1024))) char smem[ScaleLds<C>::kSmem];

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
    const int cols_valid = p.N - n0;

    const int w = threadIdx.x >> 6;
    const int wm = w / C::WN, wn = w % C::WN;
    const int am0 = wm * (TM / C::WM), bn0 = wn * (TN / C::WN);

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
            acc[i][j] = f32x16{0};

    const int64_t K = p.K, KB = p.K / 32;        // scale bytes per row
    const char* a = (const char*)p.a + m0 * K;
    const char* sfa = (const char*)p.sfa + m0 * KB;
    const char* bg = p.b_dense ? (const char*)p.b_dense + ((int64_t)g * p.N + n0) * K
                               : (const char*)p.b_ptrs[g] + (int64_t)n0 * K;
    const char* sfb = p.sfb_dense ? (const char*)p.sfb_dense + ((int64_t)g * p.N + n0) * KB
                                  : (const char*)p.sfb_ptrs[g] + (int64_t)n0 * KB;
    mx_mainloop<C>(smem, a, sfa, bg, sfb, K, K, rows_valid, cols_valid, am0, bn0, acc);

    // C of the items 10 ahead (6 for fp32 C) in flight in the epilogue (more
    // spilled registers in the dSwiGLU and dGeGLU kernels)
    dglu_epilogue<C, W32, ACT, true, Q ? (W32 ? 4 : 8) : (W32 ? 6 : 10), Q, BF>(
        p, acc, smem, m0, n0, g, rows_valid, am0, bn0);
}

hipError_t launch_dglu_mx(const DgluArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = DgluMxCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    if (info) {
        static const char* const kAct[] = {"dSwiGLU", "dGeGLU", "dSiTU-GLU"};
        snprintf(info->kernel, sizeof(info->kernel), "dglu_mx_kernel<%s, C %s, D %s%s>",
                 kAct[p.act], dtype_name(p.c_dtype), dtype_name(p.d_dtype),
                 p.dbias ? ", dbias" : "");
        info->tm = C::TM;
        info->tn = C::TN;
        info->waves = C::kWaves;
        info->grid = tiles;
    }
    auto go = [&](auto W32, auto Q, auto BF) {
        constexpr bool w32 = decltype(W32)::value, q = decltype(Q)::value;
        constexpr bool bf = decltype(BF)::value;
        if (p.act == 0)
            hipLaunchKernelGGL((dglu_mx_kernel<C, w32, 0, q, bf>), grid, block, 0, s, p);
        else if (p.act == 1)
            hipLaunchKernelGGL((dglu_mx_kernel<C, w32, 1, q, bf>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((dglu_mx_kernel<C, w32, 2, q, bf>), grid, block, 0, s, p);
    };
    const std::false_type no;
    const std::true_type yes;
    const bool w32 = p.c_dtype == kF32;
    if (p.d_dtype == kF8)
        w32 ? go(yes, yes, no) : (p.c_dtype == kBF16 ? go(no, yes, yes) : go(no, yes, no));
    else if (w32)
        go(yes, no, no);
    else if (p.c_dtype == kBF16 && p.d_dtype == kBF16)
        go(no, no, yes);
    else
        go(no, no, no);
    return hipGetLastError();
}

}  // namespace gg
