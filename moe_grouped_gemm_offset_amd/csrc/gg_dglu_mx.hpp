// gg_dglu_mx.hpp -- M-grouped block-scaled (MXFP8) dgrad fused with the
// dSwiGLU / dGeGLU / dSiTU-GLU backward on gfx950: the kernel template and
// its launcher per activation and B major, instantiated by
// gg_dglu_mx_inst.hip (one object per pair, compiled in parallel).
//
// For the rows of group g ("Grouped GEMM + dGLU (SM100)", "Block-scaled
// contract / Equations"):
//   R = alpha_g^2 * sum_k deq(A) deq(B_g)   (FP8 values -- E4M3 or E5M2,
//                                            A and B alike -- with one E8M0
//                                            scale per 32 K values of a row)
// followed by the activation backward on X = beta_g C (the BF16 contract's
// dSwiGLU and dGeGLU, or the block-scaled contract's dSiTU-GLU), which
// yields D, dprob and the optional dbias, and by the per-expert amax of the
// input-gradient and gate-gradient halves of D ("Shapes": (L, 2, 1)).  Each
// expert's codes and scales may sit at their own addresses (pointer arrays),
// as well as in one dense (L, N, K) tensor; the codes K-major or N-major
// ("Parameters / Input tensor B (dense mode)": (N, K) per expert with N
// contiguous), the scales (N, K/32) either way.  C may be fp32, bf16, fp16 or
// FP8 codes ("Parameters / Input tensor C"); D is 16/32-bit or FP8 with E8M0
// block scales (step 3).
//
// Design: the tiling of the dsReLU kernel -- the block-scaled main loop of
// gg_mx.hpp with 4 waves of 128x128 accumulators -- followed by the fused
// epilogue of gg_dglu_epi.hpp.
#pragma once
#include "gg_dglu_epi.hpp"
#include "gg_mx.hpp"
#include "gg_moe.h"

namespace gg {

using DgluMxCfg = Cfg<256, 256, 2, 2>;

// CW: bytes per C element (4 fp32, 2 bf16 / fp16, 1 FP8); ACT: 0 dSwiGLU,
// 1 dGeGLU, 2 dSiTU-GLU; QF: D 16/32-bit (0) or FP8 E4M3 (1) / E5M2 (2)
// D_row / D_col with E8M0 scales; BF: C bf16 and, unless QF, D bf16; AB:
// the operands' FP8 format (0 E4M3, 1 E5M2); BK: B's codes K-major (else
// N-major).
template <class C, int CW, int ACT, int QF, bool BF, int AB, bool BK>
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
    // B's tile: row n0 of the expert's (N, K) codes, or column n0 of its
    // (K, N) ones
    const int64_t bt = BK ? (int64_t)n0 * K : n0;
    const char* bg = p.b_dense ? (const char*)p.b_dense + (int64_t)g * p.N * K + bt
                               : (const char*)p.b_ptrs[g] + bt;
    const char* sfb = p.sfb_dense ? (const char*)p.sfb_dense + ((int64_t)g * p.N + n0) * KB
                                  : (const char*)p.sfb_ptrs[g] + (int64_t)n0 * KB;
    mx_mainloop<C, AB, BK>(smem, a, sfa, bg, sfb, K, K, rows_valid, cols_valid, am0, bn0, acc,
                           p.N);

    // C of the items 10 ahead (6 for fp32 C; 8 and 4 with FP8 output) in
    // flight in the epilogue (more spilled registers in the dSwiGLU and
    // dGeGLU kernels)
    constexpr bool W32 = CW == 4;
    dglu_epilogue<C, CW, ACT, true, QF ? (W32 ? 4 : 8) : (W32 ? 6 : 10), QF, BF>(
        p, acc, smem, m0, n0, g, rows_valid, am0, bn0);
}

// Kernel variant for the call's formats: E4M3 operands with any D, E5M2
// operands with FP8 D (the pages pair FP8 operands with FP8 outputs; the
// host rejects the rest); C fp32, bf16 (compile-time with a bf16 D or an
// FP8 one), fp16 / bf16 (run time) or FP8.
template <int ACT, bool BK>
hipError_t launch_dglu_mx_act(const DgluArgs& p, hipStream_t s) {
    using C = DgluMxCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    const int qf = p.d_dtype == kF8 ? 1 : p.d_dtype == kF8E5M2 ? 2 : 0;
    const int cw = p.c_dtype == kF32 ? 4 : (p.c_dtype == kF8 || p.c_dtype == kF8E5M2) ? 1 : 2;
    const bool bf = cw == 2 && p.c_dtype == kBF16 && (qf != 0 || p.d_dtype == kBF16);
    auto go = [&](auto CWc, auto QFc, auto BFc, auto ABc) {
        constexpr int cwc = decltype(CWc)::value, qfc = decltype(QFc)::value;
        constexpr bool bfc = decltype(BFc)::value;
        constexpr int abc = decltype(ABc)::value;
        hipLaunchKernelGGL((dglu_mx_kernel<C, cwc, ACT, qfc, bfc, abc, BK>), grid, block, 0, s, p);
    };
    auto by_c = [&](auto QFc, auto ABc) {
        using I4 = std::integral_constant<int, 4>;
        using I2 = std::integral_constant<int, 2>;
        using I1 = std::integral_constant<int, 1>;
        if (cw == 4)
            go(I4(), QFc, std::false_type(), ABc);
        else if (cw == 1)
            go(I1(), QFc, std::false_type(), ABc);
        else if (bf)
            go(I2(), QFc, std::true_type(), ABc);
        else
            go(I2(), QFc, std::false_type(), ABc);
    };
    using A0 = std::integral_constant<int, 0>;
    using A1 = std::integral_constant<int, 1>;
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    if (p.ab_e5m2) {
        if (qf == 1)
            by_c(Q1(), A1());
        else if (qf == 2)
            by_c(Q2(), A1());
        else
            return hipErrorInvalidValue;             // rejected by the host checks
    } else if (qf == 1) {
        by_c(Q1(), A0());
    } else if (qf == 2) {
        by_c(Q2(), A0());
    } else {
        by_c(Q0(), A0());
    }
    return hipGetLastError();
}

extern template hipError_t launch_dglu_mx_act<0, true>(const DgluArgs&, hipStream_t);
extern template hipError_t launch_dglu_mx_act<1, true>(const DgluArgs&, hipStream_t);
extern template hipError_t launch_dglu_mx_act<2, true>(const DgluArgs&, hipStream_t);
extern template hipError_t launch_dglu_mx_act<0, false>(const DgluArgs&, hipStream_t);
extern template hipError_t launch_dglu_mx_act<1, false>(const DgluArgs&, hipStream_t);
extern template hipError_t launch_dglu_mx_act<2, false>(const DgluArgs&, hipStream_t);

}  // namespace gg
