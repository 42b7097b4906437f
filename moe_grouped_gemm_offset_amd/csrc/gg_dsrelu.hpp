// gg_dsrelu.hpp -- M-grouped block-scaled (MXFP8) dgrad fused with the
// dsReLU backward on gfx950: the kernel template and its launcher per B
// major, instantiated by gg_dsrelu_inst.hip (one object per major).
//
// For the rows of group g ("Grouped GEMM + dsReLU (SM100)", "Equations"):
//   G = alpha_g * sum_k deq(A) deq(B_g)   (FP8 values -- E4M3 or E5M2, A and
//                                          B alike -- with one E8M0 scale per
//                                          32 K values of a row; B_g K-major
//                                          or, as the page's "Layouts" allow
//                                          for FP8, N-major)
//   D_row = prob * 2 * C * relu(G),  dprob = sum_n C relu(G)^2,
// and the per-expert Amax of |D_row| ("Shapes").
//
// Design: the M-grouped tiling of the dGLU kernel on the block-scaled main
// loop of gg_mx.hpp (4 waves of 128x128 accumulators: the fp8 MFMA consumes
// operands twice as fast as the bf16 one, so a wave needs the larger
// footprint to amortise its fragment reads).  The epilogue applies alpha,
// relu, prob and C in registers, reduces dprob across lanes (one atomic per
// row and wave) and Amax across the wave (one atomicMax on the fp32 bit
// pattern, which orders like the value because |D| >= 0).
#pragma once
#include "gg_internal.hpp"
#include "gg_fp8out.hpp"
#include "gg_mx.hpp"
#include "gg_moe.h"

namespace gg {

using DsreluCfg = Cfg<256, 256, 2, 2>;

// QF: FP8 D_row / D_col with E8M0 scales (1 E4M3, 2 E5M2; else a 16/32-bit
// D_row, 0); BF: C bf16 and, unless QF, D bf16, known at compile time
// (otherwise C's width -- fp32, 16-bit, FP8 -- is a run-time choice among
// three epilogue walks); AB: the operands' FP8 format (0 E4M3, 1 E5M2); BK:
// B's codes K-major (else N-major: (K, N) per expert, N contiguous).
template <class C, int QF, bool BF, int AB, bool BK>
__global__ void __launch_bounds__(C::kThreads, 1) dsrelu_kernel(DsreluArgs p) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    constexpr bool Q = QF != 0, BF8 = QF == 2;
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

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
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

    // ---------------- epilogue ----------------
    // Rows of 8 columns per lane: C and D are 16-byte accesses (32 for fp32).
    // C (and, off the bf16 path, prob) of the items 24 ahead (12 for fp32 C)
    // are in flight while an item is processed.  Per element: r = relu(alpha
    // G), t = C r, D = 2 prob t, row sum += t r.
    const float al = p.alpha[g];
    const int64_t N = p.N;
    float amax = 0.0f;
    constexpr int kT = 4 * MB;                     // row walk steps per lane
    float rowsum[kT];
#pragma unroll
    for (int t = 0; t < kT; t++)
        rowsum[t] = 0.0f;
    float* const elds = (float*)(smem + w * kEpiWaveBytes);
    const float nc = Q ? *p.q.norm_const : 1.0f;
    const int cdt = BF ? kBF16 : p.c_dtype, ddt = BF ? kBF16 : p.d_dtype;
    float dcol[4][8];                              // Q: a column block's 4 items
    auto epilogue = [&](auto CWc) {
        constexpr int cw = decltype(CWc)::value;
        using Pre = Pre8<cw, 1>;
        auto load = [&](int, int r, int c) {
            const int rr = am0 + r, col = n0 + bn0 + c;
            const bool ok = (rr < rows_valid) & (col < p.N);
            const int64_t row = m0 + (ok ? rr : 0);
            Pre pre;
            pre.x[0] = rawc_load<cw>(p.c, row * N + (ok ? col : 0));
            pre.row = p.prob[row];
            return pre;
        };
        auto fn = [&](int t, int r, int c, float (&v)[8], const Pre& pre) {
            const int rr = am0 + r;
            const int col = n0 + bn0 + c;
            if constexpr (Q) {
                // every lane computes (the block reductions shuffle across
                // lanes); lanes off the tile contribute zeros
                const bool ok = (rr < rows_valid) & (col < p.N);
                float d[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
                if (ok) {
                    float cv[8];
                    rawc_cvt<cw>(pre.x[0], cdt, cv);
                    const float pr2 = pre.row * 2.0f;
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        const float rl = fmaxf(al * v[k], 0.0f), cr = cv[k] * rl;
                        d[k] = pr2 * cr;
                        rowsum[t] = fmaf(cr, rl, rowsum[t]);
                        amax = fmaxf(amax, fabsf(d[k]));
                    }
                }
#pragma unroll
                for (int k = 0; k < 8; k++)
                    dcol[t & 3][k] = d[k];
                int e;
                const uint2 codes = fp8_row8<BF8>(d, nc, e);
                if (ok)
                    fp8_store_row(p.q, m0 + rr, col, codes, e);
                if ((t & 3) == 3 && p.q.d_col) {
                    const int r0 = r - 24;             // this lane's row of item t-3
                    fp8_col_block<BF8>(p.q, nc, dcol, m0 + am0 + (r0 & ~31), m0 + am0 + r0, col,
                                  col < p.N, rows_valid - (am0 + r0));
                }
            } else if (rr < rows_valid && col < p.N) {
                const int64_t row = m0 + rr;
                float cv[8], d[8];
                rawc_cvt<cw>(pre.x[0], cdt, cv);
                const float pr2 = pre.row * 2.0f;
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const float rl = fmaxf(al * v[k], 0.0f), cr = cv[k] * rl;
                    d[k] = pr2 * cr;
                    rowsum[t] = fmaf(cr, rl, rowsum[t]);
                    amax = fmaxf(amax, fabsf(d[k]));
                }
                store8(p.d, ddt, row * N + col, d);
            }
        };
        for_each_row8<C, Q ? (cw == 4 ? 6 : 12) : (cw == 4 ? 12 : 24)>(acc, elds, load, fn);
    };
    if constexpr (BF && !Q) {
        // bf16 C and D through buffer descriptors over the wave's rows: 32-bit
        // offsets from the wave's first row, record counts that end at its
        // last valid row, columns past N at an invalid offset.  Masked
        // accesses load zeros and store nothing, and zeros add nothing to
        // dprob or amax, so an item needs no test of its own; prob is loaded
        // once per row.
        constexpr int kWaveRows = TM / C::WM;
        const int rows_left = rows_valid - am0 < 0 ? 0
                            : (rows_valid - am0 > kWaveRows ? kWaveRows : rows_valid - am0);
        const int64_t wrow0 = m0 + am0;
        const uint32_t rowb = (uint32_t)(N * 2);             // bytes per row of C and D
        const uint32_t rec = (uint32_t)uniform((int)((uint32_t)rows_left * rowb));
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(uniform_ptr((const char*)p.c + wrow0 * (int64_t)rowb), rec);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(uniform_ptr((char*)p.d + wrow0 * (int64_t)rowb), rec);
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(uniform_ptr(p.prob + wrow0), (uint32_t)uniform(rows_left * 4));
        float pr2[kT];                                   // 2 prob of the lane's rows
#pragma unroll
        for (int t = 0; t < kT; t++)
            pr2[t] = 2.0f * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          rp, (uint32_t)((l >> 3) + 8 * t) * 4, 0, 0));
        auto colb = [&](int c) -> uint32_t {
            const int col = n0 + bn0 + c;
            return col < p.N ? (uint32_t)col * 2 : kInvalid;
        };
        auto loadb = [&](int, int r, int c) {
            return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rc, (uint32_t)r * rowb + colb(c), 0, 0));
        };
        auto fnb = [&](int t, int r, int c, float (&v)[8], const u32x4& x) {
            // (a uniform branch: without one per item the compiler
            // interleaves the unrolled items and spills)
            if (uniform(rows_left) > 0) {
                float cv[8], d[8];
                unpack8_16(x, kBF16, cv);
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const float rl = fmaxf(al * v[k], 0.0f), cr = cv[k] * rl;
                    d[k] = pr2[t] * cr;
                    rowsum[t] = fmaf(cr, rl, rowsum[t]);
                    amax = fmaxf(amax, fabsf(d[k]));
                }
                store_bf16x8(rd, (uint32_t)r * rowb + colb(c), d);
            }
        };
        for_each_row8<C, 24, 64, 0, -1, true>(acc, elds, loadb, fnb);
    } else if constexpr (BF) {
        epilogue(std::integral_constant<int, 2>());
    } else {
        if (p.c_dtype == kF32)
            epilogue(std::integral_constant<int, 4>());
        else if (p.c_dtype == kF8 || p.c_dtype == kF8E5M2)
            epilogue(std::integral_constant<int, 1>());
        else
            epilogue(std::integral_constant<int, 2>());
    }
    // dprob: the 8 lanes of a row hold its partial sums; one atomic per row
    // and wave
#pragma unroll
    for (int t = 0; t < kT; t++) {
        const float v = row8_sum(rowsum[t]);
        const int rr = am0 + (l >> 3) + 8 * t;
        if ((l & 7) == 4 && rr < rows_valid && n0 + bn0 < p.N)
            atomicAdd(p.dprob + m0 + rr, v);
    }
    if (p.amax) {
        amax = wave_max(amax);
        if (l == 0)
            atomicMax((int*)p.amax + g, __float_as_int(amax));
    }
}

// Kernel variant for the call's formats and the B major BK: E4M3 operands
// with any D, E5M2 operands with FP8 D (the host rejects the rest); C bf16
// at compile time with a bf16 or FP8 D, else C's width at run time.
template <bool BK>
hipError_t launch_dsrelu_bk(const DsreluArgs& p, hipStream_t s) {
    using C = DsreluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    const int qf = p.d_dtype == kF8 ? 1 : p.d_dtype == kF8E5M2 ? 2 : 0;
    const bool bf = p.c_dtype == kBF16 && (qf != 0 || p.d_dtype == kBF16);
    auto go = [&](auto QFc, auto ABc) {
        constexpr int qfc = decltype(QFc)::value, abc = decltype(ABc)::value;
        if (bf)
            hipLaunchKernelGGL((dsrelu_kernel<C, qfc, true, abc, BK>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((dsrelu_kernel<C, qfc, false, abc, BK>), grid, block, 0, s, p);
    };
    using A0 = std::integral_constant<int, 0>;
    using A1 = std::integral_constant<int, 1>;
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    if (p.ab_e5m2) {
        if (qf == 0)
            return hipErrorInvalidValue;
        qf == 1 ? go(Q1(), A1()) : go(Q2(), A1());
    } else {
        qf == 1 ? go(Q1(), A0()) : qf == 2 ? go(Q2(), A0()) : go(Q0(), A0());
    }
    return hipGetLastError();
}

extern template hipError_t launch_dsrelu_bk<true>(const DsreluArgs&, hipStream_t);
extern template hipError_t launch_dsrelu_bk<false>(const DsreluArgs&, hipStream_t);

}  // namespace gg
