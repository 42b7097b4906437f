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
// K layout, N-major discrete B in the MN layout).  In the epilogue a
// 32-column MFMA block of R lines up with one 32-wide block pair of C/D: each
// lane owns one compact column and reads its input and gate columns of C.
// dprob is reduced across the 32 lanes of a column block with lane shuffles
// and added with one atomic per row and wave; dbias column sums are reduced
// per wave and added into an fp32 workspace, which a finalize kernel folds
// into the bf16 dbias.
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "../../include/gg_moe.h"

namespace gg {

using DgluCfg = Cfg<256, 256, 4, 2>;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// X = beta * C as a single fp32 product: no contraction into a later FMA, so
// the clamp / filter comparisons see exactly the rounded product.
__device__ __forceinline__ float scaled_x(float beta, float c) {
#pragma clang fp contract(off)
    return beta * c;
}

template <class C, bool B_K>
__global__ void __launch_bounds__(C::kThreads, 1) dglu_kernel(DgluArgs p) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

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
    auto issue = [&](char* st, int kt) {
        stage_k<C, TM>(st, a, lda, rows_valid, (int64_t)kt * 128, lda);
        if constexpr (B_K)
            stage_k<C, TN>(st + TM * kRowBytes, bg + (int64_t)n0 * lda, lda, p.N - n0,
                           (int64_t)kt * 128, lda);
        else
            stage_mn<C>(st + TM * kRowBytes, bg + ((int64_t)kt * 64 * p.N + n0) * 2,
                        (int64_t)p.N * 2, p.N - n0, p.K - kt * 64);
    };
    auto compute = [&](char* st, int) {
        mfma_stage_bf16<C, true, B_K>(st, st + TM * kRowBytes, am0, bn0, acc);
    };
    mainloop<C>(smem, p.K / 64, issue, compute);

    // ---------------- epilogue ----------------
    const float al = p.alpha[g];
    const float a2 = al * al;
    const float bet = p.beta[g];
    const int64_t N2 = 2 * (int64_t)p.N;
    const int lr = l & 31;
    float rowsum[MB][16];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            rowsum[i][r] = 0.0f;
    float* dbias_ws = p.dbias ? (float*)((char*)p.ws + kWsHeader) + (int64_t)g * N2 : nullptr;

#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int nblk = n0 + bn0 + 32 * j;   // compact block start
        const bool jok = nblk < p.N;
        const int64_t pair = nblk / 32;
        const int64_t c_in = 64 * pair + (p.gate_first ? 32 : 0) + lr;
        const int64_t c_gt = 64 * pair + (p.gate_first ? 0 : 32) + lr;
        float bsum_in = 0.0f, bsum_gt = 0.0f;
#pragma unroll
        for (int i = 0; i < MB; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rr = am0 + 32 * i + acc_row(r, l);
                if (jok && rr < rows_valid) {
                    const int64_t row = m0 + rr;
                    const float R = a2 * acc[i][j][r];
                    const float u = scaled_x(bet, load_elem(p.c, p.c_dtype, row * N2 + c_in));
                    const float gt = scaled_x(bet, load_elem(p.c, p.c_dtype, row * N2 + c_gt));
                    const float Rp = R * p.prob[row];
                    float d_in, d_gt, act;
                    if (p.act == 0) {
                        const float s = sigmoidf_(gt);
                        d_in = Rp * gt * s;
                        d_gt = Rp * u * s * (1.0f + gt * (1.0f - s));
                        act = gt * s * u;
                    } else {
                        const float gc = fminf(gt, p.clamp_max);
                        const float uc = fminf(fmaxf(u, p.clamp_min), p.clamp_max);
                        const bool g_in = gt <= p.clamp_max;
                        const bool u_in = (u >= p.clamp_min) & (u <= p.clamp_max);
                        const float gf = g_in ? (p.mask_filter ? 1.0f : gt) : 0.0f;
                        const float uf = u_in ? (p.mask_filter ? 1.0f : u) : 0.0f;
                        const float s = sigmoidf_(p.geglu_alpha * gc);
                        const float ul = uc + p.linear_offset;
                        d_gt = Rp * ul * s * (1.0f + p.geglu_alpha * gc * (1.0f - s)) * gf;
                        d_in = Rp * gc * s * uf;
                        act = gc * s * ul;
                    }
                    rowsum[i][r] += R * act;
                    bsum_in += d_in;
                    bsum_gt += d_gt;
                    store_elem(p.d, p.d_dtype, row * N2 + c_in, d_in);
                    store_elem(p.d, p.d_dtype, row * N2 + c_gt, d_gt);
                }
            }
        }
        if (dbias_ws) {
            // lanes l and l + 32 hold the same column, different rows
            bsum_in += __shfl_xor(bsum_in, 32);
            bsum_gt += __shfl_xor(bsum_gt, 32);
            if (l < 32 && jok) {
                atomicAdd(dbias_ws + c_in, bsum_in);
                atomicAdd(dbias_ws + c_gt, bsum_gt);
            }
        }
    }
    // dprob: sum each row over the 32 columns of the lane group, one atomic
    // per row per wave.
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            float v = rowsum[i][r];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            const int rr = am0 + 32 * i + acc_row(r, l);
            if (lr == 0 && rr < rows_valid && n0 + bn0 < p.N)
                atomicAdd(p.dprob + m0 + rr, v);
        }
}

hipError_t launch_dglu(const DgluArgs& p, hipStream_t s) {
    using C = DgluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    if (p.b_kmajor)
        hipLaunchKernelGGL((dglu_kernel<C, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((dglu_kernel<C, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
