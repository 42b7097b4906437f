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
// K layout, N-major discrete B in the MN layout).  The epilogue stages the
// accumulators through LDS so that a lane owns 8 consecutive compact columns
// of one row; a 32-column block of R lines up with one 32-wide input/gate
// block pair of C and D, so those columns are one 16-byte access in each
// half.  dprob is reduced across the 8 lanes of a row with lane shuffles and
// added with one atomic per row and wave; dbias column sums are reduced per
// wave and added into an fp32 workspace, which a finalize kernel folds into
// the bf16 dbias.
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "gg_moe.h"

namespace gg {

using DgluCfg = Cfg<256, 256, 4, 2>;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// X = beta * C as a single fp32 product: no contraction into a later FMA, so
// the clamp / filter comparisons see exactly the rounded product.
__device__ __forceinline__ float scaled_x(float beta, float c) {
#pragma clang fp contract(off)
    return beta * c;
}

// W32: C is fp32 (else bf16 / fp16); ACT: 0 dSwiGLU, 1 dGeGLU.  Each
// combination is its own kernel so the register allocation of one epilogue
// does not burden the others.
template <class C, bool B_K, bool W32, int ACT>
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
    LoadK<C, TM> la;
    std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>> lb;
    la.init(lda, rows_valid);
    if constexpr (B_K)
        lb.init(lda, p.N - n0);
    else
        lb.init((int64_t)p.N * 2, p.N - n0);
    using LB = std::conditional_t<B_K, LoadK<C, TN>, LoadMN<C>>;
    constexpr int kLA = LoadK<C, TM>::kN;
    auto issue = [&](uint32_t st, int u, int i) {
        const int64_t kb = (int64_t)u * 128;
        if (i < kLA) {
            la.template issue<false>(st, a + kb, lda - kb, i);
        } else {
            if constexpr (B_K)
                lb.template issue<false>(st + TM * kRowBytes, bg + (int64_t)n0 * lda + kb, lda - kb,
                                         i - kLA);
            else
                lb.issue(st + TM * kRowBytes, bg + ((int64_t)u * 64 * p.N + n0) * 2,
                         (int64_t)p.K - u * 64, i - kLA);
        }
    };
    auto read = [&](const char* st, int kt, FragBf16<C>& f, int g) {
        read_bf16<C, true, B_K>(st, st + TM * kRowBytes, am0, bn0, kt & 1, f, g);
    };
    auto mma = [&](const FragBf16<C>& f, int m0_, int m1_) { mma_bf16<C>(f, acc, m0_, m1_); };
    FragBf16<C> frag[2];
    pipeline<C, kLA + LB::kN, 2 * MB * NB, MB + NB>(smem, p.K / 32, frag, issue, read, mma);

    // ---------------- epilogue ----------------
    // Rows of 8 compact columns per lane: the 8 input and 8 gate columns of C
    // and D are each one 16-byte access (32 for fp32).
    const float al = p.alpha[g];
    const float a2 = al * al;
    const float bet = p.beta[g];
    const int64_t N2 = 2 * (int64_t)p.N;
    float* dbias_ws = p.dbias ? (float*)((char*)p.ws + kWsHeader) + (int64_t)g * N2 : nullptr;
    constexpr int kT = 4 * C::MB;                  // row walk steps per lane
    float rowsum[kT], bs_in[8], bs_gt[8];
#pragma unroll
    for (int t = 0; t < kT; t++)
        rowsum[t] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++)
        bs_in[k] = bs_gt[k] = 0.0f;
    // C (input and gate columns) and prob of the items 12 ahead (6 for fp32
    // C) are in flight while an item is processed; items off the tile load
    // row 0 / column 0 (always present) and store nothing.
    float* const elds = (float*)(smem + w * kEpiWaveBytes);
    auto epilogue = [&](auto W32_, auto ACT_) {
        constexpr bool w32 = decltype(W32_)::value;
        constexpr int act_kind = decltype(ACT_)::value;
        using Pre = Pre8<w32, 2>;
        auto cols = [&](int c, int64_t& c_in, int64_t& c_gt) {
            const int n = n0 + bn0 + c;                 // first compact column
            c_in = 64 * (int64_t)(n / 32) + (p.gate_first ? 32 : 0) + n % 32;
            c_gt = 64 * (int64_t)(n / 32) + (p.gate_first ? 0 : 32) + n % 32;
        };
        auto load = [&](int, int r, int c) {
            const int rr = am0 + r;
            const bool ok = (rr < rows_valid) & (n0 + bn0 + c < p.N);
            int64_t c_in, c_gt;
            cols(c, c_in, c_gt);
            const int64_t row = m0 + (ok ? rr : 0);
            Pre pre;
            pre.x[0] = raw8_load<w32>(p.c, row * N2 + (ok ? c_in : 0));
            pre.x[1] = raw8_load<w32>(p.c, row * N2 + (ok ? c_gt : 0));
            pre.row = p.prob[row];
            return pre;
        };
        auto fn = [&](int t, int r, int c, float (&v)[8], const Pre& pre) {
            const int rr = am0 + r;
            const int n = n0 + bn0 + c;
            int64_t c_in, c_gt;
            cols(c, c_in, c_gt);
            if (rr < rows_valid && n < p.N) {
                const int64_t row = m0 + rr;
                float xin[8], xgt[8], din[8], dgt[8];
                raw8_cvt<w32>(pre.x[0], p.c_dtype, xin);
                raw8_cvt<w32>(pre.x[1], p.c_dtype, xgt);
                const float pr = pre.row;
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const float R = a2 * v[k];
                    const float u = scaled_x(bet, xin[k]);
                    const float gt = scaled_x(bet, xgt[k]);
                    const float Rp = R * pr;
                    float act;
                    if constexpr (act_kind == 0) {
                        const float sg = sigmoidf_(gt);
                        din[k] = Rp * gt * sg;
                        dgt[k] = Rp * u * sg * (1.0f + gt * (1.0f - sg));
                        act = gt * sg * u;
                    } else {
                        const float gc = fminf(gt, p.clamp_max);
                        const float uc = fminf(fmaxf(u, p.clamp_min), p.clamp_max);
                        const bool g_in = gt <= p.clamp_max;
                        const bool u_in = (u >= p.clamp_min) & (u <= p.clamp_max);
                        const float gf = g_in ? (p.mask_filter ? 1.0f : gt) : 0.0f;
                        const float uf = u_in ? (p.mask_filter ? 1.0f : u) : 0.0f;
                        const float sg = sigmoidf_(p.geglu_alpha * gc);
                        const float ul = uc + p.linear_offset;
                        dgt[k] = Rp * ul * sg * (1.0f + p.geglu_alpha * gc * (1.0f - sg)) * gf;
                        din[k] = Rp * gc * sg * uf;
                        act = gc * sg * ul;
                    }
                    rowsum[t] += R * act;
                    bs_in[k] += din[k];
                    bs_gt[k] += dgt[k];
                }
                store8(p.d, p.d_dtype, row * N2 + c_in, din);
                store8(p.d, p.d_dtype, row * N2 + c_gt, dgt);
            }
            if (t == kT - 1 && dbias_ws) {
                // column sums over the wave's rows: lanes sharing l & 7 hold
                // the same 8 columns
#pragma unroll
                for (int k = 0; k < 8; k++) {
#pragma unroll
                    for (int o = 8; o < 64; o <<= 1) {
                        bs_in[k] += __shfl_xor(bs_in[k], o);
                        bs_gt[k] += __shfl_xor(bs_gt[k], o);
                    }
                }
                if (l < 8 && n < p.N) {
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        atomicAdd(dbias_ws + c_in + k, bs_in[k]);
                        atomicAdd(dbias_ws + c_gt + k, bs_gt[k]);
                    }
                }
#pragma unroll
                for (int k = 0; k < 8; k++)
                    bs_in[k] = bs_gt[k] = 0.0f;
            }
        };
        for_each_row8<C, w32 ? 6 : 12>(acc, elds, load, fn);
    };
    epilogue(std::integral_constant<bool, W32>(), std::integral_constant<int, ACT>());
    // dprob: the 8 lanes of a row hold its partial sums; one atomic per row
    // and wave.
#pragma unroll
    for (int t = 0; t < kT; t++) {
        float v = rowsum[t];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        const int rr = am0 + (l >> 3) + 8 * t;
        if ((l & 7) == 0 && rr < rows_valid && n0 + bn0 < p.N)
            atomicAdd(p.dprob + m0 + rr, v);
    }
}

hipError_t launch_dglu(const DgluArgs& p, hipStream_t s) {
    using C = DgluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    const dim3 grid((unsigned)tiles), block(C::kThreads);
    auto go = [&](auto BK, auto W32) {
        constexpr bool bk = decltype(BK)::value, w32 = decltype(W32)::value;
        if (p.act == 0)
            hipLaunchKernelGGL((dglu_kernel<C, bk, w32, 0>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((dglu_kernel<C, bk, w32, 1>), grid, block, 0, s, p);
    };
    const bool w32 = p.c_dtype == kF32;
    if (p.b_kmajor)
        w32 ? go(std::true_type(), std::true_type()) : go(std::true_type(), std::false_type());
    else
        w32 ? go(std::false_type(), std::true_type()) : go(std::false_type(), std::false_type());
    return hipGetLastError();
}

}  // namespace gg
