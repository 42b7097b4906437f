// gg_dsrelu.hip -- M-grouped block-scaled (MXFP8) dgrad fused with the
// dsReLU backward on gfx950.
//
// For the rows of group g ("Grouped GEMM + dsReLU (SM100)", "Equations"):
//   G = alpha_g * sum_k deq(A) deq(B_g)   (E4M3 values, one E8M0 scale per
//                                          32 K values of a row)
//   D_row = prob * 2 * C * relu(G),  dprob = sum_n C relu(G)^2,
// and the per-expert Amax of |D_row| ("Shapes").
//
// Design: the M-grouped tiling of the dGLU kernel with 128 fp8 values of K
// per LDS stage, fed to v_mfma_scale_f32_32x32x64_f8f6f4.  The scales never
// go through LDS: with the data of step k+1, every lane also fetches the
// 32-bit word holding the four scale bytes of each of its fragment rows; at
// the top of step k+1 the word is shifted so that the byte of the K block the
// lane feeds to the MFMA sits in byte 0.  The epilogue applies alpha, relu,
// prob and C in registers, reduces dprob across lanes (one atomic per row
// and wave) and Amax across the wave (one atomicMax on the fp32 bit pattern,
// which orders like the value because |D| >= 0).
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "gg_moe.h"

namespace gg {

using DsreluCfg = Cfg<256, 256, 4, 2>;

template <class C>
__global__ void __launch_bounds__(C::kThreads, 1) dsrelu_kernel(DsreluArgs p) {
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
    const int cols_valid = p.N - n0;

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int wm = w / C::WN, wn = w % C::WN;
    const int am0 = wm * (TM / C::WM), bn0 = wn * (TN / C::WN);
    const int lr = l & 31, lh = l >> 5;

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
    uint32_t swa[MB], swb[NB];                 // raw scale words, prefetched one step ahead
    uint32_t sa[2][MB], sb[2][NB];             // per sub-step, byte 0 = this lane's block
    auto issue = [&](char* st, int kt) {
        stage_k<C, TM>(st, a, K, rows_valid, (int64_t)kt * 128, K);
        stage_k<C, TN>(st + TM * kRowBytes, bg, K, cols_valid, (int64_t)kt * 128, K);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(sfa + kt * 4);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(sfb + kt * 4);
#pragma unroll
        for (int i = 0; i < MB; i++) {
            const int r = am0 + 32 * i + lr;
            swa[i] = buf_load4(ra, r < rows_valid ? (uint32_t)(r * KB) : kInvalid);
        }
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int r = bn0 + 32 * j + lr;
            swb[j] = buf_load4(rb, r < cols_valid ? (uint32_t)(r * KB) : kInvalid);
        }
    };
    auto begin = [&](int) {
#pragma unroll
        for (int i = 0; i < MB; i++) {
            sa[0][i] = swa[i] >> (8 * lh);
            sa[1][i] = swa[i] >> (16 + 8 * lh);
        }
#pragma unroll
        for (int j = 0; j < NB; j++) {
            sb[0][j] = swb[j] >> (8 * lh);
            sb[1][j] = swb[j] >> (16 + 8 * lh);
        }
    };
    auto compute = [&](char* st, int) {
        mfma_stage_mx8<C>(st, st + TM * kRowBytes, am0, bn0, sa, sb, acc);
    };
    mainloop<C>(smem, p.K / 128, issue, compute, begin);

    // ---------------- epilogue ----------------
    // Rows of 8 columns per lane: C and D are 16-byte accesses (32 for fp32).
    const float al = p.alpha[g];
    const int64_t N = p.N;
    float amax = 0.0f;
    float rowsum[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        rowsum[k] = 0.0f;
    for_each_row8<C>(acc, (float*)(smem + w * kEpiWaveBytes), [&](int t, int r, int c, float (&v)[8]) {
        const int rr = am0 + r;
        const int col = n0 + bn0 + c;
        if (rr < rows_valid && col < p.N) {
            const int64_t row = m0 + rr;
            float cv[8], d[8];
            load8(p.c, p.c_dtype, row * N + col, cv);
            const float pr2 = p.prob[row] * 2.0f;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const float rl = fmaxf(al * v[k], 0.0f);
                d[k] = pr2 * cv[k] * rl;
                rowsum[t] += cv[k] * rl * rl;
                amax = fmaxf(amax, fabsf(d[k]));
            }
            store8(p.d, p.d_dtype, row * N + col, d);
        }
    });
#pragma unroll
    for (int t = 0; t < 8; t++) {
        float v = rowsum[t];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        const int rr = am0 + (l >> 3) + 8 * t;
        if ((l & 7) == 0 && rr < rows_valid && n0 + bn0 < p.N)
            atomicAdd(p.dprob + m0 + rr, v);
    }
    if (p.amax) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o));
        if (l == 0)
            atomicMax((int*)p.amax + g, __float_as_int(amax));
    }
}

hipError_t launch_dsrelu(const DsreluArgs& p, hipStream_t s) {
    using C = DsreluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    hipLaunchKernelGGL((dsrelu_kernel<C>), dim3((unsigned)tiles), dim3(C::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
