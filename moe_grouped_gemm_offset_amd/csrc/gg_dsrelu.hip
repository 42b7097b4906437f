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
// per LDS step.  The scales never go through LDS: for each K step every lane
// loads the 32-bit word holding the four scale bytes of its fragment row and
// shifts it so that the byte of the K block it feeds to
// v_mfma_scale_f32_32x32x64_f8f6f4 sits in byte 0.  Both the data and the
// scales of step k+1 are fetched before the MFMAs of step k.  The epilogue
// applies alpha, relu, prob and C in registers, reduces dprob across lanes
// (one atomic per row and wave) and Amax across the wave (one atomicMax on
// the fp32 bit pattern, valid because |D| >= 0).
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "../../include/gg_moe.h"

namespace gg {

template <int TM, int TN>
__global__ void __launch_bounds__(kThreads, 1) dsrelu_kernel(DsreluArgs p) {
    constexpr int MB = TM / 64, NB = TN / 64;
    constexpr int kBufBytes = (TM + TN) * kRowBytes;
    __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];

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
    const int wm = w >> 1, wn = w & 1;
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
    KLoader<TM> la;
    KLoader<TN> lb;
    uint32_t swa[MB], swb[NB];                 // raw scale words of the next step
    auto load = [&](int kt) {
        la.load(a, K, rows_valid, (int64_t)kt * 128, K);
        lb.load(bg, K, cols_valid, (int64_t)kt * 128, K);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(sfa + kt * 4);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(sfb + kt * 4);
#pragma unroll
        for (int i = 0; i < MB; i++) {
            const int r = wm * (TM / 2) + 32 * i + lr;
            swa[i] = buf_load4(ra, r < rows_valid ? (uint32_t)(r * KB) : kInvalid);
        }
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int r = wn * (TN / 2) + 32 * j + lr;
            swb[j] = buf_load4(rb, r < cols_valid ? (uint32_t)(r * KB) : kInvalid);
        }
    };
    uint32_t sa[2][MB], sb[2][NB];             // per sub-step, byte 0 = this lane's block
    auto take_scales = [&]() {
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
    const int nk = p.K / 128;
    load(0);
    la.store(smem);
    lb.store(smem + TM * kRowBytes);
    take_scales();
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        char* cur = smem + (kt & 1) * kBufBytes;
        char* nxt = smem + ((kt + 1) & 1) * kBufBytes;
        const bool more = kt + 1 < nk;
        if (more)
            load(kt + 1);
        mfma_step_mx8<MB, NB>(cur, cur + TM * kRowBytes, wm * (TM / 2), wn * (TN / 2), sa, sb, acc);
        if (more) {
            la.store(nxt);
            lb.store(nxt + TM * kRowBytes);
            take_scales();
        }
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    const float al = p.alpha[g];
    const int64_t N = p.N;
    float amax = 0.0f;
    float rowsum[MB][16];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            rowsum[i][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int col = n0 + wn * (TN / 2) + 32 * j + lr;
        if (n0 + wn * (TN / 2) + 32 * j >= p.N)
            continue;
#pragma unroll
        for (int i = 0; i < MB; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rr = wm * (TM / 2) + 32 * i + acc_row(r, l);
                if (rr >= rows_valid)
                    continue;
                const int64_t row = m0 + rr;
                const float G = al * acc[i][j][r];
                const float rl = fmaxf(G, 0.0f);
                const float c = load_elem(p.c, p.c_dtype, row * N + col);
                const float d = p.prob[row] * 2.0f * c * rl;
                rowsum[i][r] += c * rl * rl;
                amax = fmaxf(amax, fabsf(d));
                store_elem(p.d, p.d_dtype, row * N + col, d);
            }
    }
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
            const int rr = wm * (TM / 2) + 32 * i + acc_row(r, l);
            if (lr == 0 && rr < rows_valid && n0 + wn * (TN / 2) < p.N)
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

template <int TM, int TN>
static hipError_t launch_dsrelu_t(const DsreluArgs& p, hipStream_t s) {
    const int64_t tiles = ((p.m_rows + TM - 1) / TM) * ((p.N + TN - 1) / TN);
    if (tiles == 0)
        return hipSuccess;
    hipLaunchKernelGGL((dsrelu_kernel<TM, TN>), dim3((unsigned)tiles), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_dsrelu(const DsreluArgs& p, hipStream_t s) { return launch_dsrelu_t<256, 256>(p, s); }

}  // namespace gg
