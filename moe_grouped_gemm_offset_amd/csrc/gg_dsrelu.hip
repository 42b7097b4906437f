// gg_dsrelu.hip -- M-grouped block-scaled (MXFP8) dgrad fused with the
// dsReLU backward on gfx950.
//
// For the rows of group g ("Grouped GEMM + dsReLU (SM100)", "Equations"):
//   G = alpha_g * sum_k deq(A) deq(B_g)   (E4M3 values, one E8M0 scale per
//                                          32 K values of a row)
//   D_row = prob * 2 * C * relu(G),  dprob = sum_n C relu(G)^2,
// and the per-expert Amax of |D_row| ("Shapes").
//
// Design: the M-grouped tiling of the dGLU kernel with 64 fp8 values of K
// per stage (128 per load unit), fed to v_mfma_scale_f32_32x32x64_f8f6f4.
// The scales of 8 stages at a time (16 bytes of each of the tile's 512
// operand rows) are staged in LDS by dword LDS-writing loads, four
// row-contiguous words per 4 lanes, in two alternating buffers: the next
// group's words arrive with the load units of the current group.  A per-lane
// scale fetch per stage would instead send one cache request per row and
// stage through the vector memory path, more requests than the operand data
// itself.  With the fragments of a stage a lane reads the scale word of each
// of its fragment rows and shifts it so that the byte of the K block it
// feeds to the MFMA sits in byte 0.  The epilogue applies alpha, relu, prob
// and C in registers, reduces dprob across lanes (one atomic per row and
// wave) and Amax across the wave (one atomicMax on the fp32 bit pattern,
// which orders like the value because |D| >= 0).
#include "gg_internal.hpp"
#include "gg_tile.hpp"
#include "gg_moe.h"

namespace gg {

using DsreluCfg = Cfg<256, 256, 2, 2>;

// Scale staging: two buffers, each holding the scale words of a group of 8
// stages (4 load units; 4 words per row: one word covers 128 K values) for
// the tile's A rows (slots 0 .. TM-1) and B rows (slots TM .. TM+TN-1), 16
// bytes per slot, word w at byte 4 w.  (A stage's word of 32 consecutive
// slots is then read with 2-way bank conflicts, 8 such reads per stage and
// wave.)  Group g lives in buffer g & 1.  Group g+1 comes with units 4g+1 ..
// 4g+4, one slice of 128 slots per unit: the last slice lands with the unit
// group g+1 starts in, and the first is issued only after the barrier that
// follows the last read of group g-1.  Past the last group the slices load
// words no stage reads, which keeps the count of loads per unit fixed.
constexpr int kScaleUnits = 4;
template <class C>
struct ScaleLds {
    static constexpr int kSlots = C::TM + C::TN;
    static constexpr int kBuf = kSlots * 16;                           // bytes per buffer
    static constexpr int kBase = 2 * C::kUnit;                         // after the unit buffers
    static constexpr int kSmem = kBase + 2 * kBuf > C::kLds ? kBase + 2 * kBuf : C::kLds;
    static constexpr int kPerUnit = kSlots / kScaleUnits / 16 / C::kWaves;   // loads per wave
    static_assert(C::TM == C::TN && kPerUnit * 16 * C::kWaves * kScaleUnits == kSlots,
                  "scale slices must split evenly over waves and units");
};

template <class C>
__global__ void __launch_bounds__(C::kThreads, 1) dsrelu_kernel(DsreluArgs p) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    using S = ScaleLds<C>;
    __shared__ __attribute__((aligned(1024))) char smem[S::kSmem];

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
    const int lr = l & 31, lq = l >> 5;

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
    const int nk = (int)(K / 64);                // stages; K % 128 == 0, so nk is even
    // Scale records end at the last valid row, so rows past the tile edge
    // load zeros.  Words past the end of K are never read: they belong to no
    // stage.
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sfa, (uint32_t)(rows_valid * KB));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sfb, (uint32_t)(cols_valid * KB));
    char* const sbuf = smem + S::kBase;
    const uint32_t sbuf32 = lds_addr(sbuf);
    const int wu = uniform(w);
    // Slice s (0 .. 3) of a group: slots 128 (s & 1) + 16 (kPerUnit w + t) +
    // (l >> 2) of A (s < 2) or B (s >= 2), t < kPerUnit, lane l taking word
    // l & 3 of its slot.
    constexpr int kSliceSlots = TM / 2;
    const uint32_t sc_off = (uint32_t)((16 * S::kPerUnit * w + (l >> 2)) * KB + 4 * (l & 3));
    // load t (0 .. kPerUnit-1) of slice `slice` of scale group grp
    auto scale_load = [&](int grp, int slice, int t) {
        const int half = slice & 1;
        const bool is_a = slice < 2;
        const int slot0 = kSliceSlots * half + 16 * (S::kPerUnit * wu + t);
        const uint32_t lds = sbuf32 + (grp & 1) * S::kBuf + (is_a ? 0 : TM * 16) + slot0 * 16;
        dma4(is_a ? rsa : rsb, lds, sc_off + (uint32_t)((kSliceSlots * half + 16 * t) * KB + 16 * grp));
    };
    LoadK<C, TM> la;
    LoadK<C, TN> lb;
    la.init(K, rows_valid);
    lb.init(K, cols_valid);
    constexpr int kLA = LoadK<C, TM>::kN, kLB = LoadK<C, TN>::kN;
    auto issue = [&](uint32_t st, int u, int i) {
        const int64_t kb = (int64_t)u * 128;
        if (i < kLA) {
            la.template issue<false>(st, a + kb, K - kb, i);
        } else if (i < kLA + kLB) {
            lb.template issue<false>(st + TM * kRowBytes, bg + kb, K - kb, i - kLA);
        } else {
            // units 1 .. 4 carry group 1, 5 .. 8 group 2, ...; unit 0
            // carries a slice of group 0 again (identical words)
            const int v = u > 0 ? u - 1 : 0;
            scale_load(u > 0 ? v / kScaleUnits + 1 : 0, v % kScaleUnits, i - kLA - kLB);
        }
    };
    const int lsh = 8 * lq;
    auto read = [&](const char* st, int kt, FragMx8<C>& f, int g) {
        read_mx8<C>(st, st + TM * kRowBytes, am0, bn0, kt & 1, f, g);
        // this stage's scale word of the group's row, shifted so byte 0 is
        // this lane's K block
        const char* buf = sbuf + ((kt / 8) & 1) * S::kBuf + 4 * ((kt % 8) >> 1);
        const int sh = lsh + 16 * (kt & 1);
        if (g < MB)
            f.sa[g] = *reinterpret_cast<const uint32_t*>(buf + (am0 + 32 * g + lr) * 16) >> sh;
        else
            f.sb[g - MB] = *reinterpret_cast<const uint32_t*>(buf + (TM + bn0 + 32 * (g - MB) + lr) * 16) >> sh;
    };
    auto mma = [&](const FragMx8<C>& f, int m0_, int m1_) { mma_mx8<C>(f, acc, m0_, m1_); };
    FragMx8<C> frag[2];
    // Group 0 ahead of unit 0: complete whenever unit 0 is.
#pragma unroll
    for (int s4 = 0; s4 < kScaleUnits; s4++)
#pragma unroll
        for (int t = 0; t < S::kPerUnit; t++)
            scale_load(0, s4, t);
    pipeline<C, kLA + kLB + S::kPerUnit, MB * NB, MB + NB>(smem, nk, frag, issue, read, mma);

    // ---------------- epilogue ----------------
    // Rows of 8 columns per lane: C and D are 16-byte accesses (32 for fp32).
    // C and prob of the items 24 ahead (12 for fp32 C) are in flight while an
    // item is processed; items off the tile load row 0 / column 0 (always
    // present) and store nothing.
    const float al = p.alpha[g];
    const int64_t N = p.N;
    float amax = 0.0f;
    constexpr int kT = 4 * MB;                     // row walk steps per lane
    float rowsum[kT];
#pragma unroll
    for (int t = 0; t < kT; t++)
        rowsum[t] = 0.0f;
    float* const elds = (float*)(smem + w * kEpiWaveBytes);
    auto epilogue = [&](auto W32) {
        constexpr bool w32 = decltype(W32)::value;
        using Pre = Pre8<w32, 1>;
        auto load = [&](int, int r, int c) {
            const int rr = am0 + r, col = n0 + bn0 + c;
            const bool ok = (rr < rows_valid) & (col < p.N);
            const int64_t row = m0 + (ok ? rr : 0);
            Pre pre;
            pre.x[0] = raw8_load<w32>(p.c, row * N + (ok ? col : 0));
            pre.row = p.prob[row];
            return pre;
        };
        auto fn = [&](int t, int r, int c, float (&v)[8], const Pre& pre) {
            const int rr = am0 + r;
            const int col = n0 + bn0 + c;
            if (rr < rows_valid && col < p.N) {
                const int64_t row = m0 + rr;
                float cv[8], d[8];
                raw8_cvt<w32>(pre.x[0], p.c_dtype, cv);
                const float pr2 = pre.row * 2.0f;
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const float rl = fmaxf(al * v[k], 0.0f);
                    d[k] = pr2 * cv[k] * rl;
                    rowsum[t] += cv[k] * rl * rl;
                    amax = fmaxf(amax, fabsf(d[k]));
                }
                store8(p.d, p.d_dtype, row * N + col, d);
            }
        };
        for_each_row8<C, w32 ? 12 : 24>(acc, elds, load, fn);
    };
    if (p.c_dtype == kF32)
        epilogue(std::true_type());
    else
        epilogue(std::false_type());
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
