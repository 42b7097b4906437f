// gg_dglu_epi.hpp -- the fused dSwiGLU / dGeGLU / dSiTU-GLU epilogue of the M-grouped
// dgrad kernels (bf16 and block-scaled main loops alike).
//
// For a tile of rows of group g and compact columns n ("Grouped GEMM + dGLU
// (SM100)", "BF16 contract / Tensors, layouts, and equation"; the
// block-scaled contract applies the same steps to its dequantized product):
// R = alpha_g^2 * acc, X = beta_g C, and the 32-wide interleaved input/gate
// blocks of X feed the activation backward; D, dprob, dbias and, for the
// block-scaled contract, the per-expert amax of the input-gradient and of the
// gate-gradient columns ("Shapes": (L, 2, 1)) are produced here.
//
// The accumulators are staged through LDS so that a lane owns 8 consecutive
// compact columns of one row; a 32-column block of R lines up with one
// 32-wide input/gate block pair of C and D, so those columns are one 16-byte
// access in each half.  dprob is reduced across the 8 lanes of a row with
// lane shuffles and added with one atomic per row and wave; dbias column sums
// are reduced per wave and added into an fp32 workspace, which a finalize
// kernel folds into the bf16 dbias; amax is reduced across the wave and
// raised with one atomicMax per half on the fp32 bit pattern (which orders
// like the value because |D| >= 0).
#pragma once
#include "gg_fp8out.hpp"
#include "gg_internal.hpp"
#include "gg_tile.hpp"

namespace gg {

// The hardware reciprocal (1 ulp) instead of an IEEE division: the epilogue's
// arithmetic is a good share of the dGLU kernels' time.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// tanh(x) from u = expm1(-2|x|) in (-1, 0]: tanh|x| = -u / (u + 2).  No
// cancellation for small |x| (expm1 keeps u's relative accuracy where
// exp(-2|x|) is close to 1), no overflow for large |x| (u tends to -1).
__device__ __forceinline__ float tanhf_(float x) {
    const float u = expm1f(-2.0f * fabsf(x));
    return copysignf(-u * __builtin_amdgcn_rcpf(u + 2.0f), x);
}

// X = beta * C as a single fp32 product: no contraction into a later FMA, so
// the clamp / filter comparisons see exactly the rounded product.
__device__ __forceinline__ float scaled_x(float beta, float c) {
#pragma clang fp contract(off)
    return beta * c;
}

// CW: bytes per C element (4 fp32, 2 bf16 / fp16, 1 FP8 codes: E4M3 or
// E5M2, the block-scaled contract's FP8 C); ACT: 0 dSwiGLU, 1 dGeGLU, 2 dSiTU-GLU
// (the block-scaled contract's "Equations": T_g = b1 tanh(G/b1) sigmoid(G),
// T_u = b2 tanh(U/b2), gradients R prob T_u dT_g/dG and R prob T_g dT_u/dU,
// activation T_g T_u); AMAX: raise
// p.amax[2 g + {0: input, 1: gate}]; QF: D as FP8 D_row / D_col with E8M0
// scales (gg_fp8out.hpp; 1 E4M3, 2 E5M2) instead of a 16/32-bit D (0); BF:
// C is bf16 and, unless QF, so is D, known at compile time (no per-element
// format branches, which
// also keeps the compiler's memory-counter waits exact); DB: accumulate the
// dbias column sums (added only when p.dbias is set); FILT: dGeGLU's filters
// carry the raw value (0) or are the 0/1 indicator (1,
// GG_FLAG_GEGLU_MASK_FILTER), or follow p.mask_filter (2); kAhead: row-walk items
// whose C loads are in flight while one is processed.  The caller has
// passed the barrier that ends the main loop's use of smem.
template <class C, int CW, int ACT, bool AMAX, int kAhead, int QF = 0, bool BF = false,
          bool DB = true, int FILT = 2>
__device__ __forceinline__ void dglu_epilogue(const DgluArgs& p, const f32x16 (&acc)[C::MB][C::NB],
                                              char* smem, int64_t m0, int n0, int g,
                                              int rows_valid, int am0, int bn0) {
    constexpr bool Q = QF != 0, BF8 = QF == 2;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const float al = p.alpha[g];
    const float a2 = al * al;
    const float bet = p.beta[g];
    const int64_t N2 = 2 * (int64_t)p.N;
    const float rb1 = 1.0f / p.situ_b1, rb2 = 1.0f / p.situ_b2;
    const bool mask = FILT == 2 ? p.mask_filter != 0 : FILT == 1;
    const int cdt = BF ? kBF16 : p.c_dtype, ddt = BF ? kBF16 : p.d_dtype;
    float* dbias_ws = p.dbias ? (float*)((char*)p.ws + kWsHeader) + (int64_t)g * N2 : nullptr;
    constexpr int kT = 4 * C::MB;                  // row walk steps per lane
    float rowsum[kT], bs_in[8], bs_gt[8];
    float amax_in = 0.0f, amax_gt = 0.0f;
#pragma unroll
    for (int t = 0; t < kT; t++)
        rowsum[t] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++)
        bs_in[k] = bs_gt[k] = 0.0f;
    // C (input and gate columns) and prob of the items kAhead ahead are in
    // flight while an item is processed; items off the tile load row 0 /
    // column 0 (always present) and store nothing.
    float* const elds = (float*)(smem + w * kEpiWaveBytes);
    const float nc = Q ? *p.q.norm_const : 1.0f;
    float dcol_in[4][8], dcol_gt[4][8];            // Q: a column block's 4 items
    // Compact column n's input and gate columns of C and D.
    auto cols = [&](int c, int64_t& c_in, int64_t& c_gt) {
        const int n = n0 + bn0 + c;                 // first compact column
        c_in = 64 * (int64_t)(n / 32) + (p.gate_first ? 32 : 0) + n % 32;
        c_gt = 64 * (int64_t)(n / 32) + (p.gate_first ? 0 : 32) + n % 32;
    };
    // The activation backward of one item (8 compact columns of a row):
    // din, dgt from the accumulators v and the item's C values, with the
    // row's dprob, dbias and amax partials.  R = alpha^2 acc and the row's
    // prob enter every gradient as one factor Rp = acc (alpha^2 prob);
    // dprob's row sum of R act is accumulated as sum acc act and scaled by
    // alpha^2 once per row.
    auto grad8 = [&](int t, const float (&v)[8], const float (&xin)[8], const float (&xgt)[8],
                     float a2pr, float (&din)[8], float (&dgt)[8]) {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float u = scaled_x(bet, xin[k]);
            const float gt = scaled_x(bet, xgt[k]);
            const float Rp = v[k] * a2pr;
            float act;
            if constexpr (ACT == 0) {
                // w = gate s (the swish); d swish / d gate = s (1 + gate (1 - s))
                // = s + w - w s
                const float sg = sigmoidf_(gt);
                const float w = gt * sg;
                din[k] = Rp * w;
                dgt[k] = (Rp * u) * fmaf(-w, sg, w + sg);
                act = w * u;
            } else if constexpr (ACT == 2) {
                const float sg = sigmoidf_(gt);
                const float tg = tanhf_(gt * rb1), tu = tanhf_(u * rb2);
                const float Tg = p.situ_b1 * tg * sg, Tu = p.situ_b2 * tu;
                const float dTg = (1.0f - tg * tg) * sg + p.situ_b1 * tg * sg * (1.0f - sg);
                dgt[k] = Rp * Tu * dTg;
                din[k] = Rp * Tg * (1.0f - tu * tu);
                act = Tg * Tu;
            } else {
                // clamped values feed the activation; the filters carry the
                // raw value (or 1 with the mask filter) inside the clamp, 0
                // outside.  The input lies inside its clamp exactly when
                // clamping leaves it unchanged.
                const float gc = fminf(gt, p.clamp_max);
                const float uc = fminf(fmaxf(u, p.clamp_min), p.clamp_max);
                const float gf = gt <= p.clamp_max ? (mask ? 1.0f : gt) : 0.0f;
                const float uf = uc == u ? (mask ? 1.0f : u) : 0.0f;
                const float gag = p.geglu_alpha * gc;
                const float sg = sigmoidf_(gag);
                const float ul = uc + p.linear_offset;
                const float w = gc * sg;
                // s (1 + a gc (1 - s)) = s + gs - gs s with gs = a gc s
                const float gs = gag * sg;
                dgt[k] = ((Rp * ul) * fmaf(-gs, sg, gs + sg)) * gf;
                din[k] = (Rp * uf) * w;
                act = w * ul;
            }
            rowsum[t] = fmaf(v[k], act, rowsum[t]);
            if constexpr (DB) {
                bs_in[k] += din[k];
                bs_gt[k] += dgt[k];
            }
            if constexpr (AMAX) {
                amax_in = fmaxf(amax_in, fabsf(din[k]));
                amax_gt = fmaxf(amax_gt, fabsf(dgt[k]));
            }
        }
    };
    // dbias: after a column half's last item, the column sums over the
    // wave's rows (lanes sharing l & 7 hold the same 8 columns) go into the
    // fp32 workspace.
    auto dbias_flush = [&](int c) {
        const int n = n0 + bn0 + c;
        int64_t c_in, c_gt;
        cols(c, c_in, c_gt);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            bs_in[k] = cols8(bs_in[k], AddOp());
            bs_gt[k] = cols8(bs_gt[k], AddOp());
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
    };
    if constexpr (BF && !Q && kT <= 8) {
        // bf16 C and D (8-wave kernels, whose lanes cover 8 rows each)
        // through buffer descriptors over the wave's rows:
        // 32-bit offsets from the wave's first row, record counts that end
        // at its last valid row, and columns past N at an invalid offset.
        // Masked accesses load zeros and store nothing, and zeros yield zero
        // gradients and zero dprob / dbias / amax contributions, so an item
        // needs no test of its own.
        constexpr int kWaveRows = C::TM / C::WM;
        const int rows_left = rows_valid - am0 < 0 ? 0
                            : (rows_valid - am0 > kWaveRows ? kWaveRows : rows_valid - am0);
        const int64_t wrow0 = m0 + am0;
        const uint32_t rowb = (uint32_t)(N2 * 2);          // bytes per row of C and D
        // (wave-uniform values marked as such, so the descriptors stay scalar)
        const uint32_t rec = (uint32_t)uniform((int)((uint32_t)rows_left * rowb));
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(uniform_ptr((const char*)p.c + wrow0 * (int64_t)rowb), rec);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(uniform_ptr((char*)p.d + wrow0 * (int64_t)rowb), rec);
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(uniform_ptr(p.prob + wrow0), (uint32_t)uniform(rows_left * 4));
        const int gsel = p.gate_first ? 32 : 0;
        // byte offset, within a row, of compact column c's input (gate false)
        // or gate (true) block, or kInvalid past N
        auto colb = [&](int c, bool gate) -> uint32_t {
            const int n = n0 + bn0 + c;
            return n < p.N ? (uint32_t)(64 * (n >> 5) + (gate ? 32 - gsel : gsel) + (n & 31)) * 2
                           : kInvalid;
        };
        // prob of the lane's kT rows (row (l >> 3) + 8 t), loaded once
        float prow[kT];
#pragma unroll
        for (int t = 0; t < kT; t++)
            prow[t] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rp, (uint32_t)((l >> 3) + 8 * t) * 4, 0, 0));
        struct PreB {
            u32x4 in, gt;
        };
        auto loadb = [&](int, int r, int c) {
            const uint32_t ro = (uint32_t)r * rowb;
            PreB x;
            x.in = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, ro + colb(c, false), 0, 0));
            x.gt = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, ro + colb(c, true), 0, 0));
            return x;
        };
        auto fnb = [&](int t, int r, int c, float (&v)[8], const PreB& x) {
            // (a uniform branch: without one per item the compiler
            // interleaves the unrolled items and spills)
            if (uniform(rows_left) > 0) {
                float xin[8], xgt[8], din[8], dgt[8];
                unpack8_16(x.in, kBF16, xin);
                unpack8_16(x.gt, kBF16, xgt);
                grad8(t, v, xin, xgt, a2 * prow[t], din, dgt);
                const uint32_t ro = (uint32_t)r * rowb;
                store_bf16x8(rd, ro + colb(c, false), din);
                store_bf16x8(rd, ro + colb(c, true), dgt);
                if (DB && t == kT - 1 && dbias_ws)
                    dbias_flush(c);
            }
        };
        for_each_row8<C, kAhead, 64, 0, -1, C::kWaves == 4>(acc, elds, loadb, fnb);
    } else {
        using Pre = Pre8<CW, 2>;
        auto load = [&](int, int r, int c) {
            const int rr = am0 + r;
            const bool ok = (rr < rows_valid) & (n0 + bn0 + c < p.N);
            int64_t c_in, c_gt;
            cols(c, c_in, c_gt);
            const int64_t row = m0 + (ok ? rr : 0);
            Pre pre;
            pre.x[0] = rawc_load<CW>(p.c, row * N2 + (ok ? c_in : 0));
            pre.x[1] = rawc_load<CW>(p.c, row * N2 + (ok ? c_gt : 0));
            pre.row = p.prob[row];
            return pre;
        };
        auto fn = [&](int t, int r, int c, float (&v)[8], const Pre& pre) {
            const int rr = am0 + r;
            const int n = n0 + bn0 + c;
            int64_t c_in, c_gt;
            cols(c, c_in, c_gt);
            const bool ok = (rr < rows_valid) & (n < p.N);
            float din[8], dgt[8];
            if constexpr (Q) {
#pragma unroll
                for (int k = 0; k < 8; k++)
                    din[k] = dgt[k] = 0.0f;
            }
            if (ok) {
                const int64_t row = m0 + rr;
                float xin[8], xgt[8];
                rawc_cvt<CW>(pre.x[0], cdt, xin);
                rawc_cvt<CW>(pre.x[1], cdt, xgt);
                grad8(t, v, xin, xgt, a2 * pre.row, din, dgt);
                if constexpr (!Q) {
                    store8(p.d, ddt, row * N2 + c_in, din);
                    store8(p.d, ddt, row * N2 + c_gt, dgt);
                }
            }
            if constexpr (Q) {
                // every lane takes part in the block reductions; lanes off the
                // tile hold zeros and store nothing
                int ein, egt;
                const uint2 qin = fp8_row8<BF8>(din, nc, ein);
                const uint2 qgt = fp8_row8<BF8>(dgt, nc, egt);
                if (ok) {
                    fp8_store_row(p.q, m0 + rr, c_in, qin, ein);
                    fp8_store_row(p.q, m0 + rr, c_gt, qgt, egt);
                }
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    dcol_in[t & 3][k] = din[k];
                    dcol_gt[t & 3][k] = dgt[k];
                }
                if ((t & 3) == 3 && p.q.d_col) {
                    const int r0 = r - 24;                 // this lane's row of item t-3
                    const int64_t rb0 = m0 + am0 + (r0 & ~31), row0 = m0 + am0 + r0;
                    const int left = rows_valid - (am0 + r0);
                    fp8_col_block<BF8>(p.q, nc, dcol_in, rb0, row0, c_in, n < p.N, left);
                    fp8_col_block<BF8>(p.q, nc, dcol_gt, rb0, row0, c_gt, n < p.N, left);
                }
            }
            if (DB && t == kT - 1 && dbias_ws)
                dbias_flush(c);
        };
        for_each_row8<C, kAhead>(acc, elds, load, fn);
    }
    // dprob: the 8 lanes of a row hold its partial sums; one atomic per row
    // and wave.
#pragma unroll
    for (int t = 0; t < kT; t++) {
        const float v = row8_sum(rowsum[t] * a2);
        const int rr = am0 + (l >> 3) + 8 * t;
        if ((l & 7) == 4 && rr < rows_valid && n0 + bn0 < p.N)
            atomicAdd(p.dprob + m0 + rr, v);
    }
    if constexpr (AMAX) {
        if (p.amax) {
            amax_in = wave_max(amax_in);
            amax_gt = wave_max(amax_gt);
            if (l == 0) {
                atomicMax((int*)p.amax + 2 * g, __float_as_int(amax_in));
                atomicMax((int*)p.amax + 2 * g + 1, __float_as_int(amax_gt));
            }
        }
    }
}

}  // namespace gg
