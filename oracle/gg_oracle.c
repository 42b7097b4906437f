/*
 * gg_oracle.c -- plain, slow CPU oracle for the grouped GEMMs of the MoE
 * expert backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  The HIP product path never calls it,
 * and it shares no code, header, table or constant with that path.
 *
 * What it follows (NVIDIA cuDNN frontend documentation pages):
 *   [W] "Grouped GEMM + WGrad (Unified)": section "Operation" (the per-expert
 *       token slice and the accumulate/overwrite rule), section "BF16
 *       contract" (shapes, strides and majors of A, B, offsets and outputs),
 *       section "Block-scaled contract" (the same operation on block-scaled
 *       operands; MXFP8 here).
 *   [G] "Grouped GEMM + dGLU (SM100)": "BF16 contract / Tensors, layouts, and
 *       equation" (R_g = alpha_g^2 A_g B_g^T, X_g = beta_g C_g, the dSwiGLU and
 *       dGeGLU formulas, dprob and dbias), and "Block-scaled contract /
 *       Equations", steps 1 and 2 (the dequantized GEMM, interleave order,
 *       dprob reduction), "Equations" for dSiTU-GLU (T_g, T_u and their
 *       derivatives) and "Shapes" (per-group amax of shape (L, 2, 1)).
 *   [S] "Grouped GEMM + dsReLU (SM100)": "Equations" (G, D_row, dprob), and
 *       "Shapes" (per-expert Amax; FP8 D_row / D_col with SFD_row / SFD_col).
 *   [G] step 3 (optional quantized output): orc_quant_fp8.
 *
 * Arithmetic: every input is decoded exactly into double; every sum is taken
 * in double in the plain index order; outputs are rounded once, to nearest
 * even, by the encoders below.  The one deliberate fp32 step is X = beta*C of
 * [G], formed as a single fp32 product, because the clamp and filter tests of
 * dGeGLU compare X with +-7 and the product is what the method feeds them.
 * The FP8 output quantization of step 3 decides its scale exponents and
 * codes exactly, from the double D.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops of this file use (reported with its timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Sets that thread count (n >= 1), e.g. 1 to time a single core. */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* dtype codes used by this file (its own numbering) */
enum { ORC_BF16 = 0, ORC_F16 = 1, ORC_F32 = 2, ORC_E4M3 = 3, ORC_E5M2 = 4 };

/* ------------------------------------------------------------------------ */
/* Decoders: bit pattern -> exact double.                                    */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32: shift it back in place. */
double orc_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_double(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                    /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 15 - 10);   /* 1.m * 2^(e-15) */
    return s ? -v : v;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite 448.  The dGLU page names the
 * torch dtype float8_e4m3fn for FP8 operands. */
double orc_e4m3_to_double(uint8_t q) {
    int s = (q >> 7) & 1, e = (q >> 3) & 0xf, m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                     /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp((double)(m + 8), e - 7 - 3);        /* 1.m * 2^(e-7) */
    return s ? -v : v;
}

/* OCP FP8 E5M2 ("e5m2"): 1 sign, 5 exponent (bias 15), 2 fraction bits, with
 * infinities (S.11111.00) and NaNs (S.11111.xx, xx != 0); largest finite
 * 57344.  The pages list float8_e5m2 beside float8_e4m3fn for FP8 operands,
 * C and D ("Grouped GEMM + dGLU (SM100)", "Support Surface and Constraints /
 * Data Types"). */
double orc_e5m2_to_double(uint8_t q) {
    int s = (q >> 7) & 1, e = (q >> 2) & 0x1f, m = q & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);                    /* subnormal: m/4 * 2^-14 */
    else
        v = ldexp((double)(m + 4), e - 15 - 2);       /* 1.m * 2^(e-15) */
    return s ? -v : v;
}

/* E4M3 (fmt 0) or E5M2 (fmt 1) code to its exact value. */
static double fp8_decode(uint8_t q, int fmt) {
    return fmt ? orc_e5m2_to_double(q) : orc_e4m3_to_double(q);
}

/* OCP E8M0 scale ("float8_e8m0fnu"): the byte is a biased power-of-two
 * exponent, value 2^(e-127); 0xFF is NaN. */
double orc_e8m0_to_double(uint8_t e) {
    if (e == 0xff)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

double orc_decode(const void* base, int dtype, int64_t i) {
    switch (dtype) {
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[i]);
    case ORC_F16:  return orc_f16_to_double(((const uint16_t*)base)[i]);
    case ORC_E4M3: return orc_e4m3_to_double(((const uint8_t*)base)[i]);
    case ORC_E5M2: return orc_e5m2_to_double(((const uint8_t*)base)[i]);
    default:       return (double)((const float*)base)[i];
    }
}

/* ------------------------------------------------------------------------ */
/* Encoders: double -> nearest representable value, ties to even, rounded    */
/* once from the double (no intermediate fp32 step).                         */
/* ------------------------------------------------------------------------ */

/* Round |x| to a binary format with p significand bits (hidden bit included)
 * and minimum normal exponent emin; returns the rounded magnitude as a double
 * (exact in that format) or +inf when it exceeds maxfin after rounding. */
static double round_format(double ax, int p, int emin, double maxfin) {
    int E;
    if (ax == 0.0 || isnan(ax) || isinf(ax))
        return ax;
    frexp(ax, &E);                 /* ax = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                 /* ax in [2^e, 2^(e+1)) */
    if (e < emin)
        e = emin;                  /* subnormal range: fixed spacing */
    int ulp = e - (p - 1);
    double q = ldexp(ax, -ulp);    /* exact: scaling by a power of two */
    double r = nearbyint(q);       /* default rounding mode: ties to even */
    double y = ldexp(r, ulp);
    /* Overflow: IEEE rounds to infinity once the rounded value passes the
     * largest finite number. */
    if (y > maxfin)
        return INFINITY;
    return y;
}

uint16_t orc_double_to_bf16(double x) {
    if (isnan(x))
        return 0x7fc0;
    double y = round_format(fabs(x), 8, -126, ldexp(255.0, 120)); /* max (2-2^-7)*2^127 */
    float f = (float)y;            /* exact: y is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u >> 16) | (signbit(x) ? 0x8000u : 0u));
}

uint16_t orc_double_to_f16(double x) {
    if (isnan(x))
        return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000u : 0u;
    double y = round_format(fabs(x), 11, -14, 65504.0);
    if (isinf(y))
        return s | 0x7c00;
    if (y == 0.0)
        return s;
    int E;
    frexp(y, &E);
    int e = E - 1;
    if (e < -14)                                   /* subnormal: y = m * 2^-24 */
        return s | (uint16_t)(int)ldexp(y, 24);
    int m = (int)(ldexp(y, -e) * 1024.0) - 1024;   /* exact: 10 fraction bits */
    return s | (uint16_t)(((e + 15) << 10) | m);
}

float orc_double_to_f32(double x) {
    if (isnan(x))
        return NAN;
    double y = round_format(fabs(x), 24, -126, ldexp(16777215.0, 104));
    float f = (float)y;            /* exact */
    return signbit(x) ? -f : f;
}

/* The two FP8 formats' parameters: fraction bits, minimum normal exponent,
 * exponent bias and largest finite value (E4M3 "float8_e4m3fn": 3, -6, 7,
 * 448 = 7 * 2^6; E5M2 "float8_e5m2": 2, -14, 15, 57344 = 7 * 2^13). */
static const int kFp8Frac[2] = {3, 2}, kFp8Emin[2] = {-6, -14}, kFp8Bias[2] = {7, 15};
static const double kFp8Max[2] = {448.0, 57344.0};
static const int kFp8MaxExp[2] = {6, 13};      /* max = 7 * 2^kFp8MaxExp */

/* FP8 code (fmt 0: E4M3, 1: E5M2) of the exact value hi + lo, where lo is
 * the rounding error of hi (|lo| <= half an ulp of hi, the same sign
 * convention as the value), by round-to-nearest-even; magnitudes above the
 * format's largest finite value are clamped to it first (so neither
 * format's infinities or NaNs result from a finite input).  hi is the
 * double nearest to the value, so the value and hi fall on the same side of
 * every FP8 rounding midpoint except when hi is that midpoint: then lo
 * decides the direction. */
static uint8_t fp8_of_sum(double hi, double lo, int fmt) {
    const int fb = kFp8Frac[fmt], emin = kFp8Emin[fmt], bias = kFp8Bias[fmt];
    const double maxfin = kFp8Max[fmt];
    if (isnan(hi))
        return 0x7f;                              /* NaN in both: S.1111.111, S.11111.11 */
    uint8_t s = signbit(hi) ? 0x80u : 0u;
    double ax = fabs(hi), alo = signbit(hi) ? -lo : lo;   /* value = ax + alo, >= 0 */
    double y;
    if (ax >= maxfin) {
        y = maxfin;
    } else if (ax == 0.0) {
        y = 0.0;
    } else {
        int E;
        frexp(ax, &E);
        int e = E - 1 < emin ? emin : E - 1;      /* ax in [2^e, 2^(e+1)) or subnormal */
        int ulp = e - fb;
        double q = ldexp(ax, -ulp);               /* exact */
        double fl = floor(q);
        double r;
        if (q - fl == 0.5 && alo != 0.0)
            r = alo > 0.0 ? fl + 1.0 : fl;        /* the value lies off the midpoint */
        else
            r = nearbyint(q);                     /* ties to even */
        y = ldexp(r, ulp);
        if (y > maxfin)
            y = maxfin;
    }
    if (y == 0.0)
        return s;
    int E;
    frexp(y, &E);
    int e = E - 1;
    if (e < emin)                                  /* subnormal: y = m * 2^(emin - fb) */
        return s | (uint8_t)(int)ldexp(y, fb - emin);
    int m = (int)(ldexp(y, -e) * (double)(1 << fb)) - (1 << fb);   /* exact */
    return s | (uint8_t)(((e + bias) << fb) | m);
}

static uint8_t e4m3_of_sum(double hi, double lo) { return fp8_of_sum(hi, lo, 0); }

uint8_t orc_double_to_e4m3(double x) { return e4m3_of_sum(x, 0.0); }
uint8_t orc_double_to_e5m2(double x) { return fp8_of_sum(x, 0.0, 1); }

/* [G] "Block-scaled contract / Equations", step 3 (and the FP8 D_row / D_col
 * with SFD_row / SFD_col of [S] "Shapes"): blocks of 32 values (32 columns of
 * a row for D_row, 32 rows of a column for D_col) share one E8M0 scale
 *   SFD = norm_const * max|D| * rcp_max,   D_q = D * norm_const / SFD,
 * with rcp_max the reciprocal of the output format's largest value (1/448
 * for E4M3, 1/57344 for E5M2: the reading of rcp_max used here).  E8M0
 * holds powers of two only: SFD is taken as the smallest power of two 2^e
 * not below the product (so |D_q| <= the largest value), e clamped to
 * [-127, 127], e = -127 for an all-zero block.  Both the exponent and the
 * codes are decided in exact arithmetic on the double D: no intermediate
 * rounding of D, of the product or of the quotient. */

/* Smallest integer e with 2^e >= norm_const * amax / (7 * 2^k), k = 6 for
 * E4M3 (448) and 13 for E5M2 (57344), exactly: with amax = ia 2^(ea-53) and
 * norm_const = in 2^(en-24) (integer significands from frexp; a float's fits
 * 24 bits, a double's 53), the condition reads
 * 7 * 2^(e + k + 77 - ea - en) >= ia * in, a comparison of integers below
 * 2^80. */
static int fp8_block_exponent(double amax, float norm_const, int fmt) {
    double nc = (double)norm_const;
    if (!(amax > 0.0) || !(nc > 0.0))
        return -127;
    if (isinf(amax) || isinf(nc))
        return 127;
    int ea, en;
    double fa = frexp(amax, &ea), fn = frexp(nc, &en);
    unsigned __int128 prod = (unsigned __int128)(uint64_t)ldexp(fa, 53) *
                             (unsigned __int128)(uint64_t)ldexp(fn, 24);
    int s = 0;
    while (((unsigned __int128)7 << s) < prod)
        s++;
    int e = s - kFp8MaxExp[fmt] - 77 + ea + en;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

/* FP8 code of d * norm_const * 2^-e: the product is split exactly into its
 * double rounding and that rounding's error (a fused multiply-add recovers
 * the error exactly), and scaling by 2^-e is exact. */
static uint8_t fp8_quantize(double d, float norm_const, int e, int fmt) {
    double nc = (double)norm_const;
    double hi = d * nc;
    double lo = fma(d, nc, -hi);
    return fp8_of_sum(ldexp(hi, -e), ldexp(lo, -e), fmt);
}

/* D (nrows, W) doubles, W a multiple of 32; fmt 0: E4M3, 1: E5M2 codes.
 * q_row (nrows, W) codes and sfd_row (nrows, W/32) E8M0: row blocks; if q_col
 * is non-NULL (nrows a multiple of 32, consecutive rows): q_col (nrows, W)
 * and sfd_col (W, nrows/32), column blocks of rows 32j .. 32j+31. */
void orc_quant_fp8(const double* D, int64_t nrows, int W, float norm_const, int fmt,
                   uint8_t* q_row, uint8_t* sfd_row, uint8_t* q_col, uint8_t* sfd_col) {
    int WB = W / 32;
    for (int64_t r = 0; r < nrows; r++)
        for (int b = 0; b < WB; b++) {
            double amax = 0.0;
            for (int k = 0; k < 32; k++) {
                double v = fabs(D[r * W + 32 * b + k]);
                amax = v > amax ? v : amax;
            }
            int e = fp8_block_exponent(amax, norm_const, fmt);
            sfd_row[r * WB + b] = (uint8_t)(e + 127);
            for (int k = 0; k < 32; k++)
                q_row[r * W + 32 * b + k] = fp8_quantize(D[r * W + 32 * b + k], norm_const, e, fmt);
        }
    if (!q_col)
        return;
    int64_t RB = nrows / 32;
    for (int c = 0; c < W; c++)
        for (int64_t j = 0; j < RB; j++) {
            double amax = 0.0;
            for (int k = 0; k < 32; k++) {
                double v = fabs(D[(32 * j + k) * W + c]);
                amax = v > amax ? v : amax;
            }
            int e = fp8_block_exponent(amax, norm_const, fmt);
            sfd_col[(int64_t)c * RB + j] = (uint8_t)(e + 127);
            for (int k = 0; k < 32; k++)
                q_col[(32 * j + k) * W + c] =
                    fp8_quantize(D[(32 * j + k) * W + c], norm_const, e, fmt);
        }
}

/* Round n doubles to dtype and store them into out (uint16 or float). */
void orc_round_array(const double* in, int64_t n, int dtype, void* out) {
    for (int64_t i = 0; i < n; i++) {
        if (dtype == ORC_BF16)
            ((uint16_t*)out)[i] = orc_double_to_bf16(in[i]);
        else if (dtype == ORC_F16)
            ((uint16_t*)out)[i] = orc_double_to_f16(in[i]);
        else
            ((float*)out)[i] = orc_double_to_f32(in[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* [W] Grouped wgrad.                                                        */
/* ------------------------------------------------------------------------ */

/* Expert e owns the token slice [begin, end): begin is 0 for the first expert
 * and offsets[e-1] otherwise, end is offsets[e] ([W] "Operation").  The result
 * is Wgrad[e] = A[:, begin:end] @ B[begin:end, :].
 *
 * A is (hidden, T): a_major 0 = K-major, element (h,t) at h*T + t;
 *                    a_major 1 = M-major, element (h,t) at t*hidden + h.
 * B is (T, inter):  b_major 0 = K-major, element (t,i) at i*T + t;
 *                    b_major 1 = N-major, element (t,i) at t*inter + i.
 * ([W] "BF16 contract": strides (T,1) / (1,hidden) for A and (1,T) /
 * (inter,1) for B.)
 *
 * out is the exact product, in double, for the rows listed in hrows (all
 * hidden rows when hrows is NULL), as out[(e*nrows + r)*inter + i].  The
 * accumulate/overwrite rule and the output rounding are applied by
 * orc_wgrad_finish. */
void orc_wgrad(const uint16_t* A, int a_major, const uint16_t* B, int b_major,
               const int32_t* offsets, int E, int64_t T, int hidden, int inter,
               const int32_t* hrows, int nrows, double* out) {
    if (!hrows)
        nrows = hidden;
    for (int e = 0; e < E; e++) {
        int64_t begin = e ? offsets[e - 1] : 0;
        int64_t end = offsets[e];
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = 0; r < nrows; r++) {
            int h = hrows ? hrows[r] : r;
            double* o = out + ((int64_t)e * nrows + r) * inter;
            /* o[i] = sum over t = begin .. end-1, in that order, of A(h,t) B(t,i):
             * the t loop is outside so that B's rows are read in order; each
             * o[i] still adds its terms in increasing t. */
            for (int i = 0; i < inter; i++)
                o[i] = 0.0;
            for (int64_t t = begin; t < end; t++) {
                int64_t ia = a_major == 0 ? (int64_t)h * T + t : t * hidden + h;
                double av = orc_bf16_to_double(A[ia]);
                for (int i = 0; i < inter; i++) {
                    int64_t ib = b_major == 0 ? (int64_t)i * T + t : t * inter + i;
                    o[i] += av * orc_bf16_to_double(B[ib]);
                }
            }
        }
    }
}

/* [W] "Block-scaled contract" on MXFP8 operands: the "Operation" of the page
 * with every operand value dequantized, deq(q) = fp8(q) * 2^(e8m0 - 127),
 * fp8 the E4M3 (ab_fmt 0) or E5M2 (ab_fmt 1) value of the code,
 * one E8M0 scale per 32 consecutive tokens (the K axis) of a row.
 *   A (hidden, T) K-major codes: (h,t) at h*T + t; SFA (hidden, T/32):
 *     SFA[h*(T/32) + t/32].
 *   B (T, inter) stored K-major, i.e. as an (inter, T) array of codes:
 *     (t,i) at i*T + t; SFB (inter, T/32): SFB[i*(T/32) + t/32].
 * Outputs as for orc_wgrad (exact products, in double, per listed row); the
 * accumulate rule and the rounding are orc_wgrad_finish's. */
void orc_wgrad_mx(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                  int ab_fmt, const int32_t* offsets, int E, int64_t T, int hidden, int inter,
                  const int32_t* hrows, int nrows, double* out) {
    if (!hrows)
        nrows = hidden;
    int64_t TB = T / 32;
    for (int e = 0; e < E; e++) {
        int64_t begin = e ? offsets[e - 1] : 0;
        int64_t end = offsets[e];
        int64_t cnt = end > begin ? end - begin : 0;
        /* the expert's B values, dequantized once: Bd[(t - begin)*inter + i] */
        double* Bd = (double*)malloc(sizeof(double) * (size_t)(cnt * inter > 0 ? cnt * inter : 1));
#pragma omp parallel for schedule(static)
        for (int i = 0; i < inter; i++)
            for (int64_t t = begin; t < end; t++)
                Bd[(t - begin) * inter + i] = fp8_decode(B[(int64_t)i * T + t], ab_fmt) *
                                              orc_e8m0_to_double(SFB[(int64_t)i * TB + t / 32]);
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = 0; r < nrows; r++) {
            int h = hrows ? hrows[r] : r;
            double* o = out + ((int64_t)e * nrows + r) * inter;
            /* o[i] = sum over t = begin .. end-1, in that order, of A(h,t) B(t,i) */
            for (int i = 0; i < inter; i++)
                o[i] = 0.0;
            for (int64_t t = begin; t < end; t++) {
                double av = fp8_decode(A[(int64_t)h * T + t], ab_fmt) *
                            orc_e8m0_to_double(SFA[(int64_t)h * TB + t / 32]);
                const double* bt = Bd + (t - begin) * inter;
                for (int i = 0; i < inter; i++)
                    o[i] += av * bt[i];
            }
        }
        free(Bd);
    }
}

/* [W] "Operation": with accumulate on, the result is added to the existing
 * output; with it off the output is overwritten (an empty expert therefore
 * yields zero).  One rounding to the output dtype after the sum.
 * old and res have n elements in the output dtype; exact holds the doubles. */
void orc_wgrad_finish(const double* exact, int64_t n, int accumulate,
                      const void* old, int dtype, void* res) {
    for (int64_t j = 0; j < n; j++) {
        double y = exact[j];
        if (accumulate)
            y += orc_decode(old, dtype, j);
        if (dtype == ORC_BF16)
            ((uint16_t*)res)[j] = orc_double_to_bf16(y);
        else if (dtype == ORC_F16)
            ((uint16_t*)res)[j] = orc_double_to_f16(y);
        else
            ((float*)res)[j] = orc_double_to_f32(y);
    }
}

/* ------------------------------------------------------------------------ */
/* Groups of rows (dGLU and dsReLU pages): group g owns rows                 */
/* [padded_offsets[g-1], padded_offsets[g]), with padded_offsets[-1] = 0.    */
/* ------------------------------------------------------------------------ */
static int group_of_row(const int32_t* po, int L, int64_t m) {
    int64_t lo = 0;
    for (int g = 0; g < L; g++) {
        if (m >= lo && m < po[g])
            return g;
        lo = po[g];
    }
    return -1;                     /* at or beyond valid_m = po[L-1] */
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* ------------------------------------------------------------------------ */
/* [G] Grouped dgrad + dSwiGLU / dGeGLU.                                     */
/* ------------------------------------------------------------------------ */

/* Inputs:
 *   A (M, K) bf16, row-major (K-major): A[m*K + k].
 *   Bp[g] -> expert g's (N, K) bf16 matrix; b_major 0: (n,k) at n*K + k,
 *            b_major 1: (n,k) at k*N + n.  (Dense B of shape (N,K,L) is the
 *            case Bp[g] = B + g*N*K with b_major 0.)
 *   C (M, 2N), row-major, c_dtype; alpha, beta (L) fp32; prob (M) fp32.
 *   act 0 = dSwiGLU, 1 = dGeGLU with constants ga (1.702), clamp_lo (-7),
 *   clamp_hi (7) and linear offset lo (1); 2 = dSiTU-GLU with tanh scales
 *   situ_b1 (4) and situ_b2 (25), block-scaled only (orc_dglu_mx).
 *   gate_first 0: in every 64-column pair of C and D the first 32 columns are
 *   the input block and the next 32 the gate block ("interleaved input/gate",
 *   and the step that interleaves [ab, dswiglu]); 1 swaps the two.
 *   mask_filter 0: dGeGLU's filters carry the raw value, as the page defines
 *   gate_filter / input_filter; 1: they are the 0/1 indicator.
 * Rows listed in rows (all rows < M when rows is NULL) are computed; a row at
 * or beyond valid_m = po[L-1] belongs to no group and is left untouched.
 * Outputs (double, unrounded):
 *   D[r*2N + c]     the interleaved gradient for listed row r;
 *   dprob_sum[r]    sum over n of R * (unscaled activation);
 *   dbias_sum[g*2N + c]  (if non-NULL) sum over the listed rows of group g. */
/* The dGLU epilogue of [G] for one row m of group g, given that row's R
 * values R[n], n < N: writes the interleaved gradient D[0 .. 2N) and returns
 * the dprob sum.  Arguments as for orc_dglu. */
static double dglu_row(const double* R, int64_t m, int g, int N,
                       const void* C, int c_dtype, const float* beta, const float* prob,
                       int act, double ga, double clamp_lo, double clamp_hi, double lo,
                       double situ_b1, double situ_b2, int gate_first, int mask_filter,
                       double* D) {
    int64_t N2 = 2 * (int64_t)N;
    double pr = (double)prob[m];
    double dp = 0.0;
    for (int n = 0; n < N; n++) {
        /* 32-wide blocks: compact column n sits in pair p at offset j. */
        int p = n / 32, j = n % 32;
        int64_t c_in = 64 * (int64_t)p + (gate_first ? 32 : 0) + j;
        int64_t c_gt = 64 * (int64_t)p + (gate_first ? 0 : 32) + j;
        /* X = beta_g * C as one fp32 product (see the file header). */
        float xin = beta[g] * (float)orc_decode(C, c_dtype, m * N2 + c_in);
        float xgt = beta[g] * (float)orc_decode(C, c_dtype, m * N2 + c_gt);
        double u = xin, gt = xgt, d_in, d_gt, a;
        if (act == 0) {
            /* dSwiGLU with s = sigmoid(gate):
             *   dinput = R prob gate s
             *   dgate  = R prob input s (1 + gate (1 - s))
             * and the unscaled activation is swish(gate) * input. */
            double s = sigmoid(gt);
            d_in = R[n] * pr * gt * s;
            d_gt = R[n] * pr * u * s * (1.0 + gt * (1.0 - s));
            a = gt * s * u;
        } else if (act == 2) {
            /* dSiTU-GLU: T_g = b1 tanh(gate/b1) s, T_u = b2 tanh(input/b2),
             * s = sigmoid(gate);
             *   dT_g/dgate  = (1 - tanh^2(gate/b1)) s + b1 tanh(gate/b1) s (1 - s)
             *   dT_u/dinput = 1 - tanh^2(input/b2)
             *   dgate  = R prob T_u dT_g/dgate
             *   dinput = R prob T_g dT_u/dinput
             * and the unscaled activation is T_g T_u. */
            double s = sigmoid(gt);
            double tg = tanh(gt / situ_b1), tu = tanh(u / situ_b2);
            double Tg = situ_b1 * tg * s, Tu = situ_b2 * tu;
            double dTg = (1.0 - tg * tg) * s + situ_b1 * tg * s * (1.0 - s);
            double dTu = 1.0 - tu * tu;
            d_gt = R[n] * pr * Tu * dTg;
            d_in = R[n] * pr * Tg * dTu;
            a = Tg * Tu;
        } else {
            /* dGeGLU: clamped values feed the activation, the filters
             * carry the raw value where it lies inside the clamp. */
            double gc = gt < clamp_hi ? gt : clamp_hi;
            double uc = u < clamp_lo ? clamp_lo : (u > clamp_hi ? clamp_hi : u);
            int g_in = gt <= clamp_hi;
            int u_in = u >= clamp_lo && u <= clamp_hi;
            double gf = g_in ? (mask_filter ? 1.0 : gt) : 0.0;
            double uf = u_in ? (mask_filter ? 1.0 : u) : 0.0;
            double s = sigmoid(ga * gc);
            d_gt = R[n] * pr * (uc + lo) * s * (1.0 + ga * gc * (1.0 - s)) * gf;
            d_in = R[n] * pr * gc * s * uf;
            a = gc * s * (uc + lo);
        }
        dp += R[n] * a;
        D[c_in] = d_in;
        D[c_gt] = d_gt;
    }
    return dp;
}

/* dbias of [G]: per-expert row reduction of the interleaved output over the
 * listed rows. */
static void dglu_dbias(const double* D, const int32_t* po, int L, int N, const int64_t* rows,
                       int64_t nrows, double* dbias_sum) {
    int64_t N2 = 2 * (int64_t)N;
    for (int64_t r = 0; r < nrows; r++) {
        int64_t m = rows ? rows[r] : r;
        int g = group_of_row(po, L, m);
        if (g < 0)
            continue;
        for (int64_t c = 0; c < N2; c++)
            dbias_sum[g * N2 + c] += D[r * N2 + c];
    }
}

/* The listed rows (indices r into the row list) that belong to group g, in
 * list order; returns their count.  grp[r] holds each listed row's group. */
static int64_t rows_of_group(const int* grp, int64_t nrows, int g, int64_t* idx) {
    int64_t n = 0;
    for (int64_t r = 0; r < nrows; r++)
        if (grp[r] == g)
            idx[n++] = r;
    return n;
}

static int* groups_of_rows(const int32_t* po, int L, const int64_t* rows, int64_t nrows) {
    int* grp = (int*)malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    for (int64_t r = 0; r < nrows; r++)
        grp[r] = group_of_row(po, L, rows ? rows[r] : r);
    return grp;
}

/* R_g[m, n] = a2 * sum over k = 0 .. K-1, in that order, of Ad[k] * Bt[k*N + n],
 * for one row (Ad: its K values; Bt: the group's B values as a (K, N)
 * array).  Every R[n] adds its terms in increasing k; the k loop is outside
 * so that Bt's rows are read in order. */
static void row_product(const double* Ad, const double* Bt, int K, int N, double a2, double* R) {
    for (int n = 0; n < N; n++)
        R[n] = 0.0;
    for (int k = 0; k < K; k++) {
        double av = Ad[k];
        const double* bk = Bt + (int64_t)k * N;
        for (int n = 0; n < N; n++)
            R[n] += av * bk[n];
    }
    for (int n = 0; n < N; n++)
        R[n] *= a2;
}

void orc_dglu(const uint16_t* A, int64_t M, int K,
              const uint16_t* const* Bp, int b_major, int N,
              const void* C, int c_dtype, const int32_t* po, int L,
              const float* alpha, const float* beta, const float* prob,
              int act, double ga, double clamp_lo, double clamp_hi, double lo,
              int gate_first, int mask_filter,
              const int64_t* rows, int64_t nrows,
              double* D, double* dprob_sum, double* dbias_sum) {
    if (!rows)
        nrows = M;
    int64_t N2 = 2 * (int64_t)N;
    int* grp = groups_of_rows(po, L, rows, nrows);
    int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
    double* Bt = (double*)malloc(sizeof(double) * (size_t)K * (size_t)N);
    for (int g = 0; g < L; g++) {
        int64_t cnt = rows_of_group(grp, nrows, g, idx);
        if (cnt == 0)
            continue;
        /* expert g's B as a (K, N) array of exact values */
        const uint16_t* Bg = Bp[g];
#pragma omp parallel for schedule(static)
        for (int k = 0; k < K; k++)
            for (int n = 0; n < N; n++)
                Bt[(int64_t)k * N + n] = orc_bf16_to_double(
                    Bg[b_major == 0 ? (int64_t)n * K + k : (int64_t)k * N + n]);
        double a2 = (double)alpha[g] * (double)alpha[g];
#pragma omp parallel
        {
            double* R = (double*)malloc(sizeof(double) * (size_t)N);
            double* Ad = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
            for (int64_t j = 0; j < cnt; j++) {
                int64_t r = idx[j];
                int64_t m = rows ? rows[r] : r;
                for (int k = 0; k < K; k++)
                    Ad[k] = orc_bf16_to_double(A[m * K + k]);
                /* R_g[m, n] = alpha_g^2 * sum_k A[m,k] * B_g[n,k] */
                row_product(Ad, Bt, K, N, a2, R);
                dprob_sum[r] = dglu_row(R, m, g, N, C, c_dtype, beta, prob, act, ga, clamp_lo,
                                        clamp_hi, lo, 0.0, 0.0, gate_first, mask_filter,
                                        D + r * N2);
            }
            free(R);
            free(Ad);
        }
    }
    free(Bt);
    free(idx);
    free(grp);
    if (dbias_sum)
        dglu_dbias(D, po, L, N, rows, nrows, dbias_sum);
}

/* [G] "Block-scaled contract / Equations", steps 1 and 2, on MXFP8 operands:
 * R_g = alpha_g^2 * sum_k deq(A[m,k]) deq(B_g[n,k]), with deq(q) = fp8(q) *
 * 2^(e8m0 - 127) and one E8M0 scale per 32 K values of a row, then the dGLU
 * epilogue of orc_dglu (and dSiTU-GLU, act 2, of the same section).
 *   A (M, K) FP8 codes (ab_fmt 0: E4M3, 1: E5M2), K-major; SFA (M, K/32)
 *   E8M0: SFA[m*(K/32) + k/32].
 *   Bp[g] -> expert g's (N, K) codes, K-major; SFBp[g] -> its (N, K/32).
 *   C may also hold E4M3 or E5M2 codes (c_dtype ORC_E4M3 / ORC_E5M2, the
 *   block-scaled contract's FP8 C), decoded exactly.
 * Other arguments and outputs as for orc_dglu, plus
 *   amax[2g + h] (h 0: the input-gradient columns, 1: the gate-gradient
 *   columns) raised to max |D| over the listed rows of group g (the caller
 *   initialises it). */
void orc_dglu_mx(const uint8_t* A, const uint8_t* SFA, int64_t M, int K,
                 const uint8_t* const* Bp, const uint8_t* const* SFBp, int N, int ab_fmt,
                 const void* C, int c_dtype, const int32_t* po, int L,
                 const float* alpha, const float* beta, const float* prob,
                 int act, double ga, double clamp_lo, double clamp_hi, double lo,
                 double situ_b1, double situ_b2, int gate_first, int mask_filter,
                 const int64_t* rows, int64_t nrows,
                 double* D, double* dprob_sum, double* dbias_sum, double* amax) {
    if (!rows)
        nrows = M;
    int64_t N2 = 2 * (int64_t)N;
    int KB = K / 32;
    int* grp = groups_of_rows(po, L, rows, nrows);
    int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
    double* Bt = (double*)malloc(sizeof(double) * (size_t)K * (size_t)N);
    for (int g = 0; g < L; g++) {
        int64_t cnt = rows_of_group(grp, nrows, g, idx);
        if (cnt == 0)
            continue;
        /* expert g's dequantized B as a (K, N) array */
        const uint8_t* Bg = Bp[g];
        const uint8_t* Sg = SFBp[g];
#pragma omp parallel for schedule(static)
        for (int k = 0; k < K; k++)
            for (int n = 0; n < N; n++)
                Bt[(int64_t)k * N + n] = fp8_decode(Bg[(int64_t)n * K + k], ab_fmt) *
                                         orc_e8m0_to_double(Sg[(int64_t)n * KB + k / 32]);
        double a2 = (double)alpha[g] * (double)alpha[g];
#pragma omp parallel
        {
            double* R = (double*)malloc(sizeof(double) * (size_t)N);
            double* Ad = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
            for (int64_t j = 0; j < cnt; j++) {
                int64_t r = idx[j];
                int64_t m = rows ? rows[r] : r;
                for (int k = 0; k < K; k++)
                    Ad[k] = fp8_decode(A[m * K + k], ab_fmt) *
                            orc_e8m0_to_double(SFA[m * KB + k / 32]);
                row_product(Ad, Bt, K, N, a2, R);
                dprob_sum[r] = dglu_row(R, m, g, N, C, c_dtype, beta, prob, act, ga, clamp_lo,
                                        clamp_hi, lo, situ_b1, situ_b2, gate_first, mask_filter,
                                        D + r * N2);
            }
            free(R);
            free(Ad);
        }
    }
    free(Bt);
    free(idx);
    free(grp);
    if (dbias_sum)
        dglu_dbias(D, po, L, N, rows, nrows, dbias_sum);
    for (int64_t r = 0; r < nrows; r++) {
        int64_t m = rows ? rows[r] : r;
        int g = group_of_row(po, L, m);
        if (g < 0)
            continue;
        for (int64_t c = 0; c < N2; c++) {
            /* column c is an input-gradient column when its 32-block within
             * the 64-column pair is the input block */
            int in_block = ((c % 64) < 32) != (gate_first != 0);
            double v = fabs(D[r * N2 + c]);
            double* slot = &amax[2 * g + (in_block ? 0 : 1)];
            if (v > *slot)
                *slot = v;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* [S] Grouped dgrad + dsReLU on MXFP8 operands.                             */
/* ------------------------------------------------------------------------ */

/* Inputs:
 *   A (M, K) fp8 codes (ab_fmt 0: E4M3, 1: E5M2), row-major; SFA (M, K/32)
 *   e8m0, row-major: one scale
 *   for each 32-element K block of each row.
 *   Bp[g] -> expert g's (N, K) fp8 codes (n,k) at n*K + k; SFBp[g] -> its
 *   (N, K/32) e8m0 scales.
 *   C (M, N) row-major, c_dtype; alpha (L) fp32; prob (M) fp32.
 *   C may also hold E4M3 or E5M2 codes (c_dtype ORC_E4M3 / ORC_E5M2, the
 *   block-scaled contract's FP8 C), decoded exactly.
 * With dequantize(q, s) = fp8(q) * 2^(s-127):
 *   G[m,n]     = alpha_g * sum_k deq(A[m,k]) * deq(B_g[n,k])
 *   D_row[m,n] = prob[m] * 2 * C[m,n] * relu(G[m,n])
 *   dprob[m]   = sum_n C[m,n] * relu(G[m,n])^2
 *   amax[g]    = max |D_row| over the group's rows, before output rounding;
 *                amax is only raised here, the caller starts it at 0.
 * Outputs (double): D[r*N + n], dprob_sum[r], amax[g] for the listed rows. */
void orc_dsrelu(const uint8_t* A, const uint8_t* SFA, int64_t M, int K,
                const uint8_t* const* Bp, const uint8_t* const* SFBp, int N, int ab_fmt,
                const void* C, int c_dtype, const int32_t* po, int L,
                const float* alpha, const float* prob,
                const int64_t* rows, int64_t nrows,
                double* D, double* dprob_sum, double* amax) {
    if (!rows)
        nrows = M;
    int KB = K / 32;
    int* grp = groups_of_rows(po, L, rows, nrows);
    int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
    double* Bt = (double*)malloc(sizeof(double) * (size_t)K * (size_t)N);
    for (int g = 0; g < L; g++) {
        int64_t cnt = rows_of_group(grp, nrows, g, idx);
        if (cnt == 0)
            continue;
        /* expert g's dequantized B as a (K, N) array */
        const uint8_t* Bg = Bp[g];
        const uint8_t* Sg = SFBp[g];
#pragma omp parallel for schedule(static)
        for (int k = 0; k < K; k++)
            for (int n = 0; n < N; n++)
                Bt[(int64_t)k * N + n] = fp8_decode(Bg[(int64_t)n * K + k], ab_fmt) *
                                         orc_e8m0_to_double(Sg[(int64_t)n * KB + k / 32]);
#pragma omp parallel
        {
            double* G = (double*)malloc(sizeof(double) * (size_t)N);
            double* Ad = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
            for (int64_t j = 0; j < cnt; j++) {
                int64_t r = idx[j];
                int64_t m = rows ? rows[r] : r;
                for (int k = 0; k < K; k++)
                    Ad[k] = fp8_decode(A[m * K + k], ab_fmt) *
                            orc_e8m0_to_double(SFA[m * KB + k / 32]);
                /* G[m, n] = alpha_g * sum_k deq(A[m,k]) * deq(B_g[n,k]) */
                row_product(Ad, Bt, K, N, (double)alpha[g], G);
                double pr = (double)prob[m];
                double dp = 0.0;
                for (int n = 0; n < N; n++) {
                    double rl = G[n] > 0.0 ? G[n] : 0.0;
                    double c = orc_decode(C, c_dtype, m * (int64_t)N + n);
                    D[r * (int64_t)N + n] = pr * 2.0 * c * rl;
                    dp += c * rl * rl;
                }
                dprob_sum[r] = dp;
            }
            free(G);
            free(Ad);
        }
    }
    free(Bt);
    free(idx);
    free(grp);
    for (int64_t r = 0; r < nrows; r++) {
        int64_t m = rows ? rows[r] : r;
        int g = group_of_row(po, L, m);
        if (g < 0)
            continue;
        for (int n = 0; n < N; n++) {
            double v = fabs(D[r * (int64_t)N + n]);
            if (v > amax[g])
                amax[g] = v;
        }
    }
}
