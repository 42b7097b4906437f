// gg_fp8out.hpp -- FP8 (E4M3 or E5M2) output quantization of the
// block-scaled dgrad epilogues: "Grouped GEMM + dGLU (SM100)", "Block-scaled
// contract / Equations", step 3, and the FP8 D_row / D_col with SFD_row /
// SFD_col of the dsReLU page's "Shapes".
//
// Blocks of 32 values (32 columns of a row for D_row, 32 rows of a column for
// D_col) share one E8M0 scale SFD = 2^e, the smallest power of two not below
// norm_const * amax * rcp_max, rcp_max the reciprocal of the format's largest
// value (448 for E4M3, 57344 for E5M2; E8M0 holds powers of two only;
// rounding up keeps every code within that largest value), and
// D_q = fp8(D * norm_const / SFD).  The products are two fp32 roundings, the
// division by 2^e is exact, and the conversion (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32, round to nearest even) sees values clamped to +-max.
// BF8 (a template argument below) selects E5M2.
//
// In the row walk of the epilogues a lane holds 8 consecutive columns of one
// row per item, 4 lanes make a 32-column block (lanes differing in bits 0-1),
// and lanes that differ in bits 3-5 hold the same columns of 8 rows, so the 4
// items t = 4j .. 4j+3 of one quadrant half cover a 32-row block of those
// columns.  Row blocks reduce their amax over 2 lane shuffles; column blocks
// keep the 4 items' values in registers and reduce over 3 shuffles.
#pragma once
#include "gg_internal.hpp"
#include "gg_tile.hpp"

namespace gg {

// The output format's largest value.
template <bool BF8>
constexpr float kFp8Max = BF8 ? 57344.0f : 448.0f;

// Smallest e with 2^e >= fp32(fp32(nc * amax) * fp32(1/max)), in
// [-127, 127]; -127 when the product is 0.
template <bool BF8>
__device__ __forceinline__ int fp8_exponent(float amax, float nc) {
    const float x = __fmul_rn(__fmul_rn(nc, amax), 1.0f / kFp8Max<BF8>);
    if (!(x > 0.0f))
        return -127;
    const uint32_t u = __float_as_uint(x);
    const int E = (int)(u >> 23);                // sign is 0
    const uint32_t m = u & 0x7fffffu;
    if (E == 0xff)
        return 127;
    if (E == 0)                                  // below 2^-126: e is -126 or -127
        return m > (1u << 22) ? -126 : -127;
    const int e = E - 127 + (m != 0u);
    return e > 127 ? 127 : e;
}

// Codes of 2 values into the low (hi false) or high half of `old`.
template <bool BF8>
__device__ __forceinline__ int fp8_cvt2(float a, float b, int old, bool hi) {
    if constexpr (BF8)
        return hi ? __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, true)
                  : __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, false);
    else
        return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
                  : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Codes of 4 values scaled by nc / 2^e, packed little-endian.
template <bool BF8>
__device__ __forceinline__ uint32_t fp8_pack4(float v0, float v1, float v2, float v3, int e, float nc) {
    auto s = [&](float v) {
        const float q = ldexpf(__fmul_rn(v, nc), -e);
        return fminf(fmaxf(q, -kFp8Max<BF8>), kFp8Max<BF8>);
    };
    const int lo = fp8_cvt2<BF8>(s(v0), s(v1), 0, false);
    return (uint32_t)fp8_cvt2<BF8>(s(v2), s(v3), lo, true);
}

// Row block of the item's 8 values (32 columns over 4 lanes): every lane of
// the wave takes part; the item's codes and exponent are returned.
template <bool BF8>
__device__ __forceinline__ uint2 fp8_row8(const float (&v)[8], float nc, int& e) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++)
        m = fmaxf(m, fabsf(v[k]));
    m = quad_max(m);
    e = fp8_exponent<BF8>(m, nc);
    return uint2{fp8_pack4<BF8>(v[0], v[1], v[2], v[3], e, nc),
                 fp8_pack4<BF8>(v[4], v[5], v[6], v[7], e, nc)};
}

// Writes an item's row-quantized codes (8 bytes) and, from the block's first
// lane, its scale byte.
__device__ __forceinline__ void fp8_store_row(const Fp8Out& q, int64_t row, int64_t col, uint2 codes,
                                              int e) {
    *reinterpret_cast<uint2*>(q.d_row + row * q.W + col) = codes;
    if ((threadIdx.x & 3) == 0)
        q.sfd_row[row * (q.W / 32) + col / 32] = (uint8_t)(e + 127);
}

// Column blocks of 8 columns over the 4 items d[0..3] of this lane, rows
// row0 + 8 i, in the 32-row block that starts at row rb0: every lane takes
// part; item i is stored when col_ok and 8 i < rows_left (rows_left: valid
// rows from row0 on).
template <bool BF8>
__device__ __forceinline__ void fp8_col_block(const Fp8Out& q, float nc, const float (&d)[4][8],
                                              int64_t rb0, int64_t row0, int64_t col, bool col_ok,
                                              int rows_left) {
    int e[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        float m = fmaxf(fmaxf(fabsf(d[0][k]), fabsf(d[1][k])), fmaxf(fabsf(d[2][k]), fabsf(d[3][k])));
        m = cols8(m, MaxOp());
        e[k] = fp8_exponent<BF8>(m, nc);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (col_ok && 8 * i < rows_left) {
            auto c = [&](int k) {
                return fminf(fmaxf(ldexpf(__fmul_rn(d[i][k], nc), -e[k]), -kFp8Max<BF8>),
                             kFp8Max<BF8>);
            };
            const int lo0 = fp8_cvt2<BF8>(c(0), c(1), 0, false);
            const uint32_t w0 = (uint32_t)fp8_cvt2<BF8>(c(2), c(3), lo0, true);
            const int lo1 = fp8_cvt2<BF8>(c(4), c(5), 0, false);
            const uint32_t w1 = (uint32_t)fp8_cvt2<BF8>(c(6), c(7), lo1, true);
            *reinterpret_cast<uint2*>(q.d_col + (row0 + 8 * i) * q.W + col) = uint2{w0, w1};
        }
    }
    // the block's first row holds its scales
    if (col_ok && rows_left > 0 && row0 == rb0) {
#pragma unroll
        for (int k = 0; k < 8; k++)
            q.sfd_col[(col + k) * q.pitch + rb0 / 32] = (uint8_t)(e[k] + 127);
    }
}

}  // namespace gg
