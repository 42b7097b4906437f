// gg_wgrad_epi.hpp -- the output epilogue of the grouped wgrad kernels
// (bf16 and block-scaled main loops alike): Wgrad[e] is written, or added to
// the existing output when accumulating ("Grouped GEMM + WGrad (Unified)",
// "Operation"), rounded to nearest even in the output dtype.
#pragma once
#include "gg_internal.hpp"
#include "gg_tile.hpp"

namespace gg {

// Output: rows of 8 consecutive columns per lane (one 16-byte store for
// bf16/fp16, two for fp32).  The format and the mode are compile-time, so an
// item costs exactly the memory instructions it needs: an overwrite issues
// its stores only, an accumulation also its loads of the old values, issued
// 8 items ahead.  Items off the tile have masked offsets (kInvalid: the load
// returns zeros, the store writes nothing).  The stores are non-temporal:
// the output is not read again by the kernel, and streaming it past the
// caches measured 3-6% faster on the MoE shapes.
template <class C, int kQR, int DT, bool ACC, int kFrom, int kTo>
__device__ __forceinline__ void wgrad_epilogue_t(const f32x16 (&acc)[C::MB][C::NB], float* lds,
                                                 void* out, int hidden, int inter, int row0,
                                                 int col0) {
    constexpr bool W32 = DT == kF32;
    constexpr int kShift = W32 ? 2 : 1;
    constexpr int kNT = 2;     // cache policy of the buffer stores: non-temporal
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    // offsets (r inter + col) elements from the wave tile's first row: r < 128,
    // col < inter <= 2^21, so they fit 32 bits in bytes
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)out + ((int64_t)row0 * inter << kShift));
    auto off = [&](int r, int c) {
        const bool ok = (row0 + r < hidden) & (col0 + c < inter);
        return ok ? (uint32_t)(((int64_t)r * inter + col0 + c) << kShift) : kInvalid;
    };
    struct Old {
        u32x4 w[ACC && W32 ? 2 : 1];
    };
    auto load = [&](int, int r, int c) {
        Old x;
        if constexpr (ACC) {
            const uint32_t o = off(r, c);
            x.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, o, 0, 0));
            if constexpr (W32)
                x.w[1] = __builtin_bit_cast(u32x4,
                                            __builtin_amdgcn_raw_buffer_load_b128(ro, o + 16, 0, 0));
        }
        return x;
    };
    auto fn = [&](int, int r, int c, float (&v)[8], const Old& x) {
        if constexpr (ACC) {
            float o[8];
            if constexpr (W32) {
                const uint32_t ws[8] = {x.w[0].x, x.w[0].y, x.w[0].z, x.w[0].w,
                                        x.w[1].x, x.w[1].y, x.w[1].z, x.w[1].w};
#pragma unroll
                for (int k = 0; k < 8; k++)
                    o[k] = __builtin_bit_cast(float, ws[k]);
            } else {
                unpack8_16(x.w[0], DT, o);
            }
#pragma unroll
            for (int k = 0; k < 8; k++)
                v[k] += o[k];
        }
        const uint32_t o = off(r, c);
        if constexpr (W32) {
            i32x4 lo, hi;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                lo[k] = __builtin_bit_cast(int, v[k]);
                hi[k] = __builtin_bit_cast(int, v[4 + k]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(lo, ro, o, 0, kNT);
            __builtin_amdgcn_raw_buffer_store_b128(hi, ro, o + 16, 0, kNT);
        } else {
            i32x4 w;
#pragma unroll
            for (int k = 0; k < 4; k++)
                w[k] = DT == kBF16 ? (int)pack_bf16x2(v[2 * k], v[2 * k + 1])
                                   : (int)((uint32_t)f32_to_f16(v[2 * k]) |
                                           ((uint32_t)f32_to_f16(v[2 * k + 1]) << 16));
            __builtin_amdgcn_raw_buffer_store_b128(w, ro, o, 0, kNT);
        }
    };
    for_each_row8<C, ACC ? 8 : 1, kQR, kFrom, kTo>(acc, lds, load, fn);
}

// bf16 output, overwritten, from accumulators in the transposed layout of
// mma_bf16<C, true>: block row kI (32 rows x 32 NB columns of the wave
// tile) is rounded to bf16 and staged through the wave's LDS region, rows
// kPitchT bytes apart (8-byte writes of 32 rows at one column land on
// distinct banks), then read back as 8 consecutive columns per lane, 4 rows
// per instruction, and stored as 16-byte non-temporal stores: full 128-byte
// lines, like the fp32 row walk, at half its LDS traffic.  Each lane issues
// 8 stores per block row (the masked ones included).
constexpr int kPitchT = 264;
constexpr int kEpiBf16tBytes = 32 * kPitchT;
static_assert(kEpiBf16tBytes <= kEpiHalfBytes, "fits the fp32 half-piece region");

template <class C, int kI>
__device__ __forceinline__ void wgrad_epilogue_bf16t(const f32x16 (&acc)[C::MB][C::NB], char* lds,
                                                     void* out, int hidden, int inter, int row0,
                                                     int col0) {
    static_assert(C::NB == 4 && kI < C::MB, "a block row of the wave tile is 128 columns");
    const int l = threadIdx.x & 63;
    const int r = l & 31, h = l >> 5;
#pragma unroll
    for (int j = 0; j < C::NB; j++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const f32x16& a = acc[kI][j];
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w = {pack_bf16x2(a[4 * g], a[4 * g + 1]),
                             pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
            *reinterpret_cast<u32x2*>(lds + r * kPitchT + (32 * j + 8 * g + 4 * h) * 2) = w;
        }
    // offsets (rr inter + col) elements from the piece's first row: rr < 32,
    // col < inter <= 2^21, so they fit 32 bits in bytes
    const int prow0 = row0 + 32 * kI;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)out + ((int64_t)prow0 * inter << 1));
    const int c = 8 * (l & 15);
    typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int t = 0; t < 8; t++) {
        const int rr = 4 * t + (l >> 4);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const char* src = lds + rr * kPitchT + c * 2;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
        const bool ok = (prow0 + rr < hidden) & (col0 + c < inter);
        const uint32_t off = ok ? (uint32_t)(((int64_t)rr * inter + col0 + c) << 1) : kInvalid;
        __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y},
                                               ro, off, 0, 2);
    }
}

// Runtime dtype / mode (workgroup-uniform) to the compile-time epilogue;
// kQR: rows of the pieces staged through the wave's LDS region (64:
// kEpiWaveBytes per wave, 32: kEpiHalfBytes); items [kFrom, kTo) of the row
// walk (kTo < 0: to the end).
template <class C, int kQR = 64, int kFrom = 0, int kTo = -1>
__device__ __forceinline__ void wgrad_epilogue(const f32x16 (&acc)[C::MB][C::NB], float* lds,
                                               void* out, int dtype, int hidden, int inter,
                                               int row0, int col0, int accumulate) {
    if (dtype == kBF16) {
        if (accumulate)
            wgrad_epilogue_t<C, kQR, kBF16, true, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
        else
            wgrad_epilogue_t<C, kQR, kBF16, false, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
    } else if (dtype == kF16) {
        if (accumulate)
            wgrad_epilogue_t<C, kQR, kF16, true, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
        else
            wgrad_epilogue_t<C, kQR, kF16, false, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
    } else {
        if (accumulate)
            wgrad_epilogue_t<C, kQR, kF32, true, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
        else
            wgrad_epilogue_t<C, kQR, kF32, false, kFrom, kTo>(acc, lds, out, hidden, inter, row0, col0);
    }
}

}  // namespace gg
