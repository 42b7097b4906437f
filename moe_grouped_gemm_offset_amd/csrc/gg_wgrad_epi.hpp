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
