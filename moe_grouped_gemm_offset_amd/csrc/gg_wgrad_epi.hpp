// gg_wgrad_epi.hpp -- the output epilogue of the grouped wgrad kernels
// (bf16 and block-scaled main loops alike): Wgrad[e] is written, or added to
// the existing output when accumulating ("Grouped GEMM + WGrad (Unified)",
// "Operation"), rounded to nearest even in the output dtype.
#pragma once
#include "gg_internal.hpp"
#include "gg_tile.hpp"

namespace gg {

// Output: rows of 8 consecutive columns per lane (16-byte bf16/fp16 or
// 32-byte fp32 accesses), accumulate mode adding the old values, which are
// loaded 8 items ahead.  Items off the tile have masked loads and stores.
template <class C>
__device__ __forceinline__ void wgrad_epilogue(const f32x16 (&acc)[C::MB][C::NB], float* lds,
                                               void* out, int dtype, int hidden, int inter,
                                               int row0, int col0, int accumulate) {
    const Fmt8 fo(dtype);
    // offsets (r inter + col) bytes from the wave tile's first row: r < 128,
    // inter <= 2^21
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)out + (int64_t)row0 * inter * (fo.w32 ? 4 : 2));
    auto load = [&](int, int r, int c) {
        const int row = row0 + r, col = col0 + c;
        const bool ok = (row < hidden) & (col < inter) & (accumulate != 0);
        PreB8<1> pre;
        pre.x[0] = rawb8_load(ro, fo, fo.off(ok, (int64_t)r * inter + col));
        return pre;
    };
    auto fn = [&](int, int r, int c, float (&v)[8], const PreB8<1>& pre) {
        const int row = row0 + r, col = col0 + c;
        const bool ok = (row < hidden) & (col < inter);
        float o[8];
        rawb8_cvt(pre.x[0], fo, o);          // zeros unless accumulating
#pragma unroll
        for (int k = 0; k < 8; k++)
            v[k] += o[k];
        rawb8_store(ro, fo, fo.off(ok, (int64_t)r * inter + col), v);
    };
    for_each_row8<C, 8>(acc, lds, load, fn);
}

}  // namespace gg
