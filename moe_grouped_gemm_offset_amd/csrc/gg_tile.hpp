// gg_tile.hpp -- device building blocks shared by the gfx950 grouped-GEMM
// kernels: MFMA fragment types, the swizzled LDS tile layout, global->LDS
// tile loaders (K-contiguous sources copied, MN-contiguous sources transposed
// in registers), and the work-item remap that keeps neighbouring tiles on one
// XCD.
//
// Geometry used throughout:
//   * a workgroup is 256 threads = 4 wave64s arranged 2 x 2 over the
//     TM x TN macro tile; each wave owns (TM/2) x (TN/2) as 32x32 MFMA blocks;
//   * one K step stages 128 bytes of every tile row in LDS (64 bf16 or
//     128 fp8 values), double-buffered;
//   * an LDS tile row is 8 chunks of 16 bytes; chunk c of row r is stored at
//     chunk position c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7, so that the
//     MFMA fragment reads (8 consecutive rows, one chunk) and the transposed
//     stores (rows 8 apart, one chunk) both hit 8 distinct 16-byte bank groups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // bytes of one LDS tile row per K step

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Marks a workgroup-uniform value as such (scalar register), so buffer
// descriptors built from it stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st_lds16(char* lds, int off, u32x4 v) {
    *reinterpret_cast<u32x4*>(lds + off) = v;
}

__device__ __forceinline__ u32x4 ld_lds16(const char* lds, int off) {
    return *reinterpret_cast<const u32x4*>(lds + off);
}

// ---------------------------------------------------------------------------
// Buffer loads: the descriptor (scalar registers) holds a base that the
// caller advances per K step; each thread supplies a 32-bit byte offset.
// An offset of kInvalid lies past num_records, and the hardware returns
// zeros for it -- that is how masked rows and ragged K tails are zero-filled.
// Valid offsets stay far below 2^31 because every base is tile-relative.
// ---------------------------------------------------------------------------
constexpr uint32_t kInvalid = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7ffffff0,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Loader for a source whose K axis is contiguous.  `tile` points at the
// tile's first row at K byte 0; tile row r is `ld` bytes further per row.
// A K step covers bytes [kbyte, kbyte + 128) of each row.  Thread t moves
// chunk t&7 of rows (t>>3) + 32 i.  Rows at or past `rows_valid` (counted
// from the tile's first row) and chunks at or past `kbytes_valid` read as
// zero.
// ---------------------------------------------------------------------------
template <int R>
struct KLoader {
    static constexpr int N = R / 32;
    u32x4 v[N];

    __device__ __forceinline__ void load(const char* tile, int64_t ld_bytes, int rows_valid,
                                         int64_t kbyte, int64_t kbytes_valid) {
        const int t = threadIdx.x;
        const int c = t & 7;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile + kbyte);
        const bool cvalid = kbyte + c * 16 < kbytes_valid;
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int r = (t >> 3) + 32 * i;
            const uint32_t off = (uint32_t)(r * ld_bytes) + c * 16;
            v[i] = buf_load16(rs, (cvalid & (r < rows_valid)) ? off : kInvalid);
        }
    }

    __device__ __forceinline__ void store(char* lds) const {
        const int t = threadIdx.x;
        const int c = t & 7;
#pragma unroll
        for (int i = 0; i < N; i++)
            st_lds16(lds, lds_off((t >> 3) + 32 * i, c), v[i]);
    }
};

// Pack the low (or high) 16-bit halves of two words: result = {b.h, a.h}.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------------------
// Loader for a 16-bit source whose M (or N) axis is contiguous: global row
// k holds the tile's R rows side by side.  Thread t owns an 8 (k) x 8 (m)
// block: it reads 8 global rows of 16 bytes, transposes the 8x8 block of
// 16-bit values in registers, and writes 8 K-contiguous chunks to LDS.
// `tile` points at global row 0 of this K step's first k and at the tile's
// first column.  K rows at or past `k_rows_valid` (counted from that k) and
// columns at or past `cols_valid` (counted from the tile's first column)
// read as zero.
// ---------------------------------------------------------------------------
template <int R>
struct MNLoader16 {
    static constexpr int kBlocksM = R / 8;                  // 8-wide m blocks
    static constexpr int kBlocks = kBlocksM * 8;            // x 8 k blocks of 8
    static constexpr int N = (kBlocks + kThreads - 1) / kThreads;
    u32x4 v[N][8];

    __device__ __forceinline__ void load(const char* tile, int64_t ld_bytes, int cols_valid,
                                         int64_t k_rows_valid) {
        const int t = threadIdx.x;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile);
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int blk = t + i * kThreads;
            if (kBlocks % kThreads != 0 && blk >= kBlocks)
                break;
            const int mb = blk % kBlocksM, kb = blk / kBlocksM;
            const bool cvalid = mb * 8 < cols_valid;
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const int k = kb * 8 + r;
                const uint32_t off = (uint32_t)(k * ld_bytes) + mb * 16;
                v[i][r] = buf_load16(rs, (cvalid & (k < k_rows_valid)) ? off : kInvalid);
            }
        }
    }

    __device__ __forceinline__ void store(char* lds) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int blk = t + i * kThreads;
            if (kBlocks % kThreads != 0 && blk >= kBlocks)
                break;
            const int mb = blk % kBlocksM, kb = blk / kBlocksM;
            // word w of v[r] holds m = 2w (low half) and 2w+1 (high half);
            // output chunk for m holds k = 0..7 as words (k0,k1) .. (k6,k7).
#pragma unroll
            for (int w = 0; w < 4; w++) {
                u32x4 lo, hi;
                lo.x = pack_lo(v[i][0][w], v[i][1][w]);
                lo.y = pack_lo(v[i][2][w], v[i][3][w]);
                lo.z = pack_lo(v[i][4][w], v[i][5][w]);
                lo.w = pack_lo(v[i][6][w], v[i][7][w]);
                hi.x = pack_hi(v[i][0][w], v[i][1][w]);
                hi.y = pack_hi(v[i][2][w], v[i][3][w]);
                hi.z = pack_hi(v[i][4][w], v[i][5][w]);
                hi.w = pack_hi(v[i][6][w], v[i][7][w]);
                st_lds16(lds, lds_off(mb * 8 + 2 * w, kb), lo);
                st_lds16(lds, lds_off(mb * 8 + 2 * w + 1, kb), hi);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// bf16 MFMA over one staged K step (64 values = 4 sub-steps of 16).
// Fragment of block i: lane l reads row base + 32 i + (l & 31), chunk
// 2 ks + (l >> 5): the K layout of v_mfma_f32_32x32x16_bf16 (row l%32, eight
// consecutive K values starting at 8 (l/32)).
// ---------------------------------------------------------------------------
template <int MB, int NB>
__device__ __forceinline__ void mfma_step_bf16(const char* sa, const char* sb, int arow0,
                                               int brow0, f32x16 (&acc)[MB][NB]) {
    const int l = threadIdx.x & 63;
    const int lr = l & 31, lh = l >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        bf16x8 af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; i++) {
            u32x4 x = ld_lds16(sa, lds_off(arow0 + 32 * i + lr, 2 * ks + lh));
            af[i] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int j = 0; j < NB; j++) {
            u32x4 x = ld_lds16(sb, lds_off(brow0 + 32 * j + lr, 2 * ks + lh));
            bfr[j] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int i = 0; i < MB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// MX-scaled fp8 MFMA over one staged K step (128 values = 2 sub-steps of 64).
// v_mfma_scale_f32_32x32x64_f8f6f4: lane l (row l%32, h = l/32) supplies K
// bytes [16h, 16h+16) and [32+16h, 32+16h+16) of the 64-value sub-step, and
// the E8M0 scale of K block h of its row (scale byte selected by op_sel).
// sA_w[ks][i] / sB_w[ks][j]: per sub-step and fragment, the 32-bit word of
// this K step's four scale bytes shifted right so that byte 0 is the scale of
// K block 2 ks + h (op_sel 0 then picks it).
// ---------------------------------------------------------------------------
template <int MB, int NB>
__device__ __forceinline__ void mfma_step_mx8(const char* sa, const char* sb, int arow0, int brow0,
                                              const uint32_t (&sA_w)[2][MB], const uint32_t (&sB_w)[2][NB],
                                              f32x16 (&acc)[MB][NB]) {
    const int l = threadIdx.x & 63;
    const int lr = l & 31, lh = l >> 5;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        i32x8 af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; i++) {
            const int r = arow0 + 32 * i + lr;
            u32x4 x0 = ld_lds16(sa, lds_off(r, 4 * ks + lh));
            u32x4 x1 = ld_lds16(sa, lds_off(r, 4 * ks + 2 + lh));
            af[i] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int r = brow0 + 32 * j + lr;
            u32x4 x0 = ld_lds16(sb, lds_off(r, 4 * ks + lh));
            u32x4 x1 = ld_lds16(sb, lds_off(r, 4 * ks + 2 + lh));
            bfr[j] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                           (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int i = 0; i < MB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[i], bfr[j], acc[i][j], 0, 0, 0, (int)sA_w[ks][i], 0, (int)sB_w[ks][j]);
    }
}

// ---------------------------------------------------------------------------
// Work-item remap: workgroups are dispatched to the 8 XCDs round-robin
// (XCD = blockIdx % 8).  Within a chunk of P consecutive items (P % 8 == 0)
// the remap gives XCD x the contiguous items [x P/8, (x+1) P/8), so tiles that
// share operand rows meet in the same L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int q, int P) {
    if (P % 8 != 0)
        return q;
    return (q & 7) * (P >> 3) + (q >> 3);
}

// Element (block i, block j, register r) of an MFMA 32x32 accumulator is row
// 8 (r/4) + 4 (l/32) + r%4 and column l%32 of that block.
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// fp32 -> bf16 / fp16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// dtype codes (the gg_dtype values of the ABI)
constexpr int kBF16 = 0, kF16 = 1, kF32 = 2;

__device__ __forceinline__ float load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == kBF16)
        return bf16_to_f32(((const uint16_t*)base)[i]);
    if (dtype == kF16)
        return f16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

__device__ __forceinline__ void store_elem(void* base, int dtype, int64_t i, float v) {
    if (dtype == kBF16)
        ((uint16_t*)base)[i] = f32_to_bf16(v);
    else if (dtype == kF16)
        ((uint16_t*)base)[i] = f32_to_f16(v);
    else
        ((float*)base)[i] = v;
}

// Group of an M tile: the g with po[g-1] <= m < po[g] (po[-1] = 0), by binary
// search over the cumulative ends; L if m >= po[L-1].
__device__ __forceinline__ int group_of(const int32_t* po, int L, int64_t m) {
    int lo = 0, hi = L;           // first g with po[g] > m
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)po[mid] > m)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

}  // namespace gg
