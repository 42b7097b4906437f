// gg_tile.hpp -- device building blocks shared by the gfx950 grouped-GEMM
// kernels: MFMA fragment types, the LDS stage layouts, global->LDS stage
// loaders, fragment readers, the pipelined MFMA main loop, and the work-item
// remap that keeps neighbouring tiles on one XCD.
//
// Geometry (Cfg below): a TM x TN macro tile per workgroup, WM x WN wave64s,
// each wave owning (TM/WM) x (TN/WN) as 32x32 MFMA blocks.  One K step
// stages 128 bytes of K (64 bf16 or 128 fp8 values) of every tile row;
// two stages alternate in LDS.
//
// Global -> LDS: buffer loads that write LDS directly (no register staging).
// One wave instruction moves 1 KiB: lane l's 16 bytes land at base + 16 l.
// Each lane therefore computes which global 16 bytes belong at its LDS slot.
// An offset past the descriptor's range loads zeros, which masks rows past
// the tile edge and K past a group's end.
//
// LDS stage layouts:
//  * K-contiguous operand ("K layout"): tile row r holds 128 bytes of K as 8
//    chunks of 16 bytes; chunk c sits at chunk position c ^ swz(r),
//    swz(r) = (r ^ (r >> 3)) & 7.  MFMA fragments are 16-byte reads.
//  * M/N-contiguous bf16 operand ("MN layout", 256 columns): K row k holds
//    the tile's 256 columns as 32 units of 16 bytes; unit u sits at position
//    u ^ (4 (k & 3)).  Fragments are read with ds_read_b64_tr_b16: within a
//    16-lane group, lane 4q + j receives element j of the 8-byte pieces
//    addressed by lanes q, 4+q, 8+q, 12+q; when lane 4e + q addresses K row
//    kb + e at columns c + 4q, lane i gets column c + i at K rows kb..kb+3 --
//    the K-contiguous register fragment the MFMA needs.
// Both layouts read without bank conflicts (64 banks of 4 bytes).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define GG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kRowBytes = 128;   // bytes of one K-layout tile row per K step

// Epilogue staging: each wave owns a private LDS region holding a 64 x 64
// fp32 slice of its accumulators, rows kEpiPitch floats apart (68: the
// 16-byte row reads of 8 lanes of one row and 8 of the next fall on
// disjoint banks).
constexpr int kEpiPitch = 68;
constexpr int kEpiWaveBytes = 64 * kEpiPitch * 4;

template <int TM_, int TN_, int WM_, int WN_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
    static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
    static constexpr int MB = TM / WM / 32, NB = TN / WN / 32;   // MFMA blocks per wave
    static constexpr int kStage = (TM + TN) * kRowBytes;         // bytes per LDS stage
    static constexpr int kLds = 2 * kStage > kWaves * kEpiWaveBytes ? 2 * kStage
                                                                     : kWaves * kEpiWaveBytes;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Marks a workgroup-uniform value as such (scalar register), so buffer
// descriptors built from it stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ u32x4 ld_lds16(const char* lds, int off) {
    return *reinterpret_cast<const u32x4*>(lds + off);
}

// ---------------------------------------------------------------------------
// Buffer descriptors: a scalar base advanced per K step; 32-bit offsets per
// lane.  kInvalid lies past num_records: such loads return (or write) zeros.
// ---------------------------------------------------------------------------
constexpr uint32_t kInvalid = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7ffffff0,
                                             0x00020000);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// LDS byte address of a pointer into workgroup memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// The LDS-writing buffer load is issued through inline assembly: the
// compiler neither sees nor waits for it, so reads of the other stage are
// not held back.  Completion is awaited explicitly (wait_vm0) before the
// barrier that hands the stage to the MFMA waves.  M0 holds the wave's LDS
// base; lane l writes base + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(uniform((int)lds_addr(lds))), "v"(off), "s"(r)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(0): every outstanding vector memory operation of this
// wave, including the LDS-writing loads, has completed.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// ---------------------------------------------------------------------------
// Stage loaders.
// K layout, R rows: `tile` is the global address of the tile's row 0 at K
// byte 0, rows `ld` bytes apart; this K step covers bytes [kbyte, kbyte+128).
// Rows at or past rows_valid and K bytes at or past kbytes_valid load zeros.
// ---------------------------------------------------------------------------
template <class C, int R>
__device__ __forceinline__ void stage_k(char* lds, const char* tile, int64_t ld, int rows_valid,
                                        int64_t kbyte, int64_t kbytes_valid) {
    constexpr int kBlocks = R / 8;                       // 1 KiB blocks of 8 rows
    static_assert(kBlocks % C::kWaves == 0, "blocks must split evenly over waves");
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile + kbyte);
#pragma unroll
    for (int i = 0; i < kBlocks / C::kWaves; i++) {
        const int b = w * (kBlocks / C::kWaves) + i;
        const int row = 8 * b + (l >> 3);
        const int c = (l & 7) ^ swz(row);
        const bool ok = (row < rows_valid) & (kbyte + c * 16 < kbytes_valid);
        dma16(rs, lds + b * 1024, ok ? (uint32_t)(row * ld) + c * 16 : kInvalid);
    }
}

// MN layout (bf16, 256 columns, 64 K rows): `tile` is the global address of
// this K step's first K row at the tile's first column; K rows are `ld` bytes
// apart.  K rows at or past k_rows_valid and columns at or past cols_valid
// load zeros.
template <class C>
__device__ __forceinline__ void stage_mn(char* lds, const char* tile, int64_t ld, int cols_valid,
                                         int64_t k_rows_valid) {
    constexpr int kBlocks = 32;                          // 1 KiB = 2 K rows of 512 B
    static_assert(kBlocks % C::kWaves == 0, "blocks must split evenly over waves");
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile);
#pragma unroll
    for (int i = 0; i < kBlocks / C::kWaves; i++) {
        const int b = w * (kBlocks / C::kWaves) + i;
        const int k = 2 * b + (l >> 5);
        const int u = (l & 31) ^ (4 * (k & 3));
        const bool ok = (k < k_rows_valid) & (u * 8 < cols_valid);
        dma16(rs, lds + b * 1024, ok ? (uint32_t)(k * ld) + u * 16 : kInvalid);
    }
}

// ---------------------------------------------------------------------------
// Fragment readers (bf16, v_mfma_f32_32x32x16_bf16: lane l supplies row / col
// l % 32 with K values 8 (l / 32) .. 8 (l / 32) + 7 of the 16-value sub-step).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag_k(const char* lds, int row0, int ks) {
    const int l = threadIdx.x & 63;
    return __builtin_bit_cast(bf16x8, ld_lds16(lds, lds_off(row0 + (l & 31), 2 * ks + (l >> 5))));
}

__device__ __forceinline__ int mn_addr(int k, int col) {
    const int u = col >> 3;
    return k * 512 + ((u ^ (4 * (k & 3))) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ bf16x8 frag_mn(const char* lds, int col0, int ks) {
    const int l = threadIdx.x & 63;
    const int g = l >> 4, s = l & 15;
    const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
    const int k = 16 * ks + 8 * (g >> 1) + (s >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)GG_LDS(lds + mn_addr(k, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)GG_LDS(lds + mn_addr(k + 4, col)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <bool KMAJOR>
__device__ __forceinline__ bf16x8 frag_bf16(const char* lds, int base, int ks) {
    if constexpr (KMAJOR)
        return frag_k(lds, base, ks);
    else
        return frag_mn(lds, base, ks);
}

// One staged K step of bf16 MFMAs (4 sub-steps of 16); fragments of sub-step
// ks+1 are read while the MFMAs of ks run.
template <class C, bool A_K, bool B_K>
__device__ __forceinline__ void mfma_stage_bf16(const char* sa, const char* sb, int a0, int b0,
                                                f32x16 (&acc)[C::MB][C::NB]) {
    bf16x8 af[2][C::MB], bfr[2][C::NB];
    auto read = [&](int ks, int buf) {
#pragma unroll
        for (int i = 0; i < C::MB; i++)
            af[buf][i] = frag_bf16<A_K>(sa, a0 + 32 * i, ks);
#pragma unroll
        for (int j = 0; j < C::NB; j++)
            bfr[buf][j] = frag_bf16<B_K>(sb, b0 + 32 * j, ks);
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const int cur = ks & 1;
        if (ks + 1 < 4)
            read(ks + 1, cur ^ 1);
#pragma unroll
        for (int i = 0; i < C::MB; i++)
#pragma unroll
            for (int j = 0; j < C::NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j],
                                                                    0, 0, 0);
    }
}

// One staged K step of MX-scaled fp8 MFMAs (2 sub-steps of 64).
// v_mfma_scale_f32_32x32x64_f8f6f4: lane l (row l%32, h = l/32) supplies K
// bytes [16h, 16h+16) and [32+16h, 32+16h+16) of the sub-step, and the E8M0
// scale of K block h of its row in byte 0 of its scale operand (op_sel 0).
// sa_w[ks][i] / sb_w[ks][j] hold, per sub-step and fragment, the scale word
// already shifted so that byte 0 is block 2 ks + h.
template <class C>
__device__ __forceinline__ void mfma_stage_mx8(const char* sa, const char* sb, int a0, int b0,
                                               const uint32_t (&sa_w)[2][C::MB],
                                               const uint32_t (&sb_w)[2][C::NB],
                                               f32x16 (&acc)[C::MB][C::NB]) {
    const int l = threadIdx.x & 63;
    const int lr = l & 31, lh = l >> 5;
    i32x8 af[2][C::MB], bfr[2][C::NB];
    auto frag = [&](const char* s, int r, int ks) {
        const u32x4 x0 = ld_lds16(s, lds_off(r, 4 * ks + lh));
        const u32x4 x1 = ld_lds16(s, lds_off(r, 4 * ks + 2 + lh));
        return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    auto read = [&](int ks) {
#pragma unroll
        for (int i = 0; i < C::MB; i++)
            af[ks][i] = frag(sa, a0 + 32 * i + lr, ks);
#pragma unroll
        for (int j = 0; j < C::NB; j++)
            bfr[ks][j] = frag(sb, b0 + 32 * j + lr, ks);
    };
    read(0);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        if (ks == 0)
            read(1);
#pragma unroll
        for (int i = 0; i < C::MB; i++)
#pragma unroll
            for (int j = 0; j < C::NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0, (int)sa_w[ks][i], 0, (int)sb_w[ks][j]);
    }
}

// ---------------------------------------------------------------------------
// Pipelined main loop over nk K steps.  issue(stage, kt) queues the direct
// LDS loads of step kt into `stage`; compute(stage) runs the MFMAs of a
// staged step.  The loads of step kt+1 are in flight while step kt computes;
// one wait + barrier per step hands the stage over.
// ---------------------------------------------------------------------------
// begin(kt) runs at the top of step kt, before the loads of step kt+1 are
// queued (dsReLU uses it to take the scale words prefetched for step kt).
struct NoBegin {
    __device__ void operator()(int) const {}
};

template <class C, class Issue, class Compute, class Begin = NoBegin>
__device__ __forceinline__ void mainloop(char* smem, int nk, Issue issue, Compute compute,
                                         Begin begin = Begin()) {
    if (nk <= 0)
        return;
    issue(smem, 0);
    wait_vm0();
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        char* cur = smem + (kt & 1) * C::kStage;
        char* nxt = smem + ((kt + 1) & 1) * C::kStage;
        begin(kt);
        if (kt + 1 < nk)
            issue(nxt, kt + 1);
        compute(cur, kt);
        wait_vm0();
        __syncthreads();
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

// ---------------------------------------------------------------------------
// Eight consecutive elements of a bf16 / fp16 / fp32 row as fp32 (16 or 32
// bytes; the element index is a multiple of 8).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack8_16(u32x4 w, int dtype, float (&v)[8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if (dtype == kBF16) {
            v[2 * k] = __builtin_bit_cast(float, ws[k] << 16);
            v[2 * k + 1] = __builtin_bit_cast(float, ws[k] & 0xffff0000u);
        } else {
            v[2 * k] = f16_to_f32((uint16_t)(ws[k] & 0xffffu));
            v[2 * k + 1] = f16_to_f32((uint16_t)(ws[k] >> 16));
        }
    }
}

__device__ __forceinline__ void load8(const void* base, int dtype, int64_t i, float (&v)[8]) {
    if (dtype == kF32) {
        // (no __builtin_bit_cast of vector components: clang reads element 0
        // for every component that way)
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 a = *reinterpret_cast<const f32x4*>((const float*)base + i);
        const f32x4 b = *reinterpret_cast<const f32x4*>((const float*)base + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        unpack8_16(*reinterpret_cast<const u32x4*>((const uint16_t*)base + i), dtype, v);
    }
}

__device__ __forceinline__ void store8(void* base, int dtype, int64_t i, const float (&v)[8]) {
    if (dtype == kF32) {
        u32x4 a, b;
        a.x = __builtin_bit_cast(uint32_t, v[0]); a.y = __builtin_bit_cast(uint32_t, v[1]);
        a.z = __builtin_bit_cast(uint32_t, v[2]); a.w = __builtin_bit_cast(uint32_t, v[3]);
        b.x = __builtin_bit_cast(uint32_t, v[4]); b.y = __builtin_bit_cast(uint32_t, v[5]);
        b.z = __builtin_bit_cast(uint32_t, v[6]); b.w = __builtin_bit_cast(uint32_t, v[7]);
        *reinterpret_cast<u32x4*>((float*)base + i) = a;
        *reinterpret_cast<u32x4*>((float*)base + i + 4) = b;
    } else {
        uint32_t ws[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t lo = dtype == kBF16 ? f32_to_bf16(v[2 * k]) : f32_to_f16(v[2 * k]);
            const uint32_t hi = dtype == kBF16 ? f32_to_bf16(v[2 * k + 1]) : f32_to_f16(v[2 * k + 1]);
            ws[k] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>((uint16_t*)base + i) = u32x4{ws[0], ws[1], ws[2], ws[3]};
    }
}

// ---------------------------------------------------------------------------
// Row walk of a wave's accumulators (MB == 2: 64 rows x 32 NB columns).  The
// MFMA layout gives a lane one column and 16 rows of a block; stores want a
// lane to own consecutive columns of one row.  The walk stages 64 columns at
// a time through the wave's private LDS region and calls
//   fn(t, r, c, v)  for the 8 columns [c, c+8) of wave-tile row r, v fp32,
// where lane l visits rows (l >> 3) + 8 t, t = 0..7, at c = 8 (l & 7) + 64 h.
// Only this wave touches `lds`; the caller separates it from the main loop
// with a barrier.
// ---------------------------------------------------------------------------
template <class C, class Fn>
__device__ __forceinline__ void for_each_row8(const f32x16 (&acc)[C::MB][C::NB], float* lds, Fn fn) {
    static_assert(C::MB == 2 && C::NB % 2 == 0, "row walk expects 64-row wave tiles");
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < C::NB / 2; h++) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int jj = 0; jj < 2; jj++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    lds[(32 * i + acc_row(r, l)) * kEpiPitch + 32 * jj + (l & 31)] = acc[i][2 * h + jj][r];
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int row = (l >> 3) + 8 * t, c = 8 * (l & 7);
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            const f32x4 a = *reinterpret_cast<const f32x4*>(lds + row * kEpiPitch + c);
            const f32x4 b = *reinterpret_cast<const f32x4*>(lds + row * kEpiPitch + c + 4);
            float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            fn(t, row, 64 * h + c, v);
        }
    }
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
