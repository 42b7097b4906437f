// gg_tile.hpp -- device building blocks shared by the gfx950 grouped-GEMM
// kernels: MFMA fragment types, the LDS layouts, global->LDS loaders,
// fragment readers, the pipelined MFMA main loop, and the work-item remap
// that keeps neighbouring tiles on one XCD.
//
// Geometry (Cfg below): a TM x TN macro tile per workgroup of WM x WN wave64s,
// each wave owning (TM/WM) x (TN/WN) as 32x32 MFMA blocks held in
// accumulation registers.  The bf16 kernels run 4 x 2 waves (two per SIMD,
// 64 x 128 each: a stalled wave leaves the MFMA pipe to the other); the fp8
// kernel, whose fragments are twice as large, runs 2 x 2 (one per SIMD,
// 128 x 128 each, 512 registers).
//
// K is walked in stages of 64 bytes of every tile row (32 bf16 or 64 fp8
// values); a wave reads the next stage's MFMA fragments from LDS into one
// register set while its MFMAs consume the other.  Loads into LDS move two
// stages at a time (a "load unit", 128 bytes of every row): the load path
// of a CU moves about one 128-byte cache line per three clocks whether the
// line is wanted whole or in halves, so a unit fetches each line once.  Two
// unit buffers alternate: unit u+1 is in flight while unit u is read.
//
// Global -> LDS: buffer loads that write LDS directly (no register staging).
// One wave instruction moves 1 KiB: lane l's 16 bytes land at base + 16 l.
// Each lane therefore computes which global 16 bytes belong at its LDS slot.
// An offset past the descriptor's record count loads zeros, which masks rows
// past the tile edge and K past a group's end.
//
// LDS layouts of a unit:
//  * K-contiguous operand ("K layout"): tile row r holds 128 bytes of K as 8
//    chunks of 16 bytes; chunk c sits at chunk position c ^ swz(r),
//    swz(r) = (r ^ (r >> 3)) & 7.  Stage h (0, 1) of the unit is chunks
//    4h .. 4h+3.  MFMA fragments are 16-byte reads.
//  * M/N-contiguous bf16 operand ("MN layout", 256 columns): K row k (0..63)
//    holds the tile's 256 columns as 32 units of 16 bytes; unit u sits at
//    position u ^ (4 (k & 3)).  Stage h is K rows 32h .. 32h+31.  Fragments
//    are read with ds_read_b64_tr_b16: within a 16-lane group, lane 4q + j
//    receives element j of the 8-byte pieces addressed by lanes q, 4+q, 8+q,
//    12+q; when lane 4e + q addresses K row kb + e at columns c + 4q, lane i
//    gets column c + i at K rows kb..kb+3 -- the K-contiguous register
//    fragment the MFMA needs.
//  * N-contiguous 8-bit operand ("MN8 layout", 256 columns, 128 K rows):
//    K row k holds the 256 columns as 16 chunks of 16 bytes; chunk u sits at
//    position u ^ (2 (k & 7)).  Stage h is K rows 64h .. 64h+63.  Fragments
//    are read with ds_read_b64_tr_b8: within a 16-lane group, lane 8q + j
//    receives, as byte m, byte j of the 8-byte piece addressed by lane
//    2m + q; when lane 2e + q addresses K row kb + e at columns c + 8q, lane
//    i gets column c + i at K rows kb..kb+7.
// All layouts read without bank conflicts (64 banks of 4 bytes; a 16-byte
// read is served 16 lanes at a time, an 8-byte one 32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define GG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kRowBytes = 128;   // bytes of one K-layout tile row per load unit

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
    static constexpr int kUnit = (TM + TN) * kRowBytes;          // bytes per load unit
    static constexpr int kLds = 2 * kUnit > kWaves * kEpiWaveBytes ? 2 * kUnit
                                                                    : kWaves * kEpiWaveBytes;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Marks a workgroup-uniform value as such (scalar register), so buffer
// descriptors built from it stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The same for a pointer (e.g. one loaded from a pointer array): buffer
// descriptors built from a pointer the compiler takes for divergent would be
// wrapped in a loop over the lanes' distinct values.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Read of a workgroup-uniform address whose contents no kernel of this
// launch writes (tables from the set-up kernel, caller pointer arrays):
// through the constant address space it becomes a scalar load, awaited with
// the LDS counter, so that awaiting it leaves vector memory operations
// (output stores, an atomic) in flight.
template <class T>
__device__ __forceinline__ T scalar_read(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ u32x4 ld_lds16(const char* lds, int off) {
    return *reinterpret_cast<const u32x4*>(lds + off);
}

// ---------------------------------------------------------------------------
// Buffer descriptors: 32-bit offsets per lane from a scalar base; kInvalid
// lies past any record count used here, so such loads return (or write)
// zeros.
// ---------------------------------------------------------------------------
constexpr uint32_t kInvalid = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                        uint32_t records = 0x7ffffff0u) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)records,
                                             0x00020000);
}

// LDS byte address of a pointer into workgroup memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// The LDS-writing buffer load is issued through inline assembly: the
// compiler neither sees nor waits for it, so it cannot hold back reads of
// the other buffer.  Completion is awaited explicitly (vm_wait) before the
// barrier that hands a unit to the MFMA waves.  M0 holds the wave's LDS
// byte address (workgroup-uniform); lane l writes lds + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(uniform((int)lds)), "v"(off), "s"(r)
                 : "memory", "m0");
}

// Dword form: lane l's 4 bytes land at lds + 4 l (one wave moves 256 B).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(uniform((int)lds)), "v"(off), "s"(r)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's vector memory
// operations (which complete in issue order, the LDS-writing loads
// included) are outstanding, and all its LDS operations have completed.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void wait_all() { vm_wait<0>(); }

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have completed; vector
// memory operations may still be in flight.
__device__ __forceinline__ void lds_wait() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

// Workgroup barrier that lets the compiler move neither memory accesses nor,
// through the scheduling barriers, any other instruction across it.  (The
// fence of __syncthreads would add waits of its own.)
__device__ __forceinline__ void unit_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Unit loaders.  Each lane's byte offsets within a unit are fixed for the
// whole K loop and computed once (init); per unit only the scalar buffer
// descriptor moves.  Its record count masks what lies past the data.
//
// K layout, R rows, rows `ld` bytes apart; rows at or past rows_valid load
// zeros.  issue() loads the 128 bytes at `tile` (row 0, the unit's first K
// byte) with kleft valid K bytes left from there (<= 0: all zeros).  With
// RAGGED, kleft may end inside the unit (per-lane check); otherwise a unit
// is either wholly inside K or wholly past it.
// ---------------------------------------------------------------------------
template <class C, int R>
struct LoadK {
    static constexpr int kN = R / 8 / C::kWaves;         // 1 KiB loads (8 rows) per wave
    static_assert(kN * 8 * C::kWaves == R, "rows must split evenly over waves");
    uint32_t off[kN], c16[kN];
    __device__ __forceinline__ void init(int64_t ld, int rows_valid) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < kN; i++) {
            const int row = 8 * (w * kN + i) + (l >> 3);
            const int c = (l & 7) ^ swz(row);
            off[i] = row < rows_valid ? (uint32_t)(row * ld) + c * 16 : kInvalid;
            c16[i] = c * 16;
        }
    }
    // Load i (0 .. kN-1) of this wave.
    template <bool RAGGED>
    __device__ __forceinline__ void issue(uint32_t lds, const char* tile, int64_t kleft, int i) const {
        const int w = uniform(threadIdx.x >> 6);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(uniform_ptr(tile), (uint32_t)uniform(kleft > 0 ? 0x7ffffff0 : 0));
        const uint32_t kl = (uint32_t)(kleft < 128 ? (kleft < 0 ? 0 : kleft) : 128);
        dma16(rs, lds + (w * kN + i) * 1024, !RAGGED || c16[i] < kl ? off[i] : kInvalid);
    }
};

// MN layout (bf16, 256 columns, 64 K rows), K rows `ld` bytes apart;
// columns at or past cols_valid load zeros.  issue() loads the K rows
// starting at `tile` (the unit's first K row at the tile's first column)
// with krows valid K rows left from there.
template <class C>
struct LoadMN {
    static constexpr int kN = 32 / C::kWaves;            // 1 KiB loads (2 K rows) per wave
    static_assert(kN * C::kWaves == 32, "K rows must split evenly over waves");
    uint32_t off[kN];
    uint32_t ld;
    __device__ __forceinline__ void init(int64_t ld_, int cols_valid) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        ld = (uint32_t)ld_;
#pragma unroll
        for (int i = 0; i < kN; i++) {
            const int k = 2 * (w * kN + i) + (l >> 5);
            const int u = (l & 31) ^ (4 * (k & 3));
            off[i] = u * 8 < cols_valid ? (uint32_t)(k * ld_) + u * 16 : kInvalid;
        }
    }
    // A lane at K row k < krows and a valid column has k ld + 16 u < krows ld
    // (16 u < 2 cols_valid <= ld), so the record count krows ld masks exactly
    // the K rows past the end.
    // Load i (0 .. kN-1) of this wave.
    __device__ __forceinline__ void issue(uint32_t lds, const char* tile, int64_t krows, int i) const {
        const int w = uniform(threadIdx.x >> 6);
        const uint32_t kr = (uint32_t)(krows < 64 ? (krows < 0 ? 0 : krows) : 64);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(tile), (uint32_t)uniform((int)(kr * ld)));
        dma16(rs, lds + (w * kN + i) * 1024, off[i]);
    }
};

// MN8 layout (8-bit codes, 256 columns, 128 K rows), K rows `ld` bytes
// apart; columns at or past cols_valid (a multiple of 16) load zeros.
// issue() loads the K rows starting at `tile` (the unit's first K row at the
// tile's first column) with krows valid K rows left from there.
template <class C>
struct LoadMN8 {
    static constexpr int kN = 32 / C::kWaves;            // 1 KiB loads (4 K rows) per wave
    static_assert(kN * C::kWaves == 32 && C::TN == 256, "K rows must split evenly over waves");
    uint32_t off[kN];
    uint32_t ld;
    __device__ __forceinline__ void init(int64_t ld_, int cols_valid) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        ld = (uint32_t)ld_;
#pragma unroll
        for (int i = 0; i < kN; i++) {
            const int k = 4 * (w * kN + i) + (l >> 4);
            const int u = (l & 15) ^ (2 * (k & 7));
            off[i] = u * 16 < cols_valid ? (uint32_t)(k * ld_) + u * 16 : kInvalid;
        }
    }
    // A lane at K row k < krows and a valid column has k ld + 16 u + 16 <=
    // k ld + cols_valid <= krows ld, so the record count krows ld masks
    // exactly the K rows past the end.
    __device__ __forceinline__ void issue(uint32_t lds, const char* tile, int64_t krows, int i) const {
        const int w = uniform(threadIdx.x >> 6);
        const uint32_t kr = (uint32_t)(krows < 128 ? (krows < 0 ? 0 : krows) : 128);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(tile), (uint32_t)uniform((int)(kr * ld)));
        dma16(rs, lds + (w * kN + i) * 1024, off[i]);
    }
};

// ---------------------------------------------------------------------------
// Fragment readers (bf16, v_mfma_f32_32x32x16_bf16: lane l supplies row / col
// l % 32 with K values 8 (l / 32) .. 8 (l / 32) + 7 of a 16-value sub-step;
// stage h of a unit has sub-steps ks = 0, 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag_k(const char* lds, int row0, int chunk) {
    const int l = threadIdx.x & 63;
    return __builtin_bit_cast(bf16x8, ld_lds16(lds, lds_off(row0 + (l & 31), chunk + (l >> 5))));
}

__device__ __forceinline__ int mn_addr(int k, int col) {
    const int u = col >> 3;
    return k * 512 + ((u ^ (4 * (k & 3))) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ bf16x8 frag_mn(const char* lds, int col0, int k0) {
    const int l = threadIdx.x & 63;
    const int g = l >> 4, s = l & 15;
    const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
    const int k = k0 + 8 * (g >> 1) + (s >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)GG_LDS(lds + mn_addr(k, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)GG_LDS(lds + mn_addr(k + 4, col)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Sub-step ks of stage h: K chunk 4h + 2ks (K layout) or K row 32h + 16ks
// (MN layout).
template <bool KMAJOR>
__device__ __forceinline__ bf16x8 frag_bf16(const char* lds, int base, int h, int ks) {
    if constexpr (KMAJOR)
        return frag_k(lds, base, 4 * h + 2 * ks);
    else
        return frag_mn(lds, base, 32 * h + 16 * ks);
}

// One wave's bf16 fragments of a stage (two sub-steps of 16 K values).
template <class C>
struct FragBf16 {
    bf16x8 a[2][C::MB], b[2][C::NB];
};

// Fragment group g of stage h: A rows a0 + 32 g of `sa` (g < MB) or B rows /
// columns b0 + 32 (g - MB) of `sb`, both sub-steps.
template <class C, bool A_K, bool B_K>
__device__ __forceinline__ void read_bf16(const char* sa, const char* sb, int a0, int b0, int h,
                                          FragBf16<C>& f, int g) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        if (g < C::MB)
            f.a[ks][g] = frag_bf16<A_K>(sa, a0 + 32 * g, h, ks);
        else
            f.b[ks][g - C::MB] = frag_bf16<B_K>(sb, b0 + 32 * (g - C::MB), h, ks);
    }
}

// MFMAs m0 .. m1-1 of a stage, m = (ks MB + i) NB + j.  With kT the
// operands are swapped: block (i, j) then holds the transpose, so that a
// lane owns one row of the block (row l % 32) and, in register r, column
// 8 (r / 4) + 4 (l / 32) + r % 4 -- four consecutive columns per group of
// four registers (see acc_row for the plain layout).
template <class C, bool kT = false>
__device__ __forceinline__ void mma_bf16(const FragBf16<C>& f, f32x16 (&acc)[C::MB][C::NB], int m0,
                                         int m1) {
#pragma unroll
    for (int m = 0; m < 2 * C::MB * C::NB; m++) {
        if (m < m0 || m >= m1)
            continue;
        const int ks = m / (C::MB * C::NB), i = (m / C::NB) % C::MB, j = m % C::NB;
        if constexpr (kT)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][j], f.a[ks][i], acc[i][j], 0,
                                                                0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], f.b[ks][j], acc[i][j], 0,
                                                                0, 0);
    }
}

// One wave's MX fp8 fragments of a stage (64 K values) with their scales.
// v_mfma_scale_f32_32x32x64_f8f6f4: lane l (row l%32, q = l/32) supplies K
// bytes [16q, 16q+16) and [32+16q, 32+16q+16), and the E8M0 scale of K block
// q of its row in byte 0 of its scale operand (op_sel 0).
template <class C>
struct FragMx8 {
    i32x8 a[C::MB], b[C::NB];
    uint32_t sa[C::MB], sb[C::NB];
    // the scale words as read; sh brings this stage's byte of a lane's K
    // block to byte 0, at the MFMA (a shift at the read would wait for it)
    uint32_t sh;
};

__device__ __forceinline__ int mn8_addr(int k, int col) {
    return k * 256 + (((col >> 4) ^ (2 * (k & 7))) << 4) + (col & 15);
}

// Columns col0 .. col0+31 of stage K rows k0 .. k0+63 (MN8 layout) as MX
// fragments: lane l (column col0 + l % 32, q = l / 32) gets K rows
// k0 + 16q .. +15 and k0 + 32 + 16q .. +15, eight per transposing read.
__device__ __forceinline__ i32x8 frag_mn8(const char* lds, int col0, int k0) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const int l = threadIdx.x & 63;
    const int grp = l >> 4, s = l & 15;
    const int col = col0 + 16 * (grp & 1) + 8 * (s & 1);
    const int kq = k0 + 16 * (grp >> 1) + (s >> 1);
    i32x2 v[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
        v[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)GG_LDS(
            lds + mn8_addr(kq + 32 * (r >> 1) + 8 * (r & 1), col)));
    return i32x8{v[0].x, v[0].y, v[1].x, v[1].y, v[2].x, v[2].y, v[3].x, v[3].y};
}

// Fragment group g of stage h: A row block g (g < MB) or B row block g - MB
// (K layout; with !B_K the MN8 layout).
template <class C, bool B_K = true>
__device__ __forceinline__ void read_mx8(const char* sa, const char* sb, int a0, int b0, int h,
                                         FragMx8<C>& f, int g) {
    const int l = threadIdx.x & 63;
    const int lr = l & 31, lq = l >> 5;
    auto frag = [&](const char* s, int r) {
        const u32x4 x0 = ld_lds16(s, lds_off(r, 4 * h + lq));
        const u32x4 x1 = ld_lds16(s, lds_off(r, 4 * h + 2 + lq));
        return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    if (g < C::MB)
        f.a[g] = frag(sa, a0 + 32 * g + lr);
    else if constexpr (B_K)
        f.b[g - C::MB] = frag(sb, b0 + 32 * (g - C::MB) + lr);
    else
        f.b[g - C::MB] = frag_mn8(sb, b0 + 32 * (g - C::MB), 64 * h);
}

// MFMAs m0 .. m1-1 of a stage, m = i NB + j.
// AB: the operands' FP8 format, 0 E4M3 ("fp8"), 1 E5M2 ("bf8"): the MFMA's
// cbsz / blgp format fields for A and B.
template <class C, int AB = 0>
__device__ __forceinline__ void mma_mx8(const FragMx8<C>& f, f32x16 (&acc)[C::MB][C::NB], int m0,
                                        int m1) {
#pragma unroll
    for (int m = 0; m < C::MB * C::NB; m++) {
        if (m < m0 || m >= m1)
            continue;
        const int i = m / C::NB, j = m % C::NB;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.a[i], f.b[j], acc[i][j], AB, AB, 0, (int)(f.sa[i] >> f.sh), 0,
            (int)(f.sb[j] >> f.sh));
    }
}

// ---------------------------------------------------------------------------
// Pipelined main loop over nk stages (nk rounded up to whole units; the
// stages past nk load zeros).
//   issue(lds, u, i)     queues load i (0 .. VM-1) of this wave for unit u
//                        (stages 2u, 2u+1) into the unit buffer at LDS
//                        address lds; for units past the end every load must
//                        be masked (it then writes zeros and reads no memory);
//   read(buf, kt, f, g)  queues this wave's LDS reads of fragment group g
//                        (0 .. kGroups-1) of stage kt (unit buffer buf, half
//                        kt & 1) into f;
//   mma(f, m0, m1)       runs MFMAs m0 .. m1-1 (of kMfma) on a fragment set.
// Unit u lives in buffer u & 1.  Iteration u runs stage 2u ("even half")
// while reading stage 2u+1's fragments from the same unit -- two fragment
// groups per MFMA, so that the reads end early; one barrier then certifies
// that every wave has read all of unit u, and the first third of unit u+2's
// loads go into unit u's buffer between the even half's remaining MFMAs.
// The iteration then awaits unit u+1, passes a second barrier, and runs
// stage 2u+1 ("odd half") while issuing the rest of unit u+2 and reading
// stage 2u+2 from unit u+1.  (Issuing all of unit u+2 in the odd half
// stalled its MFMAs behind the load path: the MoE dsReLU ran 8% slower, the
// block-scaled wgrad 8%.)  !kEarlyLoads keeps all of unit u+2 in the odd
// half and the reads one group per MFMA, for callers whose registers the
// earlier loads would spill.
//
// The issue order is fixed instruction by instruction (scheduling barriers
// between the pieces): one MFMA, then the loads and reads due after it.  The
// load path of a CU accepts one 1 KiB load every 16 clocks or so, and a wave
// whose load waits for it cannot issue its next MFMA: loads spread over the
// MFMAs keep the MFMA pipes fed, where a burst of loads would stall them.
// Loads are issued past the end as well, so the loop body has no branch (a
// branch would let the compiler sink one iteration's MFMAs into the next and
// hold three fragment sets).  The trailing wait and barrier let the caller
// reuse the LDS.
// ---------------------------------------------------------------------------
template <class C, int VM, int kMfma, int kGroups, bool kEarlyLoads = true, class F, class Issue,
          class Read, class Mma>
__device__ __forceinline__ void pipeline(char* smem, int nk, F (&f)[2], Issue issue, Read read,
                                         Mma mma) {
    static_assert(kGroups <= kMfma, "one fragment group per MFMA at most");
    if (nk <= 0)
        return;
    const int nu = (nk + 1) >> 1;                        // load units
    const uint32_t lds0 = lds_addr(smem);
    auto buf = [&](int u) { return smem + (u & 1) * C::kUnit; };
    auto lds = [&](int u) { return lds0 + (uint32_t)((u & 1) * C::kUnit); };
#pragma unroll
    for (int i = 0; i < VM; i++)
        issue(lds(0), 0, i);
#pragma unroll
    for (int i = 0; i < VM; i++)
        issue(lds(1), 1, i);
    vm_wait<VM>();                                       // all of unit 0
    unit_barrier();
#pragma unroll
    for (int g = 0; g < kGroups; g++)
        read(buf(0), 0, f[0], g);
    // stage 2u, reading stage 2u+1 from the same unit, two fragment groups
    // per MFMA (the first kH MFMAs); once every wave has read all of unit u
    // (a barrier after MFMA kW-1), the first kEarly loads of unit u+2 go
    // into its buffer between the remaining MFMAs
    constexpr int kEarly = kEarlyLoads ? VM / 3 : 0;
    constexpr int kH = (kGroups + 1) / 2;
    // the barrier a few MFMAs after the last read, so that the wait for the
    // reads rarely stalls (4 more MFMAs measured 1% faster on the dsReLU)
    constexpr int kW = kH + 4 < kMfma ? kH + 4 : kH;
    static_assert(kGroups < kMfma, "MFMAs left after the reads");
    auto even = [&](int u, auto LOADS) {
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f[0], m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kEarly > 0) {
                if (2 * m < kGroups)
                    read(buf(u), 2 * u + 1, f[1], 2 * m);
                if (2 * m + 1 < kGroups)
                    read(buf(u), 2 * u + 1, f[1], 2 * m + 1);
            } else if (m < kGroups) {
                read(buf(u), 2 * u + 1, f[1], m);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (decltype(LOADS)::value && kEarly > 0) {
                if (m == kW - 1) {
                    lds_wait();
                    unit_barrier();
                }
#pragma unroll
                for (int i = 0; i < kEarly; i++)
                    if (m >= kW && i * (kMfma - kW) / kEarly == m - kW)
                        issue(lds(u), u + 2, i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    int u = 0;
    for (; u + 1 < nu; u++) {
        even(u, std::true_type{});
        // stage 2u+1: hand over unit u+1, refill unit u's buffer with u+2
        vm_wait<kEarly>();
        unit_barrier();
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f[1], m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = kEarly; i < VM; i++)
                if ((i - kEarly) * kMfma / (VM - kEarly) == m)
                    issue(lds(u), u + 2, i);
            __builtin_amdgcn_sched_barrier(0);
            if (m < kGroups)
                read(buf(u + 1), 2 * u + 2, f[0], m);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    even(u, std::false_type{});
    mma(f[1], 0, kMfma);
    wait_all();
    unit_barrier();
}

// ---------------------------------------------------------------------------
// Five-slot variant for tiles with TM == TN (bf16: 5 x 32 KiB = 160 KiB of
// LDS).  Each operand half of a unit (its A rows or its B rows) occupies one
// of five slots, so besides units u and u+1 one slot is always spare.  Unit
// u+2's A half is loaded into the spare slot during the even half of
// iteration u -- no barrier is needed, the slot's last reader passed the
// barrier of iteration u-1 -- and its B half into unit u's A slot during
// the odd half, after the barrier; unit u's B slot becomes the next spare.
// The load path thus works through both halves of every iteration instead
// of the odd half alone, and the A half gets one and a half iterations to
// land.  The wait before each barrier leaves the A half just issued in
// flight.
//   issue(lds_a, lds_b, u, i)  queues load i of unit u: i < VMA are A loads
//                              (into lds_a), VMA <= i < VM B loads (lds_b);
//   read(buf_a, buf_b, kt, f, g), mma(f, m0, m1) as for pipeline.
// ---------------------------------------------------------------------------
template <class C>
struct Slots5 {
    static constexpr int kSlot = C::TM * kRowBytes;
    static constexpr int kLds = 5 * kSlot > C::kWaves * kEpiWaveBytes ? 5 * kSlot
                                                                     : C::kWaves * kEpiWaveBytes;
    static_assert(C::TM == C::TN, "five equal slots");
};

template <class C, int VMA, int VM, int kMfma, int kGroups, class F, class Issue, class Read,
          class Mma>
__device__ __forceinline__ void pipeline5(char* smem, int nk, F (&f)[2], Issue issue, Read read,
                                          Mma mma) {
    static_assert(kGroups <= kMfma && VMA <= VM, "one fragment group per MFMA at most");
    constexpr int kSlot = Slots5<C>::kSlot;
    if (nk <= 0)
        return;
    const int nu = (nk + 1) >> 1;                        // load units
    const uint32_t lds0 = lds_addr(smem);
    auto sl = [&](int k) { return lds0 + (uint32_t)(k * kSlot); };
    auto sb = [&](int k) { return smem + k * kSlot; };
    // slots of unit u (a, b) and u+1 (a1, b1), and the spare one
    int a = 0, b = 1, a1 = 2, b1 = 3, sp = 4;
#pragma unroll
    for (int i = 0; i < VM; i++)
        issue(sl(0), sl(1), 0, i);
#pragma unroll
    for (int i = 0; i < VM; i++)
        issue(sl(2), sl(3), 1, i);
    vm_wait<VM>();                                       // all of unit 0
    unit_barrier();
#pragma unroll
    for (int g = 0; g < kGroups; g++)
        read(sb(0), sb(1), 0, f[0], g);
    int u = 0;
    for (; u + 1 < nu; u++) {
        // stage 2u, reading stage 2u+1 of unit u; unit u+2's A half into
        // the spare slot
        const uint32_t la = sl(sp);
        const char* ra = sb(a);
        const char* rb = sb(b);
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f[0], m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < VMA; i++)
                if (i * kMfma / VMA == m)
                    issue(la, 0u, u + 2, i);
            __builtin_amdgcn_sched_barrier(0);
            if (m < kGroups)
                read(ra, rb, 2 * u + 1, f[1], m);
            __builtin_amdgcn_sched_barrier(0);
        }
        // unit u+1 has landed once only the A half just issued is in flight
        vm_wait<VMA>();
        unit_barrier();
        // stage 2u+1, reading stage 2u+2 of unit u+1; unit u+2's B half
        // into unit u's A slot
        const uint32_t lb = sl(a);
        const char* qa = sb(a1);
        const char* qb = sb(b1);
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f[1], m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = VMA; i < VM; i++)
                if ((i - VMA) * kMfma / (VM - VMA) == m)
                    issue(0u, lb, u + 2, i);
            __builtin_amdgcn_sched_barrier(0);
            if (m < kGroups)
                read(qa, qb, 2 * u + 2, f[0], m);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int na = sp, nb = a, ns = b;
        a = a1;
        b = b1;
        a1 = na;
        b1 = nb;
        sp = ns;
    }
    {
        const char* ra = sb(a);
        const char* rb = sb(b);
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f[0], m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (m < kGroups)
                read(ra, rb, 2 * u + 1, f[1], m);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mma(f[1], 0, kMfma);
    wait_all();
    unit_barrier();
}

// ---------------------------------------------------------------------------
// Ping-pong variant of the five-slot loop, for 8 waves (TM == TN).  Waves
// 0-3 and 4-7 form two groups with one wave of each on every SIMD.  Each
// wave alternates a memory phase (its fragment reads of one stage, then
// half of its share of one half-unit's loads) and a compute phase (that
// stage's MFMAs at raised issue priority, with the other half of those loads
// issued between them), and the second group runs one phase behind the
// first: in every phase one wave per SIMD feeds the MFMA pipe while the
// other reads its next fragments from LDS.  One barrier separates
// consecutive phases; one fragment set per wave suffices, since a wave never
// reads while it computes.  (With all loads in the memory phases those were
// the longer phases: fragment reads plus load issue took ~600 clocks
// against the 512 of a compute phase; with all of them in the compute
// phases, the MFMAs waited on load issue instead.)
//
// Slots (32 KiB each) at the start of window u (stages 2u, 2u+1): A(u) and
// B(u) are read, A(u+1) has landed or is landing, and two are free (unit
// u-1's, whose last reads ended before the window's first barrier).  The
// first group issues its share of B(u+1) into the first free slot in its
// first memory and compute phases of window u, and of A(u+2) into the
// second in its second ones.  The second group, one phase behind, would
// have only its second memory phase left before B(u+1) must have landed; it
// therefore issues its share of B(u+1) one phase earlier, in its last
// memory and compute phases of window u-1 (into unit u-1's A slot once its
// own reads of it have completed, and after the barrier that freed it), and
// its share of A(u+2) in its first ones of window u.  B(u+1) must land
// before window u+1: the first group waits for it at the end of its second
// compute phase, the second at the end of its second memory phase -- both
// with only the loads issued after it left in flight.  Each group runs its
// own copy of the loop, so that no group-dependent branch inside it lets the
// compiler merge the two groups' compute phases (which spilled the
// accumulators).
//   issue, read, mma as for pipeline5; f is a single fragment set.
// With kPre, the caller has already issued unit 0 into slots 0 and 1, and
// either at least kPending other vector memory operations after it (e.g. a
// previous tile's output stores) or unit 0 has landed: since they complete
// in issue order, the first wait leaves kPending of them in flight, to be
// awaited with B(1), one window later.
// ---------------------------------------------------------------------------
template <class C, int VMA, int VM, int kMfma, int kGroups, bool kPre = false, int kPending = 0,
          class F, class Issue, class Read, class Mma>
__device__ __forceinline__ void pipeline_pp(char* smem, int nk, F& f, Issue issue, Read read,
                                            Mma mma) {
    static_assert(kPending == 0 || kPre, "operations after unit 0 only when it is prefetched");
    static_assert(C::kWaves == 8 && VMA <= VM, "two groups of four waves");
    static_assert(VM + kPending < 64, "vmcnt is 6 bits");
    constexpr int kSlot = Slots5<C>::kSlot;
    if (nk <= 0) {
        if constexpr (kPre)
            wait_all();                                  // the prefetched unit has landed
        return;
    }
    const int nu = (nk + 1) >> 1;                        // load units
    const bool second = uniform(threadIdx.x >> 6) >= 4;
    const uint32_t lds0 = lds_addr(smem);
    auto sl = [&](int k) { return lds0 + (uint32_t)(k * kSlot); };
    auto sb = [&](int k) { return smem + k * kSlot; };
    int a = 0, b = 1, a1 = 2, f1 = 3, f2 = 4;
    if constexpr (!kPre) {
#pragma unroll
        for (int i = 0; i < VM; i++)
            issue(sl(0), sl(1), 0, i);
    }
#pragma unroll
    for (int i = 0; i < VMA; i++)
        issue(sl(2), 0u, 1, i);
    if (second) {
        // the second group's share of B(1), ahead of its first window
#pragma unroll
        for (int i = VMA; i < VM; i++)
            issue(0u, sl(3), 1, i);
        vm_wait<VM + kPending>();                        // A(0), B(0)
    } else {
        vm_wait<VMA + kPending>();                       // A(0), B(0)
    }
    unit_barrier();
    if (second)
        unit_barrier();                                  // one phase behind
    // of each half-unit's loads, the first kMem* go out at the end of a
    // memory phase, the rest between the next compute phase's MFMAs
    constexpr int kMemA = VMA / 2, kMemB = (VM - VMA) / 2;
    auto mem_a = [&](uint32_t la, int uu) {
#pragma unroll
        for (int i = 0; i < kMemA; i++)
            issue(la, 0u, uu, i);
    };
    auto mem_b = [&](uint32_t lb, int uu) {
#pragma unroll
        for (int i = VMA; i < VMA + kMemB; i++)
            issue(0u, lb, uu, i);
    };
    // compute phase: the stage's MFMAs with the rest spread between them
    auto compute_a = [&](uint32_t la, int uu) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f, m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = kMemA; i < VMA; i++)
                if ((i - kMemA) * kMfma / (VMA - kMemA) == m)
                    issue(la, 0u, uu, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute_b = [&](uint32_t lb, int uu) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int m = 0; m < kMfma; m++) {
            mma(f, m, m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = VMA + kMemB; i < VM; i++)
                if ((i - VMA - kMemB) * kMfma / (VM - VMA - kMemB) == m)
                    issue(0u, lb, uu, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto G2) {
        constexpr bool kG2 = decltype(G2)::value;
        for (int u = 0; u < nu; u++) {
            const char* ra = sb(a);
            const char* rb = sb(b);
#pragma unroll
            for (int g = 0; g < kGroups; g++)
                read(ra, rb, 2 * u, f, g);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kG2)
                mem_a(sl(f2), u + 2);
            else
                mem_b(sl(f1), u + 1);
            lds_wait();
            unit_barrier();
            if constexpr (kG2)
                compute_a(sl(f2), u + 2);
            else
                compute_b(sl(f1), u + 1);
            unit_barrier();
#pragma unroll
            for (int g = 0; g < kGroups; g++)
                read(ra, rb, 2 * u + 1, f, g);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kG2) {
                lds_wait();                              // own reads of slot a done
                mem_b(sl(a), u + 2);
                vm_wait<VMA + kMemB>();                  // B(u+1) has landed
            } else {
                mem_a(sl(f2), u + 2);
                lds_wait();
            }
            unit_barrier();
            if constexpr (kG2) {
                compute_b(sl(a), u + 2);
            } else {
                compute_a(sl(f2), u + 2);
                vm_wait<VMA>();                          // B(u+1) has landed
            }
            unit_barrier();
            const int na = a1, nb = f1, na1 = f2;
            f1 = a;
            f2 = b;
            a = na;
            b = nb;
            a1 = na1;
        }
    };
    if (second)
        run(std::true_type{});
    else
        run(std::false_type{});
    if (!second)
        unit_barrier();                                  // the second group's last phase
    wait_all();
    unit_barrier();
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

// Two-dimensional variant for a tiles_m x tiles_n chunk: the chunk is cut into
// a gm x (8/gm) grid of equal blocks of tiles, and XCD x takes block
// (x / (8/gm), x % (8/gm)), so that an M-tile row's A panel is read by 8/gm
// XCDs and an N-tile column's B panel by gm, instead of 1 and 8.  gm divides
// 8 and tiles_m, 8/gm divides tiles_n (the caller checks); gm = 0 falls back
// to xcd_remap.
__device__ __forceinline__ void xcd_remap2d(int q, int tiles_m, int tiles_n, int gm, int& mt,
                                            int& nt) {
    if (gm == 0) {
        const int r = xcd_remap(q, tiles_m * tiles_n);
        mt = r / tiles_n;
        nt = r % tiles_n;
        return;
    }
    const int gn = 8 / gm, bm = tiles_m / gm, bn = tiles_n / gn;
    const int x = q & 7, j = q >> 3;
    mt = (x / gn) * bm + j / bn;
    nt = (x % gn) * bn + j % bn;
}

// Element (block i, block j, register r) of an MFMA 32x32 accumulator is row
// 8 (r/4) + 4 (l/32) + r%4 and column l%32 of that block.
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// fp32 -> bf16 / fp16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);      // v_cvt_pk_bf16_f32: RNE
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

// Two fp32 values as one word of two bf16, round to nearest even (one
// v_cvt_pk_bf16_f32; a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight fp32 values as eight bf16 through a buffer descriptor: one 16-byte
// non-temporal store (the kernels never read these outputs back).
__device__ __forceinline__ void store_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[8]) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 w = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3]),
                     (int)pack_bf16x2(v[4], v[5]), (int)pack_bf16x2(v[6], v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 2);
}

// dtype codes (the gg_dtype values of the ABI)
constexpr int kBF16 = 0, kF16 = 1, kF32 = 2, kF8 = 3, kF8E5M2 = 4;   // gg_dtype codes

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

// Stores of results the kernel does not read again are non-temporal.
__device__ __forceinline__ void store8(void* base, int dtype, int64_t i, const float (&v)[8]) {
    if (dtype == kF32) {
        u32x4 a, b;
        a.x = __builtin_bit_cast(uint32_t, v[0]); a.y = __builtin_bit_cast(uint32_t, v[1]);
        a.z = __builtin_bit_cast(uint32_t, v[2]); a.w = __builtin_bit_cast(uint32_t, v[3]);
        b.x = __builtin_bit_cast(uint32_t, v[4]); b.y = __builtin_bit_cast(uint32_t, v[5]);
        b.z = __builtin_bit_cast(uint32_t, v[6]); b.w = __builtin_bit_cast(uint32_t, v[7]);
        __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>((float*)base + i));
        __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>((float*)base + i + 4));
    } else {
        uint32_t ws[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
            ws[k] = dtype == kBF16 ? pack_bf16x2(v[2 * k], v[2 * k + 1])
                                   : (uint32_t)f32_to_f16(v[2 * k]) |
                                         ((uint32_t)f32_to_f16(v[2 * k + 1]) << 16);
        __builtin_nontemporal_store(u32x4{ws[0], ws[1], ws[2], ws[3]},
                                    reinterpret_cast<u32x4*>((uint16_t*)base + i));
    }
}

// Eight FP8 codes (E4M3, or E5M2 when dtype is kF8E5M2) to fp32, exactly.
__device__ __forceinline__ void unpack8_8(uint32_t lo, uint32_t hi, int dtype, float (&v)[8]) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const uint32_t ws[2] = {lo, hi};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        f32x2 a, b;
        if (dtype == kF8E5M2) {
            a = __builtin_amdgcn_cvt_pk_f32_bf8((int)ws[h], false);
            b = __builtin_amdgcn_cvt_pk_f32_bf8((int)ws[h], true);
        } else {
            a = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[h], false);
            b = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[h], true);
        }
        v[4 * h] = a.x;
        v[4 * h + 1] = a.y;
        v[4 * h + 2] = b.x;
        v[4 * h + 3] = b.y;
    }
}

// ---------------------------------------------------------------------------
// Raw loads of 8 consecutive elements of CW bytes each (CW 1: FP8 codes, 8
// bytes; 2: bf16 / fp16, 16 bytes; 4: fp32, 32 bytes), converted to fp32
// only when used, so that a caller can have many in flight.  The element
// index is a multiple of 8.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int CW>
struct RawC {
    static_assert(CW == 1 || CW == 2 || CW == 4, "element widths 1, 2, 4");
    std::conditional_t<CW == 1, u32x2, u32x4> w[CW == 4 ? 2 : 1];
};

template <int CW>
__device__ __forceinline__ RawC<CW> rawc_load(const void* base, int64_t i) {
    RawC<CW> r;
    if constexpr (CW == 4) {
        r.w[0] = *reinterpret_cast<const u32x4*>((const float*)base + i);
        r.w[1] = *reinterpret_cast<const u32x4*>((const float*)base + i + 4);
    } else if constexpr (CW == 2) {
        r.w[0] = *reinterpret_cast<const u32x4*>((const uint16_t*)base + i);
    } else {
        r.w[0] = *reinterpret_cast<const u32x2*>((const uint8_t*)base + i);
    }
    return r;
}

// dtype: kF32 for CW 4; kBF16 or kF16 for CW 2; kF8 or kF8E5M2 for CW 1.
template <int CW>
__device__ __forceinline__ void rawc_cvt(const RawC<CW>& r, int dtype, float (&v)[8]) {
    if constexpr (CW == 4) {
        const uint32_t ws[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w,
                                r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
        for (int k = 0; k < 8; k++)
            v[k] = __builtin_bit_cast(float, ws[k]);
    } else if constexpr (CW == 2) {
        unpack8_16(r.w[0], dtype, v);
    } else {
        unpack8_8(r.w[0].x, r.w[0].y, dtype, v);
    }
}

// ---------------------------------------------------------------------------
// Eight consecutive elements of a bf16 / fp16 / fp32 row (16 or 32 bytes)
// through a buffer descriptor, with the element type a runtime value and no
// branch: both 16-byte halves are always issued, the second at kInvalid
// (load zeros / store nothing) for 16-bit types, and conversions select
// between the formats.  An item whose offset is kInvalid is masked the same
// way.  Branch-free item code keeps the compiler's memory-counter waits
// exact, so that many loads can be in flight ahead of their use.
// ---------------------------------------------------------------------------
struct RawB8 {
    u32x4 w[2];
};

// Bitwise select (mask all ones: a, all zeros: b): the conditions here are
// workgroup-uniform, and a ternary would let the compiler branch.
__device__ __forceinline__ uint32_t bsel(uint32_t mask, uint32_t a, uint32_t b) {
    return (a & mask) | (b & ~mask);
}

// Element format of a row piece: bytes per element and, for 16-bit, fp16
// rather than bf16 (w32, f16 as flags; m32, m16 as all-ones masks).
struct Fmt8 {
    uint32_t w32, f16, m32, m16;
    __device__ __forceinline__ explicit Fmt8(int dtype)
        : w32(dtype == kF32), f16(dtype == kF16), m32(0u - w32), m16(0u - f16) {}
    // byte offset of element i (a multiple of 8), or kInvalid
    __device__ __forceinline__ uint32_t off(bool ok, int64_t i) const {
        return ok ? (uint32_t)(i << (w32 ? 2 : 1)) : kInvalid;
    }
};

__device__ __forceinline__ RawB8 rawb8_load(__amdgpu_buffer_rsrc_t r, const Fmt8& fm, uint32_t off) {
    RawB8 x;
    x.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    x.w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          r, fm.w32 ? off + 16 : kInvalid, 0, 0));
    return x;
}

__device__ __forceinline__ void rawb8_cvt(const RawB8& x, const Fmt8& fm, float (&v)[8]) {
    const uint32_t ws[8] = {x.w[0].x, x.w[0].y, x.w[0].z, x.w[0].w,
                            x.w[1].x, x.w[1].y, x.w[1].z, x.w[1].w};
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint32_t h = (ws[k >> 1] >> (16 * (k & 1))) & 0xffffu;   // 16-bit element k
        const uint32_t v16 = bsel(fm.m16, __builtin_bit_cast(uint32_t, f16_to_f32((uint16_t)h)), h << 16);
        v[k] = __builtin_bit_cast(float, bsel(fm.m32, ws[k], v16));
    }
}

__device__ __forceinline__ void rawb8_store(__amdgpu_buffer_rsrc_t r, const Fmt8& fm, uint32_t off,
                                           const float (&v)[8]) {
    uint32_t a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t lo = bsel(fm.m16, f32_to_f16(v[2 * k]), f32_to_bf16(v[2 * k]));
        const uint32_t hi = bsel(fm.m16, f32_to_f16(v[2 * k + 1]), f32_to_bf16(v[2 * k + 1]));
        a[k] = bsel(fm.m32, __builtin_bit_cast(uint32_t, v[k]), lo | (hi << 16));
        b[k] = __builtin_bit_cast(uint32_t, v[4 + k]);
    }
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)a[0], (int)a[1], (int)a[2], (int)a[3]}, r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, r,
                                           fm.w32 ? off + 16 : kInvalid, 0, 0);
}

// Cross-lane steps in the vector ALU (no LDS round trip).  dpp<CTRL>(v):
// the value of the lane a DPP control selects (0xB1: lane ^ 1, 0x4E: lane ^
// 2, 0x124 / 0x128: lane - 4 / - 8 within the 16-lane row, rotating).
// x16 / x32(v, op): op of v and its lane ^ 16 / lane ^ 32 partner's, through
// v_permlane16_swap / v_permlane32_swap, whose two results (both operands v)
// hold the lane's own v and its partner's -- the order does not matter to a
// commutative op.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, true));
}
template <class Op>
__device__ __forceinline__ float x16(float v, Op op) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                    __builtin_bit_cast(unsigned, v), false, false);
    return op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
template <class Op>
__device__ __forceinline__ float x32(float v, Op op) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                    __builtin_bit_cast(unsigned, v), false, false);
    return op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
struct MaxOp {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
    __device__ float operator()(float a, float b) const { return a + b; }
};

// Max of v over the lanes of a quad (lane ^ 1, ^ 2), in every lane.
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    return fmaxf(v, dpp<0x4E>(v));
}

// Max of v over the wave, in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = quad_max(v);
    v = fmaxf(v, dpp<0x124>(v));              // the 16-lane row: quads q, q - 1, ...
    v = fmaxf(v, dpp<0x128>(v));
    return x32(x16(v, MaxOp()), MaxOp());
}

// op of v over the lanes that differ in bits 3, 4 and 5 (lane ^ 8, ^ 16,
// ^ 32), in every lane: the pairwise tree of a butterfly on those bits.
template <class Op>
__device__ __forceinline__ float cols8(float v, Op op) {
    v = op(v, dpp<0x128>(v));
    return x32(x16(v, op), op);
}

// Sum of v over the 8 lanes that share lane >> 3 (a row of the row walk),
// complete in the lanes with (lane & 7) >= 4; lanes 0 .. 3 of each group end
// with a partial sum.  Two quad permutations (lane ^ 1, lane ^ 2) and a shift
// by 4 within the 16-lane DPP row, all in the vector ALU: the same pairwise
// tree as a lane ^ 1, ^ 2, ^ 4 butterfly, so the same sum.
__device__ __forceinline__ float row8_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x114, 0xF, 0xF, true));
    return v;
}

// ---------------------------------------------------------------------------
// Row walk of a wave's accumulators (32 MB rows x 32 NB columns, MB and NB
// even).  The MFMA layout gives a lane one column and 16 rows of a block;
// stores want a lane to own consecutive columns of one row.  The walk stages
// kQR x 64 pieces (kQR = 64: quadrants of 2 x 2 blocks, the wave's LDS
// region kEpiWaveBytes; kQR = 32: 1 x 2 blocks, kEpiHalfBytes) through the
// wave's private LDS region and visits, for lane l, the items (t, r, c): the
// 8 columns [c, c+8) of wave-tile row r, r = (l >> 3) + 8 t,
// t = 0 .. 4 MB - 1, c = 8 (l & 7) + 64 h; for each h the t values come in
// increasing order.  The caller's loads run kAhead items ahead of their use,
// so that many are in flight at once:
//   load(t, r, c)            queue the loads of an item, returning them;
//   fn(t, r, c, v, pre)      process an item with its accumulators v (fp32)
//                            and what load returned for it.
// Only this wave touches `lds`; the caller separates it from the main loop
// with a barrier.  Items [kFrom, kTo) alone are visited (kTo < 0: to the
// end), whole pieces, so that a caller can split the walk.  kLdsAhead reads
// each item's accumulators one item early (for one wave per SIMD, where
// nothing else covers the LDS latency: 2-3% on the block-scaled dsReLU and
// dGLU; with two waves per SIMD it measured no gain, and it cost registers
// in the FP8-output and run-time-format walks).
// ---------------------------------------------------------------------------
constexpr int kEpiHalfBytes = 32 * kEpiPitch * 4;

template <class C, int kAhead, int kQR = 64, int kFrom = 0, int kTo = -1, bool kLdsAhead = false,
          class Load, class Fn>
__device__ __forceinline__ void for_each_row8(const f32x16 (&acc)[C::MB][C::NB], float* lds, Load load,
                                              Fn fn) {
    static_assert(C::MB % 2 == 0 && C::NB % 2 == 0, "row walk expects 64 x 64 quadrants");
    static_assert(kQR == 64 || kQR == 32, "staged pieces of 64 or 32 rows");
    constexpr int kBR = kQR / 32;                        // block rows per piece
    constexpr int kPer = kQR / 8;                        // items per piece
    constexpr int kAll = 8 * (C::MB / 2) * (C::NB / 2);
    constexpr int kItems = kTo < 0 ? kAll : kTo;
    static_assert(kFrom % kPer == 0 && kItems % kPer == 0 && kFrom < kItems && kItems <= kAll,
                  "whole pieces");
    const int l = threadIdx.x & 63;
    // item i: piece q = i / kPer (h = q / (MB/kBR), mh = q % (MB/kBR)), ti = i % kPer
    auto item = [&](int i, int& t, int& r, int& c) {
        const int q = i / kPer, h = q / (C::MB / kBR), mh = q % (C::MB / kBR), ti = i % kPer;
        t = kPer * mh + ti;
        r = kQR * mh + (l >> 3) + 8 * ti;
        c = 64 * h + 8 * (l & 7);
    };
    using P = decltype(load(0, 0, 0));
    P pre[kItems];
#pragma unroll
    for (int i = kFrom; i < kFrom + kAhead && i < kItems; i++) {
        int t, r, c;
        item(i, t, r, c);
        pre[i] = load(t, r, c);
    }
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    // the piece that item i starts, into the wave's region
    auto stage = [&](int i) {
        const int q = i / kPer, h = q / (C::MB / kBR), mh = q % (C::MB / kBR);
#pragma unroll
        for (int b = 0; b < kBR; b++)
#pragma unroll
            for (int jj = 0; jj < 2; jj++)
#pragma unroll
                for (int e = 0; e < 16; e++)
                    lds[(32 * b + acc_row(e, l)) * kEpiPitch + 32 * jj + (l & 31)] =
                        acc[kBR * mh + b][2 * h + jj][e];
    };
    auto fetch = [&](int i, f32x4& a, f32x4& b) {
        int t, r, c;
        item(i, t, r, c);
        const int rq = r % kQR, cq = c & 63;
        a = *reinterpret_cast<const f32x4*>(lds + rq * kEpiPitch + cq);
        b = *reinterpret_cast<const f32x4*>(lds + rq * kEpiPitch + cq + 4);
    };
    // kLdsAhead: item i+1's accumulators are read before item i is
    // processed, so that the LDS latency hides behind item i's arithmetic
    // (a wave's LDS accesses complete in issue order, so the next piece may
    // be written over the one whose last reads are still in flight).
    // Otherwise each item's reads come right before its use.
    f32x4 ca, cb;
    stage(kFrom);
    if constexpr (kLdsAhead)
        fetch(kFrom, ca, cb);
#pragma unroll
    for (int i = kFrom; i < kItems; i++) {
        f32x4 na, nb;
        if constexpr (kLdsAhead) {
            if (i + 1 < kItems) {
                if ((i + 1) % kPer == 0)
                    stage(i + 1);
                fetch(i + 1, na, nb);
            }
        } else if (i > kFrom && i % kPer == 0) {
            stage(i);
        }
        if (i + kAhead < kItems) {
            int t, r, c;
            item(i + kAhead, t, r, c);
            pre[i + kAhead] = load(t, r, c);
        }
        if constexpr (!kLdsAhead)
            fetch(i, ca, cb);
        int t, r, c;
        item(i, t, r, c);
        float v[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        fn(t, r, c, v, pre[i]);
        if constexpr (kLdsAhead) {
            if (i + 1 < kItems) {
                ca = na;
                cb = nb;
            }
        }
    }
}

// Loads of one row-walk item: NC raw 8-element loads and one fp32 per-row
// value (plain pointers, compile-time width; or buffer descriptors, runtime
// width).
template <int CW, int NC>
struct Pre8 {
    RawC<CW> x[NC];
    float row;
};
template <int NC>
struct PreB8 {
    RawB8 x[NC];
    float row;
};

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
