// gg_internal.hpp -- parameter blocks and launchers shared between the host
// API (gg_api.cpp) and the kernel translation units.  Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdio>

namespace gg {

// Workspace layout (every op): a 256-byte header whose first int32 is the
// device error word, followed by the op's own region.
constexpr size_t kWsHeader = 256;
// int32 index, in the header, of the 8 work-queue counters of the persistent
// wgrad kernel (one per XCD), cleared by the set-up kernel
constexpr int kWsQueue = 16;
// wgrad region after the header: by rank (experts by token count, largest
// first) an int32 x 4 entry {expert, offsets[expert-1] (0 for the first),
// offsets[expert], 0}, written by the set-up kernel
constexpr size_t kWsRankBytes = 16;

// Compute units of the current device (cached per device), and the grid of a
// persistent kernel over `items` work items: one workgroup per CU, a multiple
// of 8 so that every XCD gets the same number, and at least 8 (or one per
// item) so that every XCD's queue is served.
inline int cu_count() {
    // host threads may race to fill an entry; they all store the same value
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
inline int64_t persistent_grid(int64_t items) {
    int64_t g = cu_count() & ~7;
    if (g > items)
        g = items >= 8 ? (items & ~7) : items;
    if (g < 8 && items >= 8)
        g = 8;
    return g;
}

// FP8 outputs of the block-scaled dgrad epilogues (d_dtype E4M3).
struct Fp8Out {
    uint8_t* d_row;           // (rows, W) codes
    uint8_t* d_col;           // (rows, W) codes, or null
    uint8_t* sfd_row;         // (rows, W/32)
    uint8_t* sfd_col;         // (W, pitch): column c, row block j at c * pitch + j
    const float* norm_const;  // [1]
    int64_t W, pitch;
};

struct WgradArgs {
    const void* a;            // bf16, or FP8 codes (block-scaled)
    const void* b;
    const uint8_t* sfa;       // block-scaled only: E8M0 scales of A and B
    const uint8_t* sfb;
    const int32_t* offsets;
    int32_t* ws;              // header + rank table (E entries of kWsRankBytes)
    void* out_dense;
    const int64_t* out_ptrs;
    int64_t T;
    int hidden, inter, E;
    int a_kmajor, b_kmajor;
    int ragged;               // K-major operands stored tensor_ragged
    int static_sched;         // persistent kernel: fixed item order, no queue
    int ab_e5m2;              // block-scaled only: codes E5M2 (else E4M3)
    int xcd_gm;               // XCD block grid rows for xcd_remap2d (0: 1-D remap)
    int out_dtype, accumulate;
};

struct DgluArgs {
    const void* a;            // bf16, or E4M3 codes (block-scaled)
    const void* b_dense;
    const int64_t* b_ptrs;
    const uint8_t* sfa;       // block-scaled only: E8M0 scales of A and B
    const uint8_t* sfb_dense;
    const int64_t* sfb_ptrs;
    float* amax;              // block-scaled only: [L][2] or NULL
    const void* c;
    const int32_t* po;
    const float* alpha;
    const float* beta;
    const float* prob;
    void* d;
    float* dprob;
    void* dbias;
    int32_t* ws;              // header + float dbias accumulators [L][2N]
    int64_t m_rows;
    int K, N, L;
    int b_kmajor;
    int c_dtype, d_dtype;
    int act;                  // 0 dSwiGLU, 1 dGeGLU, 2 dSiTU-GLU (block-scaled)
    int gate_first, mask_filter;
    float geglu_alpha, clamp_min, clamp_max, linear_offset;
    float situ_b1, situ_b2;   // dSiTU-GLU tanh scales
    int ab_e5m2;              // block-scaled only: codes E5M2 (else E4M3)
    Fp8Out q;                 // block-scaled only, with an FP8 d_dtype
};

struct DsreluArgs {
    const uint8_t* a;
    const uint8_t* sfa;
    const uint8_t* b_dense;
    const uint8_t* sfb_dense;
    const int64_t* b_ptrs;
    const int64_t* sfb_ptrs;
    const void* c;
    const int32_t* po;
    const float* alpha;
    const float* prob;
    void* d;
    float* dprob;
    float* amax;
    int32_t* ws;
    int64_t m_rows;
    int K, N, L;
    int b_kmajor;             // B's codes (N, K) per expert (else (K, N))
    int c_dtype, d_dtype;
    int ab_e5m2;              // codes E5M2 (else E4M3)
    Fp8Out q;                 // with an FP8 d_dtype
};

// Launchers (return the HIP status of the launch).
// Name of a gg_dtype code, for diagnostics.
inline const char* dtype_name(int d) {
    static const char* const kNames[] = {"bf16", "fp16", "fp32", "e4m3", "e5m2"};
    return d >= 0 && d < 5 ? kNames[d] : "?";
}

// What a launcher chose (reported when GG_LOG is set): the kernel and its
// variant, the workgroup tile, waves per workgroup and grid size.
struct LaunchInfo {
    char kernel[112];
    int tm, tn, waves;
    int64_t grid;
};

hipError_t launch_wgrad(const WgradArgs& p, hipStream_t s, LaunchInfo* info);
hipError_t launch_wgrad_mx(const WgradArgs& p, hipStream_t s, LaunchInfo* info);
hipError_t launch_dglu(const DgluArgs& p, hipStream_t s, LaunchInfo* info);
hipError_t launch_dglu_mx(const DgluArgs& p, hipStream_t s, LaunchInfo* info);
hipError_t launch_dsrelu(const DsreluArgs& p, hipStream_t s, LaunchInfo* info);

// Prologue: clears the error word, `nclear` floats at `clear` and `nclear2`
// floats at `clear2`, checks the offsets (wgrad: last == total; dgrad: last
// <= total) and, when order is non-NULL, writes the rank table (kWsRankBytes
// per expert, largest count first) there.
hipError_t launch_prologue(const int32_t* offsets, int n, int64_t total, int dgrad,
                           int32_t* err, int32_t* order, float* clear, int64_t nclear,
                           float* clear2, int64_t nclear2, hipStream_t s);
// dbias[i] = bf16(float(dbias[i]) + acc[i]) for i < n.
hipError_t launch_dbias_finalize(uint16_t* dbias, const float* acc, int64_t n, hipStream_t s);

}  // namespace gg
