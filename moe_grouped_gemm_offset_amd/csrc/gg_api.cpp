// gg_api.cpp -- the C ABI of libgg_moe (declared in include/gg_moe.h).
//
// Every entry point validates its arguments on the host first (pointers,
// enums, sizes, alignment, the one-of output / weight modes), so a rejected
// call queues no device work.  Only then does it check that the current
// device is a gfx950, and queue: a set-up kernel (clears the workspace,
// checks offsets on the device, ranks experts), the grouped GEMM, and for
// dGLU with dbias a finalize kernel -- all on the caller's stream.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gg_moe.h"
#include "gg_internal.hpp"

namespace {

// The last error message of this thread (a fixed buffer: no entry point
// allocates memory, on any path).
thread_local char g_err[512];

gg_status fail(gg_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

gg_status ok() {
    g_err[0] = '\0';
    return GG_OK;
}

// GG_LOG set (to anything but "0"): every launch reports the kernel variant
// it chose, the workgroup tile and the grid on stderr, one line per call.
// Read at every call (a getenv, no allocation).
bool log_enabled() {
    const char* v = getenv("GG_LOG");
    return v && *v && strcmp(v, "0") != 0;
}

void log_launch(const char* op, const gg::LaunchInfo& i, const char* shape) {
    fprintf(stderr, "[gg] %s %s: %s, tile %dx%d, %d waves, grid %lld\n", op, shape, i.kernel,
            i.tm, i.tn, i.waves, (long long)i.grid);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_out_dtype(gg_dtype d) { return d == GG_BF16 || d == GG_F16 || d == GG_F32; }

bool is_fp8(gg_dtype d) { return d == GG_F8E4M3 || d == GG_F8E5M2; }

// Current device must be a gfx950; the answer is cached per device ordinal.
gg_status check_device() {
    static std::mutex mu;
    static int cache[64];            // 0 unknown, 1 gfx950, 2 other
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(GG_ERR_DEVICE, "no HIP device is available");
    if (dev >= 64)
        return fail(GG_ERR_DEVICE, "device ordinal %d is beyond the 64 this library tracks", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(GG_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (cache[dev] != 1)
            return fail(GG_ERR_DEVICE, "device %d is %s; this library is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (cache[dev] != 1)
        return fail(GG_ERR_DEVICE, "device %d is not a gfx950", dev);
    return GG_OK;
}

gg_status hip_fail(hipError_t e, const char* what) {
    return fail(GG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// GG_FLAG_VALIDATE_OFFSETS: read the offsets on the host and apply the
// pages' rules.  dgrad: last <= total; wgrad: last == total.
gg_status validate_offsets_host(const int32_t* offsets, int n, int64_t total, bool dgrad,
                                hipStream_t s) {
    // n <= 1024 (every caller checks the group count first): a stack buffer,
    // so that no entry point allocates, not even host memory
    int32_t h[1024];
    if (n < 0 || n > 1024)
        return fail(GG_ERR_SHAPE, "offsets arrays hold 1..1024 entries");
    hipError_t e = hipMemcpyAsync(h, offsets, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_fail(e, "reading offsets");
    int64_t prev = 0;
    for (int i = 0; i < n; i++) {
        if (h[i] < prev)
            return fail(GG_ERR_OFFSETS, "offsets[%d] = %d is smaller than its predecessor %lld", i,
                        h[i], (long long)prev);
        if ((h[i] - prev) % 256 != 0)
            return fail(GG_ERR_OFFSETS, "group %d has %lld rows, not a multiple of 256", i,
                        (long long)(h[i] - prev));
        prev = h[i];
    }
    if (dgrad ? prev > total : prev != total)
        return fail(GG_ERR_OFFSETS, "last offset %lld %s %lld", (long long)prev,
                    dgrad ? "exceeds the row count" : "differs from tokens_sum", (long long)total);
    return GG_OK;
}

// Scratch of gg_wgrad_noalloc, for callers that cannot allocate: the
// workspace of a wgrad call with up to 1024 experts (header, then the
// 16-byte rank table).  Each GPU holds its own copy for the life of the process; host
// code reaches it only through the address hipGetSymbolAddress returns for
// the current device (the array's name is a host-side stand-in).
constexpr size_t kNoallocBytes = gg::kWsHeader + gg::kWsRankBytes * 1024;
static __device__ __align__(256) int32_t scratch[kNoallocBytes / sizeof(int32_t)];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
gg_status scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(GG_ERR_DEVICE, "no HIP device is available");
    if (dev >= 64)
        return fail(GG_ERR_DEVICE, "device ordinal %d is beyond the 64 this library tracks", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GG_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return GG_OK;
}

}  // namespace

extern "C" {

int gg_abi_version(void) { return GG_ABI_VERSION; }

const char* gg_last_error(void) { return g_err; }

gg_status gg_device_error(const void* workspace, void* stream, int32_t* code) {
    if (!workspace || !code)
        return fail(GG_ERR_NULL, "workspace and code must be non-NULL");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess)
        e = hipMemcpy(code, workspace, sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "reading the device error word");
    return ok();
}

size_t gg_wgrad_workspace_size(int32_t num_experts) {
    if (num_experts < 0)
        num_experts = 0;
    return round256(gg::kWsHeader + gg::kWsRankBytes * (size_t)num_experts);
}

size_t gg_dglu_workspace_size(int32_t L, int32_t n, int32_t generate_dbias) {
    size_t extra = generate_dbias && L > 0 && n > 0 ? sizeof(float) * (size_t)L * 2 * (size_t)n : 0;
    return round256(gg::kWsHeader + extra);
}

size_t gg_dsrelu_workspace_size(int32_t L) {
    (void)L;
    return round256(gg::kWsHeader);
}

// Host checks of the shared wgrad arguments that need neither the device nor
// the workspace.
static gg_status wgrad_host_checks(const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                                   int32_t hidden, int32_t intermediate, void* wgrad_dense,
                                   const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype, uint32_t flags,
                                   bool mx, const char* name) {
    if (!is_out_dtype(wgrad_dtype))
        return fail(GG_ERR_DTYPE, "wgrad_dtype must be GG_BF16, GG_F16 or GG_F32");
    if ((wgrad_dense != nullptr) == (wgrad_ptrs != nullptr))
        return fail(GG_ERR_MODE, "exactly one of wgrad_dense and wgrad_ptrs must be given");
    if (num_experts < 1 || num_experts > 1024)
        return fail(GG_ERR_SHAPE, "num_experts must be in 1..1024 (got %d)", num_experts);
    if (tokens_sum < 0 || tokens_sum > INT32_MAX)
        return fail(GG_ERR_SHAPE, "tokens_sum must be in 0..2^31-1");
    if (hidden <= 0 || intermediate <= 0)
        return fail(GG_ERR_SHAPE, "hidden and intermediate must be positive");
    if (hidden % 64 || intermediate % 64)
        return fail(GG_ERR_UNSUPPORTED, "hidden and intermediate must be multiples of 64");
    if (mx ? tokens_sum % 128 : tokens_sum % 8)
        return fail(GG_ERR_ALIGN, mx ? "tokens_sum must be a multiple of 128"
                                     : "tokens_sum must be a multiple of 8 (16-byte rows)");
    // tile-relative 32-bit buffer offsets: 256 rows of the largest pitch
    if (tokens_sum > (1 << 21) || hidden > (1 << 21) || intermediate > (1 << 21))
        return fail(GG_ERR_UNSUPPORTED, "tokens_sum, hidden and intermediate are limited to 2^21");
    // the work items (256 x 256 output tiles of every expert) are numbered in
    // int32 by the kernels' schedulers
    if ((int64_t)((hidden + 255) / 256) * ((intermediate + 255) / 256) * num_experts > (1 << 28))
        return fail(GG_ERR_UNSUPPORTED, "more than 2^28 output tiles (256 x 256, all experts)");
    if (!aligned16(wgrad_dense) || !aligned16(wgrad_ptrs) || ((uintptr_t)offsets & 3u))
        return fail(GG_ERR_ALIGN, "the output must be 16-byte aligned, offsets 4-byte");
    if (flags & ~(uint32_t)(GG_FLAG_VALIDATE_OFFSETS | GG_FLAG_TENSOR_RAGGED | GG_FLAG_STATIC_SCHED |
                            (mx ? GG_FLAG_AB_E5M2 : 0u)))
        return fail(GG_ERR_MODE, "unsupported flags 0x%x for %s", flags, name);
    return GG_OK;
}

// Checks shared by the wgrad entries (all but the operand pointers, majors
// and scales), then the prologue and the launch.
static gg_status run_wgrad(gg::WgradArgs& p, bool mx, const int32_t* offsets, int32_t num_experts,
                           int64_t tokens_sum, int32_t hidden, int32_t intermediate,
                           void* wgrad_dense, const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype,
                           int32_t accumulate, uint32_t flags, void* workspace,
                           size_t workspace_bytes, void* stream) {
    gg_status st = wgrad_host_checks(offsets, num_experts, tokens_sum, hidden, intermediate,
                                     wgrad_dense, wgrad_ptrs, wgrad_dtype, flags, mx,
                                     mx ? "gg_wgrad_mx" : "gg_wgrad");
    if (st != GG_OK)
        return st;
    if ((uintptr_t)workspace & 255u)
        return fail(GG_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < gg_wgrad_workspace_size(num_experts))
        return fail(GG_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
                    gg_wgrad_workspace_size(num_experts));
    st = check_device();
    if (st != GG_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (flags & GG_FLAG_VALIDATE_OFFSETS) {
        st = validate_offsets_host(offsets, num_experts, tokens_sum, false, s);
        if (st != GG_OK)
            return st;
    }
    int32_t* ws = (int32_t*)workspace;
    hipError_t e = gg::launch_prologue(offsets, num_experts, tokens_sum, 0, ws,
                                       ws + gg::kWsHeader / 4, nullptr, 0, nullptr, 0, s);
    if (e != hipSuccess)
        return hip_fail(e, "launching the wgrad prologue");
    p.offsets = offsets;
    p.ws = ws;
    p.out_dense = wgrad_dense;
    p.out_ptrs = wgrad_ptrs;
    p.T = tokens_sum;
    p.hidden = hidden;
    p.inter = intermediate;
    p.E = num_experts;
    p.ragged = (flags & GG_FLAG_TENSOR_RAGGED) != 0;
    p.static_sched = (flags & GG_FLAG_STATIC_SCHED) != 0;
    p.ab_e5m2 = (flags & GG_FLAG_AB_E5M2) != 0;
    // XCD blocks of an expert's tiles: the gm x (8/gm) grid that reads the
    // fewest operand panels (an A panel per M tile by 8/gm XCDs, a B panel
    // per N tile by gm), among those that divide the tile grid
    {
        const int tm = (hidden + 255) / 256, tn = (intermediate + 255) / 256;
        int best = 0, best_cost = 0;
        for (int gm = 1; gm <= 8; gm *= 2) {
            const int gn = 8 / gm;
            if (tm % gm || tn % gn)
                continue;
            const int cost = tm * gn + tn * gm;
            if (best == 0 || cost < best_cost)
                best = gm, best_cost = cost;
        }
        p.xcd_gm = best;
    }
    p.out_dtype = (int)wgrad_dtype;
    p.accumulate = accumulate ? 1 : 0;
    gg::LaunchInfo info{};
    gg::LaunchInfo* li = log_enabled() ? &info : nullptr;
    e = mx ? gg::launch_wgrad_mx(p, s, li) : gg::launch_wgrad(p, s, li);
    if (e != hipSuccess)
        return hip_fail(e, mx ? "launching gg_wgrad_mx" : "launching gg_wgrad");
    if (li && info.grid > 0) {
        char shape[128];
        snprintf(shape, sizeof shape, "(E %d, hidden %d, intermediate %d, tokens %lld, out %s%s)",
                 num_experts, hidden, intermediate, (long long)tokens_sum,
                 gg::dtype_name(p.out_dtype), p.accumulate ? " +=" : "");
        log_launch(mx ? "gg_wgrad_mx" : "gg_wgrad", info, shape);
    }
    return ok();
}

gg_status gg_wgrad(const void* a, gg_major a_major, const void* b, gg_major b_major,
                   const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                   int32_t hidden, int32_t intermediate, void* wgrad_dense,
                   const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype, int32_t accumulate,
                   uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
    if (!offsets || !workspace)
        return fail(GG_ERR_NULL, "offsets and workspace must be non-NULL");
    if ((!a || !b) && tokens_sum > 0)
        return fail(GG_ERR_NULL, "a and b must be non-NULL");
    if (a_major != GG_MAJOR_K && a_major != GG_MAJOR_M)
        return fail(GG_ERR_LAYOUT, "a_major must be GG_MAJOR_K or GG_MAJOR_M");
    if (b_major != GG_MAJOR_K && b_major != GG_MAJOR_N)
        return fail(GG_ERR_LAYOUT, "b_major must be GG_MAJOR_K or GG_MAJOR_N");
    if (!aligned16(a) || !aligned16(b))
        return fail(GG_ERR_ALIGN, "a, b and the output must be 16-byte aligned");
    gg::WgradArgs p = {};
    p.a = a;
    p.b = b;
    p.a_kmajor = a_major == GG_MAJOR_K;
    p.b_kmajor = b_major == GG_MAJOR_K;
    return run_wgrad(p, false, offsets, num_experts, tokens_sum, hidden, intermediate, wgrad_dense,
                     wgrad_ptrs, wgrad_dtype, accumulate, flags, workspace, workspace_bytes, stream);
}

gg_status gg_wgrad_noalloc(const void* a, gg_major a_major, const void* b, gg_major b_major,
                           const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                           int32_t hidden, int32_t intermediate, void* wgrad_dense,
                           const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype, int32_t accumulate,
                           uint32_t flags, void* stream) {
    if (num_experts > 0 && gg_wgrad_workspace_size(num_experts) > kNoallocBytes)
        return fail(GG_ERR_WORKSPACE,
                    "gg_wgrad_noalloc: %d experts need %zu bytes of scratch; its static scratch "
                    "holds %zu (1024 experts)",
                    num_experts, gg_wgrad_workspace_size(num_experts), kNoallocBytes);
    if (!offsets)
        return fail(GG_ERR_NULL, "offsets must be non-NULL");
    if ((!a || !b) && tokens_sum > 0)
        return fail(GG_ERR_NULL, "a and b must be non-NULL");
    if (a_major != GG_MAJOR_K && a_major != GG_MAJOR_M)
        return fail(GG_ERR_LAYOUT, "a_major must be GG_MAJOR_K or GG_MAJOR_M");
    if (b_major != GG_MAJOR_K && b_major != GG_MAJOR_N)
        return fail(GG_ERR_LAYOUT, "b_major must be GG_MAJOR_K or GG_MAJOR_N");
    if (!aligned16(a) || !aligned16(b))
        return fail(GG_ERR_ALIGN, "a, b and the output must be 16-byte aligned");
    gg::WgradArgs p = {};
    p.a = a;
    p.b = b;
    p.a_kmajor = a_major == GG_MAJOR_K;
    p.b_kmajor = b_major == GG_MAJOR_K;
    // the scratch address is looked up only for a call that passes every
    // host check
    gg_status st = wgrad_host_checks(offsets, num_experts, tokens_sum, hidden, intermediate,
                                     wgrad_dense, wgrad_ptrs, wgrad_dtype, flags, false,
                                     "gg_wgrad_noalloc");
    if (st != GG_OK)
        return st;
    st = check_device();
    if (st != GG_OK)
        return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != GG_OK)
        return st;
    return run_wgrad(p, false, offsets, num_experts, tokens_sum, hidden, intermediate, wgrad_dense,
                     wgrad_ptrs, wgrad_dtype, accumulate, flags, ws, kNoallocBytes, stream);
}

gg_status gg_wgrad_mx(const void* a_fp8, const uint8_t* sfa, const void* b_fp8, const uint8_t* sfb,
                      const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                      int32_t hidden, int32_t intermediate, void* wgrad_dense,
                      const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype, int32_t accumulate,
                      uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
    if (!offsets || !workspace)
        return fail(GG_ERR_NULL, "offsets and workspace must be non-NULL");
    if ((!a_fp8 || !b_fp8 || !sfa || !sfb) && tokens_sum > 0)
        return fail(GG_ERR_NULL, "a_fp8, sfa, b_fp8 and sfb must be non-NULL");
    if (!aligned16(a_fp8) || !aligned16(b_fp8) || ((uintptr_t)sfa & 3u) || ((uintptr_t)sfb & 3u))
        return fail(GG_ERR_ALIGN, "codes must be 16-byte aligned, scales 4-byte aligned");
    gg::WgradArgs p = {};
    p.a = a_fp8;
    p.b = b_fp8;
    p.sfa = sfa;
    p.sfb = sfb;
    p.a_kmajor = p.b_kmajor = 1;
    return run_wgrad(p, true, offsets, num_experts, tokens_sum, hidden, intermediate, wgrad_dense,
                     wgrad_ptrs, wgrad_dtype, accumulate, flags, workspace, workspace_bytes, stream);
}

static gg_status check_rows(const int32_t* po, int32_t L, int64_t m_rows, const void* c,
                            const float* prob, const void* d_row, const float* dprob,
                            void* workspace) {
    if (!po || !c || !prob || !d_row || !dprob || !workspace)
        return fail(GG_ERR_NULL, "padded_offsets, c, prob, d_row, dprob and workspace must be non-NULL");
    if (L < 1 || L > 1024)
        return fail(GG_ERR_SHAPE, "the expert count must be in 1..1024 (got %d)", L);
    if (m_rows < 0 || m_rows > INT32_MAX)
        return fail(GG_ERR_SHAPE, "m_rows must be in 0..2^31-1");
    if (!aligned16(c) || !aligned16(d_row) || ((uintptr_t)prob & 3u) || ((uintptr_t)dprob & 3u) ||
        ((uintptr_t)po & 3u))
        return fail(GG_ERR_ALIGN, "c and d_row must be 16-byte aligned, prob/dprob 4-byte");
    if ((uintptr_t)workspace & 255u)
        return fail(GG_ERR_ALIGN, "workspace must be 256-byte aligned");
    return GG_OK;
}

// Checks of the activation, output and flag arguments shared by gg_dglu and
// gg_dglu_mx.
static gg_status check_dglu_common(gg_dtype c_dtype, gg_dtype d_dtype, gg_act act, bool mx,
                                   const float* alpha, const float* beta, const void* dbias,
                                   uint32_t flags, const char* name) {
    if (!alpha || !beta)
        return fail(GG_ERR_NULL, "alpha and beta must be non-NULL");
    if (!(is_out_dtype(c_dtype) || (mx && is_fp8(c_dtype))) ||
        !(is_out_dtype(d_dtype) || (mx && is_fp8(d_dtype))))
        return fail(GG_ERR_DTYPE, mx ? "c_dtype and d_dtype must be GG_BF16, GG_F16, GG_F32, "
                                       "GG_F8E4M3 or GG_F8E5M2"
                                     : "c_dtype and d_dtype must be GG_BF16, GG_F16 or GG_F32");
    if (act == GG_DSITUGLU && !mx)
        return fail(GG_ERR_MODE, "GG_DSITUGLU is defined for the block-scaled gg_dglu_mx only");
    if (act != GG_DSWIGLU && act != GG_DGEGLU && act != GG_DSITUGLU)
        return fail(GG_ERR_MODE, "act must be GG_DSWIGLU, GG_DGEGLU or GG_DSITUGLU");
    if (!aligned16(dbias) || ((uintptr_t)alpha & 3u) || ((uintptr_t)beta & 3u))
        return fail(GG_ERR_ALIGN, "dbias must be 16-byte aligned, alpha and beta 4-byte");
    if (flags & ~(uint32_t)(GG_FLAG_GATE_FIRST | GG_FLAG_GEGLU_MASK_FILTER | GG_FLAG_VALIDATE_OFFSETS |
                            GG_FLAG_STATIC_SCHED | (mx ? GG_FLAG_AB_E5M2 : 0u)))
        return fail(GG_ERR_MODE, "unsupported flags 0x%x for %s", flags, name);
    if ((flags & GG_FLAG_AB_E5M2) && !is_fp8(d_dtype))
        return fail(GG_ERR_UNSUPPORTED, "E5M2 operands (GG_FLAG_AB_E5M2) need an FP8 d_dtype");
    return GG_OK;
}

// Fills the epilogue fields of the dGLU parameter block and queues prologue,
// kernel and dbias finalize (the operand fields are set by the caller).
static gg_status run_dglu(gg::DgluArgs& p, bool mx, const void* c, gg_dtype c_dtype,
                          const int32_t* padded_offsets, int32_t L, const float* alpha,
                          const float* beta, const float* prob, void* d_row, gg_dtype d_dtype,
                          float* dprob, void* dbias, float* amax, gg_act act, float geglu_alpha,
                          float clamp_min, float clamp_max, float linear_offset, float situ_b1,
                          float situ_b2, uint32_t flags, void* workspace, size_t workspace_bytes,
                          void* stream) {
    size_t need = gg_dglu_workspace_size(L, p.N, dbias != nullptr);
    if (workspace_bytes < need)
        return fail(GG_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    gg_status st = check_device();
    if (st != GG_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (flags & GG_FLAG_VALIDATE_OFFSETS) {
        st = validate_offsets_host(padded_offsets, L, p.m_rows, true, s);
        if (st != GG_OK)
            return st;
    }
    int32_t* ws = (int32_t*)workspace;
    float* acc = dbias ? (float*)((char*)workspace + gg::kWsHeader) : nullptr;
    const int64_t nacc = dbias ? (int64_t)L * 2 * p.N : 0;
    hipError_t e = gg::launch_prologue(padded_offsets, L, p.m_rows, 1, ws, nullptr, acc, nacc,
                                       amax, amax ? 2 * (int64_t)L : 0, s);
    if (e != hipSuccess)
        return hip_fail(e, "launching the dglu prologue");
    p.c = c;
    p.po = padded_offsets;
    p.alpha = alpha;
    p.beta = beta;
    p.prob = prob;
    p.d = d_row;
    p.dprob = dprob;
    p.dbias = dbias;
    p.amax = amax;
    p.ws = ws;
    p.L = L;
    p.c_dtype = (int)c_dtype;
    p.d_dtype = (int)d_dtype;
    p.act = (int)act;
    p.gate_first = (flags & GG_FLAG_GATE_FIRST) != 0;
    p.mask_filter = (flags & GG_FLAG_GEGLU_MASK_FILTER) != 0;
    p.geglu_alpha = geglu_alpha;
    p.clamp_min = clamp_min;
    p.clamp_max = clamp_max;
    p.linear_offset = linear_offset;
    p.situ_b1 = situ_b1;
    p.situ_b2 = situ_b2;
    gg::LaunchInfo info{};
    gg::LaunchInfo* li = log_enabled() ? &info : nullptr;
    e = mx ? gg::launch_dglu_mx(p, s, li) : gg::launch_dglu(p, s, li);
    if (e != hipSuccess)
        return hip_fail(e, mx ? "launching gg_dglu_mx" : "launching gg_dglu");
    if (li && info.grid > 0) {
        char shape[128];
        snprintf(shape, sizeof shape, "(L %d, m_rows %lld, k %d, n %d)", L, (long long)p.m_rows,
                 p.K, p.N);
        log_launch(mx ? "gg_dglu_mx" : "gg_dglu", info, shape);
    }
    if (dbias) {
        e = gg::launch_dbias_finalize((uint16_t*)dbias, acc, nacc, s);
        if (e != hipSuccess)
            return hip_fail(e, "launching the dbias finalize");
    }
    return ok();
}

// FP8 outputs (d_dtype GG_F8E4M3 / GG_F8E5M2 of the block-scaled dgrad entries): checks
// them and fills q; width is W, the columns of D.
static gg_status check_fp8_out(const gg_fp8_out* f, const void* d_row, int64_t m_rows, int64_t width,
                               gg::Fp8Out& q) {
    if (!f || !f->sfd_row || !f->norm_const)
        return fail(GG_ERR_NULL, "an FP8 d_dtype needs fp8_out with sfd_row and norm_const");
    if ((f->d_col != nullptr) != (f->sfd_col != nullptr))
        return fail(GG_ERR_MODE, "give both of fp8_out->d_col and fp8_out->sfd_col, or neither");
    if (!aligned16(f->d_col) || ((uintptr_t)f->norm_const & 3u))
        return fail(GG_ERR_ALIGN, "fp8_out->d_col must be 16-byte aligned, norm_const 4-byte");
    q.d_row = (uint8_t*)d_row;
    q.d_col = (uint8_t*)f->d_col;
    q.sfd_row = f->sfd_row;
    q.sfd_col = f->sfd_col;
    q.norm_const = f->norm_const;
    q.W = width;
    q.pitch = (m_rows + 31) / 32;
    return GG_OK;
}

gg_status gg_dglu(const void* a, int64_t m_rows, int32_t k, const void* b_dense,
                  const int64_t* b_ptrs, gg_major b_major, int32_t n, const void* c,
                  gg_dtype c_dtype, const int32_t* padded_offsets, int32_t L, const float* alpha,
                  const float* beta, const float* prob, void* d_row, gg_dtype d_dtype,
                  float* dprob, void* dbias, gg_act act, float geglu_alpha, float clamp_min,
                  float clamp_max, float linear_offset, uint32_t flags, void* workspace,
                  size_t workspace_bytes, void* stream) {
    gg_status st = check_rows(padded_offsets, L, m_rows, c, prob, d_row, dprob, workspace);
    if (st != GG_OK)
        return st;
    if (!a)
        return fail(GG_ERR_NULL, "a must be non-NULL");
    if ((b_dense != nullptr) == (b_ptrs != nullptr))
        return fail(GG_ERR_MODE, "exactly one of b_dense and b_ptrs must be given");
    if (b_major != GG_MAJOR_K && b_major != GG_MAJOR_N)
        return fail(GG_ERR_LAYOUT, "b_major must be GG_MAJOR_K or GG_MAJOR_N");
    if (b_dense && b_major != GG_MAJOR_K)
        return fail(GG_ERR_LAYOUT, "dense B must be K-major");
    st = check_dglu_common(c_dtype, d_dtype, act, false, alpha, beta, dbias, flags, "gg_dglu");
    if (st != GG_OK)
        return st;
    if (n <= 0 || n % 32)
        return fail(GG_ERR_SHAPE, "n must be a positive multiple of 32 (got %d)", n);
    if (k <= 0)
        return fail(GG_ERR_SHAPE, "k must be positive");
    if (k % 64)
        return fail(GG_ERR_UNSUPPORTED, "k must be a multiple of 64");
    if (k > (1 << 21) || n > (1 << 20))
        return fail(GG_ERR_UNSUPPORTED, "k is limited to 2^21 and n to 2^20");
    if (!aligned16(a) || !aligned16(b_dense) || !aligned16(b_ptrs))
        return fail(GG_ERR_ALIGN, "a and b must be 16-byte aligned");
    gg::DgluArgs p = {};
    p.a = a;
    p.b_dense = b_dense;
    p.b_ptrs = b_ptrs;
    p.m_rows = m_rows;
    p.K = k;
    p.N = n;
    p.b_kmajor = b_major == GG_MAJOR_K;
    return run_dglu(p, false, c, c_dtype, padded_offsets, L, alpha, beta, prob, d_row, d_dtype,
                    dprob, dbias, nullptr, act, geglu_alpha, clamp_min, clamp_max, linear_offset,
                    1.0f, 1.0f, flags, workspace, workspace_bytes, stream);
}

gg_status gg_dglu_mx(const void* a_fp8, const uint8_t* sfa, int64_t m_rows, int32_t k,
                     const void* b_fp8, const uint8_t* sfb, const int64_t* b_ptrs,
                     const int64_t* sfb_ptrs, gg_major b_major, int32_t n, const void* c,
                     gg_dtype c_dtype,
                     const int32_t* padded_offsets, int32_t L, const float* alpha,
                     const float* beta, const float* prob, void* d_row, gg_dtype d_dtype,
                     float* dprob, void* dbias, float* amax, const gg_fp8_out* fp8_out, gg_act act,
                     float geglu_alpha, float clamp_min, float clamp_max, float linear_offset,
                     float situ_beta1,
                     float situ_beta2, uint32_t flags, void* workspace, size_t workspace_bytes,
                     void* stream) {
    gg_status st = check_rows(padded_offsets, L, m_rows, c, prob, d_row, dprob, workspace);
    if (st != GG_OK)
        return st;
    if (!a_fp8 || !sfa)
        return fail(GG_ERR_NULL, "a_fp8 and sfa must be non-NULL");
    const bool dense = b_fp8 || sfb;
    const bool discrete = b_ptrs || sfb_ptrs;
    if (dense == discrete || (dense && (!b_fp8 || !sfb)) || (discrete && (!b_ptrs || !sfb_ptrs)))
        return fail(GG_ERR_MODE, "give exactly one of (b_fp8, sfb) and (b_ptrs, sfb_ptrs)");
    if (b_major != GG_MAJOR_K && b_major != GG_MAJOR_N)
        return fail(GG_ERR_LAYOUT, "b_major must be GG_MAJOR_K or GG_MAJOR_N");
    st = check_dglu_common(c_dtype, d_dtype, act, true, alpha, beta, dbias, flags, "gg_dglu_mx");
    if (st != GG_OK)
        return st;
    if (act == GG_DSITUGLU && !(situ_beta1 > 0.0f && situ_beta1 <= FLT_MAX &&
                                situ_beta2 > 0.0f && situ_beta2 <= FLT_MAX))
        return fail(GG_ERR_VALUE, "situ_beta1 and situ_beta2 must be positive and finite");
    if (n <= 0 || n % 32)
        return fail(GG_ERR_SHAPE, "n must be a positive multiple of 32 (got %d)", n);
    if (k <= 0)
        return fail(GG_ERR_SHAPE, "k must be positive");
    if (k % 128)
        return fail(GG_ERR_UNSUPPORTED, "k must be a multiple of 128");
    if (k > (1 << 21) || n > (1 << 20))
        return fail(GG_ERR_UNSUPPORTED, "k is limited to 2^21 and n to 2^20");
    if (!aligned16(a_fp8) || !aligned16(b_fp8) || !aligned16(b_ptrs) || !aligned16(sfb_ptrs) ||
        ((uintptr_t)sfa & 3u) || ((uintptr_t)sfb & 3u) || ((uintptr_t)amax & 3u))
        return fail(GG_ERR_ALIGN, "operands must be 16-byte aligned, scales and amax 4-byte aligned");
    gg::DgluArgs p = {};
    if (is_fp8(d_dtype)) {
        st = check_fp8_out(fp8_out, d_row, m_rows, 2 * (int64_t)n, p.q);
        if (st != GG_OK)
            return st;
    }
    p.a = a_fp8;
    p.sfa = sfa;
    p.b_dense = b_fp8;
    p.sfb_dense = sfb;
    p.b_ptrs = b_ptrs;
    p.sfb_ptrs = sfb_ptrs;
    p.m_rows = m_rows;
    p.K = k;
    p.N = n;
    p.b_kmajor = b_major == GG_MAJOR_K;
    p.ab_e5m2 = (flags & GG_FLAG_AB_E5M2) != 0;
    return run_dglu(p, true, c, c_dtype, padded_offsets, L, alpha, beta, prob, d_row, d_dtype,
                    dprob, dbias, amax, act, geglu_alpha, clamp_min, clamp_max, linear_offset,
                    act == GG_DSITUGLU ? situ_beta1 : 1.0f, act == GG_DSITUGLU ? situ_beta2 : 1.0f,
                    flags, workspace, workspace_bytes, stream);
}

gg_status gg_dsrelu(const void* a_fp8, const uint8_t* sfa, int64_t m_rows, int32_t k,
                    const void* b_fp8, const uint8_t* sfb, const int64_t* b_ptrs,
                    const int64_t* sfb_ptrs, gg_major b_major, int32_t n, const void* c,
                    gg_dtype c_dtype,
                    const int32_t* padded_offsets, int32_t L, const float* alpha,
                    const float* prob, void* d_row, gg_dtype d_dtype, float* dprob, float* amax,
                    const gg_fp8_out* fp8_out, uint32_t flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
    gg_status st = check_rows(padded_offsets, L, m_rows, c, prob, d_row, dprob, workspace);
    if (st != GG_OK)
        return st;
    if (!a_fp8 || !sfa || !alpha)
        return fail(GG_ERR_NULL, "a_fp8, sfa and alpha must be non-NULL");
    const bool dense = b_fp8 || sfb;
    const bool discrete = b_ptrs || sfb_ptrs;
    if (dense == discrete || (dense && (!b_fp8 || !sfb)) || (discrete && (!b_ptrs || !sfb_ptrs)))
        return fail(GG_ERR_MODE, "give exactly one of (b_fp8, sfb) and (b_ptrs, sfb_ptrs)");
    if (b_major != GG_MAJOR_K && b_major != GG_MAJOR_N)
        return fail(GG_ERR_LAYOUT, "b_major must be GG_MAJOR_K or GG_MAJOR_N");
    if (!(is_out_dtype(c_dtype) || is_fp8(c_dtype)) || !(is_out_dtype(d_dtype) || is_fp8(d_dtype)))
        return fail(GG_ERR_DTYPE, "c_dtype and d_dtype must be GG_BF16, GG_F16, GG_F32, GG_F8E4M3 or "
                                  "GG_F8E5M2");
    if (n <= 0 || n % 32)
        return fail(GG_ERR_SHAPE, "n must be a positive multiple of 32 (got %d)", n);
    if (k <= 0)
        return fail(GG_ERR_SHAPE, "k must be positive");
    if (k % 128)
        return fail(GG_ERR_UNSUPPORTED, "k must be a multiple of 128");
    if (k > (1 << 21) || n > (1 << 21))
        return fail(GG_ERR_UNSUPPORTED, "k and n are limited to 2^21");
    if (!aligned16(a_fp8) || !aligned16(b_fp8) || !aligned16(b_ptrs) || !aligned16(sfb_ptrs) ||
        ((uintptr_t)sfa & 3u) || ((uintptr_t)sfb & 3u) || ((uintptr_t)alpha & 3u) ||
        ((uintptr_t)amax & 3u))
        return fail(GG_ERR_ALIGN, "operands must be 16-byte aligned, scales 4-byte aligned");
    if (flags & ~(uint32_t)(GG_FLAG_VALIDATE_OFFSETS | GG_FLAG_STATIC_SCHED | GG_FLAG_AB_E5M2))
        return fail(GG_ERR_MODE, "unsupported flags 0x%x for gg_dsrelu", flags);
    if ((flags & GG_FLAG_AB_E5M2) && !is_fp8(d_dtype))
        return fail(GG_ERR_UNSUPPORTED, "E5M2 operands (GG_FLAG_AB_E5M2) need an FP8 d_dtype");
    size_t need = gg_dsrelu_workspace_size(L);
    if (workspace_bytes < need)
        return fail(GG_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    gg::DsreluArgs p = {};
    if (is_fp8(d_dtype)) {
        st = check_fp8_out(fp8_out, d_row, m_rows, n, p.q);
        if (st != GG_OK)
            return st;
    }
    st = check_device();
    if (st != GG_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (flags & GG_FLAG_VALIDATE_OFFSETS) {
        st = validate_offsets_host(padded_offsets, L, m_rows, true, s);
        if (st != GG_OK)
            return st;
    }
    int32_t* ws = (int32_t*)workspace;
    hipError_t e = gg::launch_prologue(padded_offsets, L, m_rows, 1, ws, nullptr, amax,
                                       amax ? L : 0, nullptr, 0, s);
    if (e != hipSuccess)
        return hip_fail(e, "launching the dsrelu prologue");
    p.a = (const uint8_t*)a_fp8;
    p.sfa = sfa;
    p.b_dense = (const uint8_t*)b_fp8;
    p.sfb_dense = sfb;
    p.b_ptrs = b_ptrs;
    p.sfb_ptrs = sfb_ptrs;
    p.c = c;
    p.po = padded_offsets;
    p.alpha = alpha;
    p.prob = prob;
    p.d = d_row;
    p.dprob = dprob;
    p.amax = amax;
    p.ws = ws;
    p.m_rows = m_rows;
    p.K = k;
    p.N = n;
    p.L = L;
    p.b_kmajor = b_major == GG_MAJOR_K;
    p.c_dtype = (int)c_dtype;
    p.d_dtype = (int)d_dtype;
    p.ab_e5m2 = (flags & GG_FLAG_AB_E5M2) != 0;
    gg::LaunchInfo info{};
    gg::LaunchInfo* li = log_enabled() ? &info : nullptr;
    e = gg::launch_dsrelu(p, s, li);
    if (e != hipSuccess)
        return hip_fail(e, "launching gg_dsrelu");
    if (li && info.grid > 0) {
        char shape[128];
        snprintf(shape, sizeof shape, "(L %d, m_rows %lld, k %d, n %d)", L, (long long)m_rows, k, n);
        log_launch("gg_dsrelu", info, shape);
    }
    return ok();
}

}  // extern "C"
