/*
 * gg_moe.h -- C ABI of libgg_moe: grouped GEMMs of the MoE expert backward
 * pass on AMD Instinct MI355X (gfx950).
 *
 * The entry points, each defined on an NVIDIA cuDNN frontend documentation
 * page (the pages describe the method; this library is an independent
 * implementation for CDNA4):
 *
 *   gg_wgrad   "Grouped GEMM + WGrad (Unified)", section "Operation":
 *              Wgrad[e] = A[:, begin:end] @ B[begin:end, :] over the token
 *              slice of expert e, accumulate or overwrite.
 *   gg_wgrad_mx  the same, section "Block-scaled contract", on MXFP8
 *              operands.
 *   gg_dglu    "Grouped GEMM + dGLU (SM100)", section "BF16 contract /
 *              Tensors, layouts, and equation": R_g = alpha_g^2 A_g B_g^T
 *              fused with the dSwiGLU / dGeGLU backward over 32-wide
 *              interleaved blocks of X_g = beta_g C_g, a dprob row reduction
 *              and an optional per-expert dbias.
 *   gg_dglu_mx "Grouped GEMM + dGLU (SM100)", section "Block-scaled
 *              contract / Equations": the same fused op on MXFP8 operands,
 *              R_g = alpha_g^2 deq(A_g) deq(B_g)^T, with the per-expert amax
 *              of the input and gate halves of D ("Shapes": (L, 2, 1)).
 *   gg_dsrelu  "Grouped GEMM + dsReLU (SM100)", section "Equations":
 *              G = alpha_g deq(A) deq(B)^T on MXFP8 operands,
 *              D_row = prob * 2 * C * relu(G), dprob = sum_n C relu(G)^2,
 *              plus the per-expert Amax of section "Shapes".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are device pointers unless marked [host].  Every buffer is
 *   owned by the caller; the library allocates no memory.  Its scratch space
 *   is the caller's `workspace` (size from the matching *_workspace_size),
 *   which makes the calls safe to capture into a HIP graph.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  Pointer arrays and the memory they point to must stay alive
 *   and unmoved until the stream has finished the call ("Output modes" of
 *   the wgrad page; the pointer-array note of the dGLU page).  Two calls that
 *   may overlap must not share a workspace (wgrad page, "Block-scaled
 *   contract", on the descriptor workspace).
 * - Every entry point returns a gg_status.  All argument checks run on the
 *   host, before any device work is queued; on failure nothing is launched
 *   and gg_last_error() holds a message.
 * - The values of offsets / padded_offsets live in device memory and are not
 *   read by the host (the pages' traced paths cannot host-validate them
 *   either).  The kernels clamp every range they derive from them, so a
 *   malformed array never causes an out-of-bounds access; the violation is
 *   recorded in the workspace's error word, readable with gg_device_error().
 *   GG_FLAG_VALIDATE_OFFSETS instead copies the array to the host, waits
 *   for `stream`, and rejects a malformed array with GG_ERR_OFFSETS.
 */
#ifndef GG_MOE_H
#define GG_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GG_ABI_VERSION 3

typedef enum {
    GG_OK = 0,
    GG_ERR_NULL = 1,         /* a required pointer is NULL                       */
    GG_ERR_SHAPE = 2,        /* a size is out of range or inconsistent           */
    GG_ERR_DTYPE = 3,        /* unsupported dtype or dtype pairing               */
    GG_ERR_LAYOUT = 4,       /* unsupported major / stride                       */
    GG_ERR_ALIGN = 5,        /* a base pointer or row pitch is not 16-B aligned  */
    GG_ERR_MODE = 6,         /* not exactly one output (wgrad) / weight mode     */
    GG_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than required          */
    GG_ERR_UNSUPPORTED = 8,  /* valid per the pages but outside this library     */
    GG_ERR_DEVICE = 9,       /* no gfx950 device current                         */
    GG_ERR_HIP = 10,         /* a HIP runtime call failed                        */
    GG_ERR_OFFSETS = 11,     /* offsets rejected by GG_FLAG_VALIDATE_OFFSETS     */
    GG_ERR_VALUE = 12        /* a scalar parameter is outside its domain         */
} gg_status;

typedef enum {
    GG_BF16 = 0,
    GG_F16 = 1,
    GG_F32 = 2,
    GG_F8E4M3 = 3,           /* OCP E4M3 ("float8_e4m3fn"): max 448, no inf     */
    GG_F8E5M2 = 4            /* OCP E5M2 ("float8_e5m2"): max 57344, inf / NaN  */
} gg_dtype;

typedef enum {
    GG_MAJOR_K = 0,          /* the reduction axis is contiguous                  */
    GG_MAJOR_M = 1,          /* the M axis (rows of the product) is contiguous    */
    GG_MAJOR_N = 2           /* the N axis (columns of the product) is contiguous */
} gg_major;

/* GG_DSITUGLU is defined for the block-scaled contract only (gg_dglu_mx). */
typedef enum { GG_DSWIGLU = 0, GG_DGEGLU = 1, GG_DSITUGLU = 2 } gg_act;

enum {
    /* dGLU: in each 64-column pair of C and D the gate block comes first.
     * Default (flag clear): the input block comes first, as the dGLU page's
     * "interleaved input/gate" C and its interleave of [dinput, dgate] say. */
    GG_FLAG_GATE_FIRST = 1u,
    /* dGeGLU: use 0/1 indicator filters (the derivative of the clamped
     * activation) instead of the page's value-bearing filters, which carry
     * the raw gate / input value inside the clamp range. */
    GG_FLAG_GEGLU_MASK_FILTER = 2u,
    /* Copy offsets / padded_offsets to the host, wait for `stream`, and
     * return GG_ERR_OFFSETS unless they are non-decreasing, every group is a
     * multiple of 256, and the last value equals tokens_sum (wgrad) or is at
     * most m_rows (dgrad).  Off by default: it synchronises the stream. */
    GG_FLAG_VALIDATE_OFFSETS = 4u,
    /* wgrad: K-major operands are stored "tensor_ragged" (the wgrad page's
     * input_order): expert e's (rows, count_e) block is K-contiguous, with
     * row pitch count_e, and the blocks are concatenated in expert order, so
     * that block e starts at element rows * offsets[e-1] (0 for e = 0).
     * M-/N-major operands hold each token contiguously either way, so the
     * flag leaves them as they are. */
    GG_FLAG_TENSOR_RAGGED = 8u,
    /* Static scheduling (the pages' use_dynamic_sched=False, dGLU page
     * "Class API").  The persistent bf16 wgrad kernel then walks its items in
     * a fixed order -- workgroup j of an XCD's W workgroups takes that XCD's
     * items j, j + W, j + 2W, ... -- instead of taking them from the XCD's
     * atomic work queue in finish order.  The results are identical.  The
     * other kernels launch one workgroup per tile, dispatched by the
     * hardware in a fixed order, so for them both settings are the same
     * schedule and the flag is accepted with no effect. */
    GG_FLAG_STATIC_SCHED = 16u,
    /* Block-scaled entries (gg_wgrad_mx, gg_dglu_mx, gg_dsrelu): the FP8
     * codes of A and B are E5M2 rather than E4M3 -- the other MXFP8 ab_dtype
     * of the dGLU page's "Data Types" table; A and B always share one format
     * ("Additional Type Constraints").  The dgrad entries take it with an
     * FP8 d_dtype only (the same section pairs FP8 operands with FP8
     * outputs), else GG_ERR_UNSUPPORTED; gg_wgrad_mx with any wgrad_dtype. */
    GG_FLAG_AB_E5M2 = 32u
};

/*
 * FP8 outputs of the block-scaled dgrad entries (gg_dglu_mx, gg_dsrelu) when
 * d_dtype is GG_F8E4M3 or GG_F8E5M2 ("Grouped GEMM + dGLU (SM100)",
 * "Block-scaled contract / Equations", step 3, and its "Data Types" d_dtype
 * column; the dsReLU page's FP8 D_row / D_col with SFD_row / SFD_col).  W is
 * the width of D (2n for dGLU, n for dsReLU).  Blocks of 32 values -- 32
 * columns of a row for d_row, 32 rows of a column for d_col -- share one
 * E8M0 scale SFD = 2^e, e the smallest integer with
 *   2^e >= fp32(fp32(norm_const * max|D|) * fp32(1/fmax))
 * fmax the format's largest value (448 for E4M3, 57344 for E5M2; the page's
 * norm_const * max|D| * rcp_max, rounded up to a power of two, which keeps
 * every code within fmax; e in [-127, 127], -127 for an all-zero block), and
 * each value is stored as fp8(D * norm_const / 2^e), clamped to +-fmax,
 * round to nearest even.  D here is the fp32 result before any rounding;
 * d_row and d_col share the one format.
 * A plain layout replaces the pages' MMA-interleaved scale tensors; the
 * column scales of one group occupy its own row-block range of every column
 * (groups are multiples of 256 rows, so no block straddles two).
 */
typedef struct {
    void* d_col;               /* (m_rows, W) FP8 column-quantized D, row-major, 16-B
                                  aligned; or NULL for no column output             */
    uint8_t* sfd_row;          /* (m_rows, W/32): row m, block b at m*(W/32) + b      */
    uint8_t* sfd_col;          /* (W, P), P = ceil(m_rows/32): column c, rows 32j ..
                                  32j+31 at c*P + j; NULL exactly when d_col is NULL */
    const float* norm_const;   /* float[1], device memory                              */
} gg_fp8_out;

/* Bits of the device error word (see gg_device_error). */
enum {
    GG_DEVERR_DECREASING = 1,   /* an offset is smaller than its predecessor   */
    GG_DEVERR_GRANULE = 2,      /* a group size is not a multiple of 256       */
    GG_DEVERR_LAST = 4,         /* last offset != tokens_sum / > m_rows        */
    GG_DEVERR_SKIPPED = 8       /* a group was too malformed to compute        */
};

/* ABI version of the loaded library (GG_ABI_VERSION of its build). */
int gg_abi_version(void);

/* Message for the last non-GG_OK status returned on this thread ("" if
 * none).  Valid until the next gg_* call on the same thread. */
const char* gg_last_error(void);

/* Waits for `stream`, then stores into *code [host] the device error word
 * that the last call using `workspace` left (0 = no violation; otherwise an
 * OR of GG_DEVERR_*).  The word is cleared by the next call on the
 * workspace. */
gg_status gg_device_error(const void* workspace, void* stream, int32_t* code);

/* ------------------------------------------------------------------------ */
/* Grouped wgrad                                                             */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace gg_wgrad needs for num_experts experts. */
size_t gg_wgrad_workspace_size(int32_t num_experts);

/*
 * Wgrad[e] = A[:, begin:end] @ B[begin:end, :] for every expert e, with
 * begin = 0 for e = 0, begin = offsets[e-1] otherwise, end = offsets[e]
 * ("Grouped GEMM + WGrad (Unified)", "Operation"); fp32 accumulation.
 *
 * a          A, logical shape (hidden, tokens_sum), bf16 ("BF16 contract"):
 *              a_major GG_MAJOR_K: element (h,t) at a[h*tokens_sum + t]
 *              a_major GG_MAJOR_M: element (h,t) at a[t*hidden + h]
 * b          B, logical shape (tokens_sum, intermediate), bf16:
 *              b_major GG_MAJOR_K: element (t,i) at b[i*tokens_sum + t]
 *              b_major GG_MAJOR_N: element (t,i) at b[t*intermediate + i]
 * offsets    int32[num_experts], non-decreasing cumulative token ends; every
 *            count a multiple of 256 and offsets[E-1] == tokens_sum ("BF16
 *            contract").  Counts that are multiples of 8 but not of 256 are
 *            computed exactly and flagged (GG_DEVERR_GRANULE); a group whose
 *            bounds are not multiples of 8 is skipped (GG_DEVERR_SKIPPED).
 * num_experts 1..1024.  tokens_sum >= 0, a multiple of 8.
 * hidden, intermediate  multiples of 64, >= 64; at most 2^28 output tiles
 *            of 256 x 256 over all experts (GG_ERR_UNSUPPORTED beyond).
 * Output, exactly one of ("Output modes"):
 * wgrad_dense  (num_experts, hidden, intermediate) row-major, or NULL;
 * wgrad_ptrs   int64[num_experts] device array of 16-B-aligned, non-NULL
 *              addresses, one (hidden, intermediate) row-major matrix per
 *              expert; or NULL.
 * wgrad_dtype  GG_BF16, GG_F16 or GG_F32.
 * accumulate   nonzero: out = round(old + result) (the caller initialises
 *              every output); zero: out = round(result), an empty expert
 *              gives exact zeros.  Rounding is to nearest even.
 * flags        OR of GG_FLAG_VALIDATE_OFFSETS, GG_FLAG_TENSOR_RAGGED
 *              ("input_order": the K-major operands' storage, see the flag)
 *              and GG_FLAG_STATIC_SCHED.
 * workspace    >= gg_wgrad_workspace_size(num_experts) bytes, 256-B aligned.
 *              Besides the error word and the experts' rank table it holds the
 *              work-queue counters of the kernel's scheduler, reset by every
 *              call; calls that may overlap must not share it.
 */
gg_status gg_wgrad(const void* a, gg_major a_major, const void* b, gg_major b_major,
                   const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                   int32_t hidden, int32_t intermediate,
                   void* wgrad_dense, const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype,
                   int32_t accumulate, uint32_t flags,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gg_wgrad without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Every argument has gg_wgrad's meaning;
 * the scratch the kernels use (error word, work-queue counters, expert
 * rank table) is a static array of 16640 bytes inside the library, one per
 * GPU, held until the process ends, which limits num_experts to 1024 (beyond:
 * GG_ERR_WORKSPACE; gg_wgrad's own limit is the same).  No path of the call
 * allocates memory, host or device.
 *   - All calls on one GPU share that GPU's scratch: calls that may overlap
 *     on one GPU (different streams, or host threads) race and must not be
 *     issued.  Each call clears what it needs before its kernels run.
 *   - The device error word lives in that scratch and is not readable by
 *     the caller; use GG_FLAG_VALIDATE_OFFSETS to have malformed offsets
 *     rejected (GG_ERR_OFFSETS), or gg_wgrad with a workspace to read it.
 */
gg_status gg_wgrad_noalloc(const void* a, gg_major a_major, const void* b, gg_major b_major,
                           const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                           int32_t hidden, int32_t intermediate,
                           void* wgrad_dense, const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype,
                           int32_t accumulate, uint32_t flags, void* stream);

/*
 * The same operation on block-scaled operands ("Grouped GEMM + WGrad
 * (Unified)", "Block-scaled contract"), MXFP8: E4M3 codes (E5M2 with
 * GG_FLAG_AB_E5M2) with one E8M0 scale per 32 consecutive tokens of a row,
 * deq(q, s) = fp8(q) * 2^(s-127), fp32 accumulation.  The reduction axis is
 * contiguous in both operands:
 * a_fp8      A (hidden, tokens_sum) K-major: (h,t) at a[h*tokens_sum + t];
 * sfa        (hidden, tokens_sum/32): sfa[h*(tokens_sum/32) + t/32];
 * b_fp8      B (tokens_sum, intermediate) stored K-major, as an
 *            (intermediate, tokens_sum) array: (t,i) at b[i*tokens_sum + t];
 * sfb        (intermediate, tokens_sum/32): sfb[i*(tokens_sum/32) + t/32].
 *            With GG_FLAG_TENSOR_RAGGED all four hold per-expert blocks
 *            instead: expert e's codes at a[hidden*begin + h*count + t-begin]
 *            and scales at sfa[(hidden*begin + h*count + t-begin)/32]
 *            (likewise b, sfb with intermediate).
 * tokens_sum a multiple of 128, as is every expert's count (the pages ask
 *            for 256; a count that is not a multiple of 128 is skipped and
 *            flagged GG_DEVERR_SKIPPED, one of 128 but not 256 computed and
 *            flagged GG_DEVERR_GRANULE).
 * flags      as for gg_wgrad, and GG_FLAG_AB_E5M2.
 * Codes 16-byte, scales 4-byte aligned.  Every other argument as for
 * gg_wgrad; the pages' global scales belong to formats other than MXFP8 and
 * are not taken.
 */
gg_status gg_wgrad_mx(const void* a_fp8, const uint8_t* sfa, const void* b_fp8, const uint8_t* sfb,
                      const int32_t* offsets, int32_t num_experts, int64_t tokens_sum,
                      int32_t hidden, int32_t intermediate,
                      void* wgrad_dense, const int64_t* wgrad_ptrs, gg_dtype wgrad_dtype,
                      int32_t accumulate, uint32_t flags,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped dgrad + dSwiGLU / dGeGLU                                          */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace gg_dglu needs for L experts and compact width n. */
size_t gg_dglu_workspace_size(int32_t L, int32_t n, int32_t generate_dbias);

/*
 * For the rows m of group g (po[g-1] <= m < po[g], po[-1] = 0) and compact
 * columns n ("Grouped GEMM + dGLU (SM100)", "BF16 contract"):
 *   R[m,n] = alpha_g^2 * sum_k A[m,k] B_g[n,k]          (fp32 accumulation)
 *   X = beta_g * C[m,:]  (one fp32 product per element)
 *   compact column n lies in block pair p = n/32 at j = n%32; its input
 *   column is 64p + j and its gate column 64p + 32 + j (GG_FLAG_GATE_FIRST
 *   swaps them).
 *   dSwiGLU, s = sigmoid(gate):
 *     D[input] = R prob gate s
 *     D[gate]  = R prob input s (1 + gate (1 - s))
 *     dprob   += R gate s input
 *   dGeGLU, gc = min(gate, clamp_max), uc = clamp(input, clamp_min,
 *   clamp_max), s = sigmoid(geglu_alpha gc), filters
 *   fg = gate if gate <= clamp_max else 0, fu = input if clamp_min <= input
 *   <= clamp_max else 0 (1 instead of the raw value with
 *   GG_FLAG_GEGLU_MASK_FILTER):
 *     D[gate]  = R prob (uc + linear_offset) s (1 + geglu_alpha gc (1 - s)) fg
 *     D[input] = R prob gc s fu
 *     dprob   += R gc s (uc + linear_offset)
 *   dbias[g, c] += sum over the group's rows of D[m, c] (before rounding).
 *
 * a          A (m_rows, k) bf16, K-major: a[m*k + kk].
 * m_rows     rows of A, C, D, prob, dprob; >= valid_m = padded_offsets[L-1].
 *            Rows at or past valid_m are neither read for output nor written.
 * k          reduction size, a multiple of 64, at most 2^21.
 * b_dense    dense weights, the pages' (N, K, L) tensor with strides
 *            (K, 1, N*K): expert g's (n, k) element at b[g*n*k + n*k + kk].
 * b_ptrs     or: int64[L] device array, expert g's (n, k) bf16 matrix at
 *            b_ptrs[g]; K-major (element at n*k + kk) when b_major is
 *            GG_MAJOR_K, N-major (element at kk*n + nn) when GG_MAJOR_N.
 *            Exactly one of b_dense / b_ptrs is non-NULL; b_dense requires
 *            GG_MAJOR_K.
 * n          compact gradient width N, a multiple of 32, at most 2^20
 *            (GG_ERR_UNSUPPORTED beyond either limit).
 * c          forward activation (m_rows, 2n), row-major, dtype c_dtype
 *            (GG_BF16, GG_F16 or GG_F32).
 * padded_offsets  int32[L] cumulative group ends, each group a multiple of
 *            256 (m_aligned).  L in 1..1024.
 * alpha, beta  float[L];  prob  float[m_rows].
 * d_row      output (m_rows, 2n), row-major, d_dtype (GG_BF16, GG_F16 or
 *            GG_F32), rounded to nearest even.
 * dprob      float[m_rows], caller-zeroed, accumulated into ("must be
 *            zero-initialized").
 * dbias      bf16 (L, 2n) row-major, caller-zeroed and accumulated into
 *            (one rounding of old + sum), or NULL for no dbias.
 * act        GG_DSWIGLU or GG_DGEGLU; geglu_alpha, clamp_min, clamp_max,
 *            linear_offset are the dGeGLU constants (the pages' defaults:
 *            1.702, -7, 7, 1); ignored for dSwiGLU.
 * flags      OR of GG_FLAG_GATE_FIRST, GG_FLAG_GEGLU_MASK_FILTER,
 *            GG_FLAG_VALIDATE_OFFSETS, GG_FLAG_STATIC_SCHED.
 * workspace  >= gg_dglu_workspace_size(L, n, dbias != NULL), 256-B aligned.
 */
gg_status gg_dglu(const void* a, int64_t m_rows, int32_t k,
                  const void* b_dense, const int64_t* b_ptrs, gg_major b_major, int32_t n,
                  const void* c, gg_dtype c_dtype,
                  const int32_t* padded_offsets, int32_t L,
                  const float* alpha, const float* beta, const float* prob,
                  void* d_row, gg_dtype d_dtype, float* dprob, void* dbias,
                  gg_act act, float geglu_alpha, float clamp_min, float clamp_max,
                  float linear_offset, uint32_t flags,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped dgrad + dSwiGLU / dGeGLU on MXFP8 operands                        */
/* ------------------------------------------------------------------------ */

/*
 * For the rows m of group g ("Grouped GEMM + dGLU (SM100)", "Block-scaled
 * contract / Equations"):
 *   R[m,n] = alpha_g^2 * sum_k deq(A[m,k]) deq(B_g[n,k])   (fp32 accumulation)
 * with deq(q, s) = e4m3(q) * 2^(s - 127), one E8M0 scale byte per 32
 * consecutive K values of a row (MXFP8: "sf_vec_size 32" in the page's
 * data-type table), followed by exactly the dSwiGLU / dGeGLU, dprob and dbias
 * steps documented for gg_dglu.  In addition ("Shapes": amax (L, 2, 1) for
 * a bf16 / fp16 D):
 *   amax[2g + 0] = max |D| over the group's input-gradient columns,
 *   amax[2g + 1] = max |D| over its gate-gradient columns,
 * taken before rounding (0 for an empty group).
 *
 * a_fp8      A (m_rows, k) FP8 codes (E4M3, or E5M2 with GG_FLAG_AB_E5M2),
 *            K-major: a[m*k + kk].
 * sfa        E8M0 scales (m_rows, k/32), row-major: sfa[m*(k/32) + kk/32]
 *            (a plain layout; the pages' MMA-interleaved scale layout is not
 *            used).
 * m_rows     as for gg_dglu.  k: a multiple of 128, at most 2^21.
 * b_fp8,sfb  dense weights (L, n, k) FP8 (A's format), element at
 *            b[g*n*k + nn*k + kk] (GG_MAJOR_K) or b[g*n*k + kk*n + nn]
 *            (GG_MAJOR_N), and scales (L, n, k/32) at
 *            sfb[(g*n + nn)*(k/32) + kk/32] for either major;
 * b_ptrs, sfb_ptrs  or: int64[L] device arrays of per-expert (n, k) codes
 *            and (n, k/32) scales with the same in-matrix layout (the page's
 *            discrete b_ptrs / sfb_ptrs).  Exactly one of the dense pair /
 *            the pointer pair is given.
 * b_major    GG_MAJOR_K or GG_MAJOR_N ("Parameters / Input tensor B (dense
 *            mode)": K-major or N-major), for dense and discrete B alike;
 *            else GG_ERR_LAYOUT.
 * n          compact width, a multiple of 32, at most 2^20
 *            (GG_ERR_UNSUPPORTED beyond either limit).
 * c_dtype    as for gg_dglu, or GG_F8E4M3 / GG_F8E5M2 (the dGLU page's
 *            "Input tensor C" dtypes): an FP8 C is read as its exact value.
 * c, padded_offsets, L, alpha, beta, prob, d_row, dprob, dbias, geglu_alpha,
 * clamp_min, clamp_max, linear_offset
 *            as for gg_dglu.
 * act        GG_DSWIGLU, GG_DGEGLU, or GG_DSITUGLU: the page's dSiTU-GLU
 *            ("Block-scaled contract / Equations") on gate G and input U of
 *            X = beta_g C, b1 = situ_beta1, b2 = situ_beta2 (the page's
 *            defaults: 4 and 25; both positive and finite, else
 *            GG_ERR_VALUE; ignored for the other activations):
 *              T_g = b1 tanh(G/b1) sigmoid(G),   T_u = b2 tanh(U/b2)
 *              D[gate]  = R prob T_u ((1 - tanh^2(G/b1)) sigmoid(G)
 *                         + b1 tanh(G/b1) sigmoid(G) (1 - sigmoid(G)))
 *              D[input] = R prob T_g (1 - tanh^2(U/b2))
 *              dprob   += R T_g T_u
 * amax       float[2L] ((L, 2) row-major), written by the call (the library
 *            clears it first), or NULL.
 * d_dtype    as for gg_dglu, or GG_F8E4M3 / GG_F8E5M2: d_row then holds
 *            the row-quantized FP8 D ((m_rows, 2n), 16-B aligned) and
 *            fp8_out [host] the rest of the FP8 output (see gg_fp8_out);
 *            fp8_out is ignored for the other dtypes.
 * flags      as for gg_dglu, and GG_FLAG_AB_E5M2 (with an FP8 d_dtype).
 * workspace  >= gg_dglu_workspace_size(L, n, dbias != NULL), 256-B aligned.
 */
gg_status gg_dglu_mx(const void* a_fp8, const uint8_t* sfa, int64_t m_rows, int32_t k,
                     const void* b_fp8, const uint8_t* sfb,
                     const int64_t* b_ptrs, const int64_t* sfb_ptrs, gg_major b_major, int32_t n,
                     const void* c, gg_dtype c_dtype,
                     const int32_t* padded_offsets, int32_t L,
                     const float* alpha, const float* beta, const float* prob,
                     void* d_row, gg_dtype d_dtype, float* dprob, void* dbias, float* amax,
                     const gg_fp8_out* fp8_out, gg_act act, float geglu_alpha, float clamp_min, float clamp_max,
                     float linear_offset, float situ_beta1, float situ_beta2, uint32_t flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped dgrad + dsReLU on MXFP8 operands                                  */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace gg_dsrelu needs for L experts. */
size_t gg_dsrelu_workspace_size(int32_t L);

/*
 * For the rows m of group g ("Grouped GEMM + dsReLU (SM100)", "Equations"):
 *   G[m,n]     = alpha_g * sum_k deq(A[m,k]) deq(B_g[n,k])   (fp32 accumulation)
 *   D_row[m,n] = prob[m] * 2 * C[m,n] * relu(G[m,n])
 *   dprob[m]  += sum_n C[m,n] * relu(G[m,n])^2
 *   amax[g]    = max |D_row| over the group, before rounding (0 if empty)
 * with deq(q, s) = fp8(q) * 2^(s - 127): MXFP8, one E8M0 scale byte per 32
 * consecutive K values of a row ("sf_vec_size 32" for MXFP8 on the dGLU
 * page's data-type table), the codes E4M3, or E5M2 with GG_FLAG_AB_E5M2 (A
 * and B alike).
 *
 * a_fp8      A (m_rows, k) FP8 codes, K-major: a[m*k + kk].
 * sfa        E8M0 scales (m_rows, k/32), row-major: sfa[m*(k/32) + kk/32].
 *            (A plain row-major layout; the pages' 6-D MMA-interleaved scale
 *            layout is not used.)
 * m_rows     as for gg_dglu.  k: a multiple of 128, at most 2^21.
 * b_fp8,sfb  dense weights (L, n, k) FP8 (A's format), element at
 *            b[g*n*k + nn*k + kk] (GG_MAJOR_K) or b[g*n*k + kk*n + nn]
 *            (GG_MAJOR_N), and scales (L, n, k/32) at
 *            sfb[(g*n + nn)*(k/32) + kk/32] for either major;
 * b_ptrs, sfb_ptrs  or: int64[L] device arrays of per-expert (n, k) codes
 *            and (n, k/32) scales with the same in-matrix layout.
 *            Exactly one of the dense pair / the pointer pair is given.
 * b_major    GG_MAJOR_K or GG_MAJOR_N (the page's "Layouts" allow an
 *            N-major B for FP8 operands), else GG_ERR_LAYOUT.
 * n          a multiple of 32, at most 2^21 (GG_ERR_UNSUPPORTED beyond either
 *            limit).
 * c          (m_rows, n) row-major, c_dtype GG_BF16, GG_F16, GG_F32,
 *            GG_F8E4M3 or GG_F8E5M2 (the dsReLU page's "Input tensor C"
 *            dtypes; an FP8 C is read as its exact value).
 * padded_offsets, L  as for gg_dglu.
 * alpha      float[L];  prob  float[m_rows].
 * d_row      (m_rows, n) row-major, d_dtype GG_BF16, GG_F16 or GG_F32; or
 *            GG_F8E4M3 / GG_F8E5M2, the row-quantized D, with fp8_out [host]
 *            giving the rest of the FP8 output (see gg_fp8_out; ignored
 *            otherwise).
 * dprob      float[m_rows], caller-zeroed, accumulated into.
 * amax       float[L], written by the call (the library clears it first), or
 *            NULL.
 * flags      OR of GG_FLAG_VALIDATE_OFFSETS, GG_FLAG_STATIC_SCHED and
 *            GG_FLAG_AB_E5M2 (with an FP8 d_dtype).
 * workspace  >= gg_dsrelu_workspace_size(L), 256-B aligned.
 */
gg_status gg_dsrelu(const void* a_fp8, const uint8_t* sfa, int64_t m_rows, int32_t k,
                    const void* b_fp8, const uint8_t* sfb,
                    const int64_t* b_ptrs, const int64_t* sfb_ptrs, gg_major b_major, int32_t n,
                    const void* c, gg_dtype c_dtype,
                    const int32_t* padded_offsets, int32_t L,
                    const float* alpha, const float* prob,
                    void* d_row, gg_dtype d_dtype, float* dprob, float* amax,
                    const gg_fp8_out* fp8_out, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GG_MOE_H */
