"""CPU oracle for the grouped GEMMs of the MoE expert backward pass.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg call this module; the HIP product path never does, and the two
share no code.  The arithmetic lives in gg_oracle.c (plain loops, double
accumulation, exact decoding, one round-to-nearest-even at the end); this file
marshals numpy arrays and applies the pages' output rules:

* "Grouped GEMM + WGrad (Unified)", section "Operation": accumulate adds the
  result to the existing output, overwrite replaces it, an empty expert
  produces zero.
* "Grouped GEMM + dGLU (SM100)", "BF16 contract": dprob and dbias are
  caller-zeroed and accumulated into; dbias is BF16.
* "Grouped GEMM + dsReLU (SM100)", "Equations" and "Shapes": dprob is the row
  sum, Amax is per expert (shape (L, 1)).

All raw operands are numpy arrays of bit patterns: uint16 for bf16/fp16,
uint8 for FP8 (E4M3 or E5M2) codes and e8m0 scales, float32 for fp32.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16, F16, F32, E4M3, E5M2 = 0, 1, 2, 3, 4
_DT_NP = {BF16: np.uint16, F16: np.uint16, F32: np.float32, E4M3: np.uint8, E5M2: np.uint8}


def _fmt(fp8_dtype):
    """The C file's FP8 format index: 0 for E4M3, 1 for E5M2."""
    assert fp8_dtype in (E4M3, E5M2), fp8_dtype
    return fp8_dtype - E4M3

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        F = ctypes.c_float
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = D
        L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_double.restype = D
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_double.restype = D
        L.orc_e5m2_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_to_double.restype = D
        L.orc_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_double.restype = D
        L.orc_double_to_bf16.argtypes = [D]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_double_to_f16.argtypes = [D]
        L.orc_double_to_f16.restype = ctypes.c_uint16
        L.orc_double_to_f32.argtypes = [D]
        L.orc_double_to_f32.restype = F
        L.orc_round_array.argtypes = [P, I64, I, P]
        L.orc_round_array.restype = None
        L.orc_wgrad.argtypes = [P, I, P, I, P, I, I64, I, I, P, I, P]
        L.orc_wgrad.restype = None
        L.orc_wgrad_finish.argtypes = [P, I64, I, P, I, P]
        L.orc_wgrad_mx.argtypes = [P, P, P, P, I, P, I, I64, I, I, P, I, P]
        L.orc_double_to_e4m3.argtypes = [D]
        L.orc_double_to_e4m3.restype = ctypes.c_uint8
        L.orc_double_to_e5m2.argtypes = [D]
        L.orc_double_to_e5m2.restype = ctypes.c_uint8
        L.orc_quant_fp8.argtypes = [P, I64, I, ctypes.c_float, I, P, P, P, P]
        L.orc_quant_fp8.restype = None
        L.orc_wgrad_mx.restype = None
        L.orc_wgrad_finish.restype = None
        L.orc_dglu.argtypes = [P, I64, I, P, I, I, P, I, P, I, P, P, P,
                               I, D, D, D, D, I, I, P, I64, P, P, P]
        L.orc_dglu.restype = None
        L.orc_dsrelu.argtypes = [P, P, I64, I, P, P, I, I, P, I, P, I, P, P,
                                 P, I64, P, P, P]
        L.orc_dsrelu.restype = None
        L.orc_dglu_mx.argtypes = [P, P, I64, I, P, P, I, I, P, I, P, I, P, P, P,
                                  I, D, D, D, D, D, D, I, I, P, I64, P, P, P, P]
        L.orc_dglu_mx.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = I
        L.orc_set_threads.argtypes = [I]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def num_threads():
    """Threads the oracle's OpenMP loops use."""
    return lib().orc_num_threads()


def set_threads(n):
    """Sets the threads of the oracle's OpenMP loops (n >= 1)."""
    lib().orc_set_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar codecs (exposed so that the tests can pin them)
# --------------------------------------------------------------------------

def decode(bits, dtype):
    """Exact values (float64) of an array of bf16/fp16 bit patterns or fp32."""
    bits = np.asarray(bits)
    f = {BF16: lib().orc_bf16_to_double, F16: lib().orc_f16_to_double}.get(dtype)
    if f is None:
        return bits.astype(np.float64)
    return np.array([f(int(b)) for b in bits.ravel()], np.float64).reshape(bits.shape)


def decode_e4m3(codes):
    codes = np.asarray(codes)
    return np.array([lib().orc_e4m3_to_double(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


def decode_e5m2(codes):
    codes = np.asarray(codes)
    return np.array([lib().orc_e5m2_to_double(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


def decode_e8m0(codes):
    codes = np.asarray(codes)
    return np.array([lib().orc_e8m0_to_double(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


def round_to(x, dtype):
    """Round float64 values once, to nearest even, into dtype's bit patterns
    (uint16 for bf16/fp16, float32 for fp32)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, _DT_NP[dtype])
    lib().orc_round_array(_p(x), x.size, dtype, _p(out))
    return out


def encode_e4m3(x):
    """OCP E4M3 codes (uint8) of float64 values, RNE, magnitudes clamped to 448."""
    x = np.asarray(x, np.float64).ravel()
    return np.array([lib().orc_double_to_e4m3(float(v)) for v in x], np.uint8)


def encode_e5m2(x):
    """OCP E5M2 codes (uint8) of float64 values, RNE, magnitudes clamped to 57344."""
    x = np.asarray(x, np.float64).ravel()
    return np.array([lib().orc_double_to_e5m2(float(v)) for v in x], np.uint8)


def quant_fp8(D, norm_const, with_col=True, d_dtype=E4M3):
    """Step 3 of the block-scaled dGLU contract (and the FP8 outputs of the
    dsReLU page) on a float64 (nrows, W) D: row-quantized codes (E4M3, or
    E5M2 with d_dtype=E5M2) and E8M0 scales per 32 columns, and (with_col,
    nrows a multiple of 32) the column-quantized codes with scales per 32
    rows, laid out (W, nrows/32)."""
    D = np.ascontiguousarray(D, np.float64)
    nrows, W = D.shape
    q_row = np.zeros((nrows, W), np.uint8)
    sfd_row = np.zeros((nrows, W // 32), np.uint8)
    q_col = np.zeros((nrows, W), np.uint8) if with_col else None
    sfd_col = np.zeros((W, nrows // 32), np.uint8) if with_col else None
    lib().orc_quant_fp8(_p(D), nrows, W, float(norm_const), _fmt(d_dtype), _p(q_row),
                        _p(sfd_row), _p(q_col), _p(sfd_col))
    return {"q_row": q_row, "sfd_row": sfd_row, "q_col": q_col, "sfd_col": sfd_col}


# --------------------------------------------------------------------------
# grouped wgrad
# --------------------------------------------------------------------------

def wgrad(a, a_major, b, b_major, offsets, hidden, inter, tokens_sum,
          out_dtype=F32, accumulate=False, old=None, hrows=None):
    """Wgrad[e] = A[:, begin:end] @ B[begin:end, :] for every expert e.

    a: flat uint16 bf16 bits of A (hidden, tokens_sum); a_major 0 = K-major
    ((h,t) at h*T+t), 1 = M-major ((h,t) at t*hidden+h).
    b: flat uint16 bf16 bits of B (tokens_sum, inter); b_major 0 = K-major
    ((t,i) at i*T+t), 1 = N-major ((t,i) at t*inter+i).
    old: the existing output (E, hidden, inter) in out_dtype's bit patterns,
    required when accumulating.
    hrows: optional list of hidden rows to compute (every row when None).
    Returns (exact, result): exact is the float64 result of the product
    (plus the old value when accumulating), result the rounded output of
    shape (E, nrows, inter)."""
    offsets = _c(offsets, np.int32)
    E = offsets.size
    a = _c(a, np.uint16).ravel()
    b = _c(b, np.uint16).ravel()
    assert a.size == hidden * tokens_sum and b.size == tokens_sum * inter
    hr = None if hrows is None else _c(hrows, np.int32)
    nrows = hidden if hr is None else hr.size
    prod = np.zeros((E, nrows, inter), np.float64)
    lib().orc_wgrad(_p(a), a_major, _p(b), b_major, _p(offsets), E, tokens_sum,
                    hidden, inter, _p(hr), nrows, _p(prod))
    if accumulate:
        old = _c(old, _DT_NP[out_dtype])
        if hr is not None:
            old = np.ascontiguousarray(old[:, hr, :])
        assert old.shape == prod.shape
    else:
        old = np.zeros(prod.shape, _DT_NP[out_dtype])
    res = np.empty(prod.shape, _DT_NP[out_dtype])
    lib().orc_wgrad_finish(_p(prod), prod.size, int(bool(accumulate)), _p(old),
                           out_dtype, _p(res))
    exact = prod + (decode_array(old, out_dtype) if accumulate else 0.0)
    return exact, res


def wgrad_mx(a, sfa, b, sfb, offsets, hidden, inter, tokens_sum, out_dtype=F32,
             accumulate=False, old=None, hrows=None, ab_dtype=E4M3):
    """Block-scaled (MXFP8) Wgrad[e] = deq(A)[:, begin:end] @ deq(B)[begin:end, :].

    a: uint8 FP8 codes (E4M3, or E5M2 with ab_dtype=E5M2; B alike) of A
    (hidden, tokens_sum), K-major; sfa: uint8 E8M0
    (hidden, tokens_sum/32).  b: codes of B stored K-major, i.e. an
    (inter, tokens_sum) array; sfb: (inter, tokens_sum/32).  Other arguments
    and the return value as for wgrad."""
    offsets = _c(offsets, np.int32)
    E = offsets.size
    a, sfa = _c(a, np.uint8).ravel(), _c(sfa, np.uint8).ravel()
    b, sfb = _c(b, np.uint8).ravel(), _c(sfb, np.uint8).ravel()
    assert a.size == hidden * tokens_sum and b.size == tokens_sum * inter
    assert sfa.size == hidden * (tokens_sum // 32) and sfb.size == inter * (tokens_sum // 32)
    hr = None if hrows is None else _c(hrows, np.int32)
    nrows = hidden if hr is None else hr.size
    prod = np.zeros((E, nrows, inter), np.float64)
    lib().orc_wgrad_mx(_p(a), _p(sfa), _p(b), _p(sfb), _fmt(ab_dtype), _p(offsets), E, tokens_sum,
                       hidden, inter, _p(hr), nrows, _p(prod))
    if accumulate:
        old = _c(old, _DT_NP[out_dtype])
        if hr is not None:
            old = np.ascontiguousarray(old[:, hr, :])
        assert old.shape == prod.shape
    else:
        old = np.zeros(prod.shape, _DT_NP[out_dtype])
    res = np.empty(prod.shape, _DT_NP[out_dtype])
    lib().orc_wgrad_finish(_p(prod), prod.size, int(bool(accumulate)), _p(old),
                           out_dtype, _p(res))
    exact = prod + (decode_array(old, out_dtype) if accumulate else 0.0)
    return exact, res


def decode_array(bits, dtype):
    """Vectorised exact decode of bf16/fp16 bit patterns (or fp32) to float64."""
    bits = np.asarray(bits)
    if dtype == F32:
        return bits.astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# grouped dgrad + dGLU
# --------------------------------------------------------------------------

DSWIGLU, DGEGLU, DSITUGLU = 0, 1, 2   # dSiTU-GLU: block-scaled only


def dglu(a, m_rows, k, b_list, b_major, n, c, c_dtype, padded_offsets,
         alpha, beta, prob, act=DSWIGLU, geglu_alpha=1.702, clamp_min=-7.0,
         clamp_max=7.0, linear_offset=1.0, gate_first=False, mask_filter=False,
         d_dtype=BF16, dprob_in=None, dbias_in=None, rows=None):
    """Grouped dgrad fused with dSwiGLU / dGeGLU.

    a: uint16 bf16 bits (m_rows, k); b_list: L arrays of uint16 bf16 bits
    (one (n, k) matrix per expert, K-major when b_major is 0, N-major
    ((n,k) at k*n_dim+n) when 1); c: (m_rows, 2n) in c_dtype bits.
    Returns a dict with D (float64, listed rows), D_q (rounded), dprob
    (float64: dprob_in + row sum), and, when dbias_in is given, dbias
    (float64: dbias_in + column sums) and dbias_q (bf16 bits)."""
    assert act in (DSWIGLU, DGEGLU), "dSiTU-GLU is defined for the block-scaled contract only"
    po = _c(padded_offsets, np.int32)
    L = po.size
    a = _c(a, np.uint16).ravel()
    bl = [_c(x, np.uint16).ravel() for x in b_list]
    assert len(bl) == L
    bptr = (ctypes.c_void_p * L)(*[x.ctypes.data for x in bl])
    c = _c(c, _DT_NP[c_dtype]).ravel()
    rr = None if rows is None else _c(rows, np.int64)
    nrows = m_rows if rr is None else rr.size
    D = np.zeros((nrows, 2 * n), np.float64)
    dps = np.zeros(nrows, np.float64)
    want_bias = dbias_in is not None
    dbs = np.zeros((L, 2 * n), np.float64) if want_bias else None
    lib().orc_dglu(_p(a), m_rows, k, ctypes.cast(bptr, ctypes.c_void_p), b_major, n,
                   _p(c), c_dtype, _p(po), L, _p(_c(alpha, np.float32)),
                   _p(_c(beta, np.float32)), _p(_c(prob, np.float32)),
                   act, geglu_alpha, clamp_min, clamp_max, linear_offset,
                   int(bool(gate_first)), int(bool(mask_filter)),
                   _p(rr), nrows, _p(D), _p(dps), _p(dbs))
    valid = _valid_rows(po, m_rows, rr)
    out = {"D": D, "D_q": round_to(D, d_dtype), "valid": valid}
    dp_in = np.zeros(m_rows, np.float32) if dprob_in is None else np.asarray(dprob_in, np.float32)
    dp_in = dp_in if rr is None else dp_in[rr]
    out["dprob"] = dp_in.astype(np.float64) + dps
    if want_bias:
        out["dbias"] = decode_array(_c(dbias_in, np.uint16), BF16).reshape(L, 2 * n) + dbs
        out["dbias_q"] = round_to(out["dbias"], BF16)
    return out


def _valid_rows(po, m_rows, rr):
    valid_m = int(po[-1]) if po.size else 0
    idx = np.arange(m_rows) if rr is None else rr
    return idx < valid_m


# --------------------------------------------------------------------------
# block-scaled grouped dgrad + dGLU (MXFP8)
# --------------------------------------------------------------------------

def dglu_mx(a, sfa, m_rows, k, b_list, sfb_list, n, c, c_dtype, padded_offsets,
            alpha, beta, prob, act=DSWIGLU, geglu_alpha=1.702, clamp_min=-7.0,
            clamp_max=7.0, linear_offset=1.0, situ_beta1=4.0, situ_beta2=25.0,
            gate_first=False, mask_filter=False, d_dtype=BF16, dprob_in=None,
            dbias_in=None, rows=None, ab_dtype=E4M3):
    """Block-scaled (MXFP8) grouped dgrad fused with dSwiGLU / dGeGLU /
    dSiTU-GLU (act DSITUGLU, tanh scales situ_beta1 and situ_beta2).

    a: uint8 FP8 codes (E4M3, or E5M2 with ab_dtype=E5M2; B alike)
    (m_rows, k); sfa: uint8 e8m0 (m_rows, k/32);
    b_list / sfb_list: per expert K-major (n, k) codes and (n, k/32) scales;
    c: (m_rows, 2n) in c_dtype bits.  Returns what dglu returns, plus amax
    (float64 (L, 2): max |D| of the input-gradient and the gate-gradient
    columns of each expert's listed rows, from 0)."""
    po = _c(padded_offsets, np.int32)
    L = po.size
    a = _c(a, np.uint8).ravel()
    sfa = _c(sfa, np.uint8).ravel()
    bl = [_c(x, np.uint8).ravel() for x in b_list]
    sl = [_c(x, np.uint8).ravel() for x in sfb_list]
    assert len(bl) == L and len(sl) == L
    bptr = (ctypes.c_void_p * L)(*[x.ctypes.data for x in bl])
    sptr = (ctypes.c_void_p * L)(*[x.ctypes.data for x in sl])
    c = _c(c, _DT_NP[c_dtype]).ravel()
    rr = None if rows is None else _c(rows, np.int64)
    nrows = m_rows if rr is None else rr.size
    D = np.zeros((nrows, 2 * n), np.float64)
    dps = np.zeros(nrows, np.float64)
    want_bias = dbias_in is not None
    dbs = np.zeros((L, 2 * n), np.float64) if want_bias else None
    amax = np.zeros((L, 2), np.float64)
    lib().orc_dglu_mx(_p(a), _p(sfa), m_rows, k, ctypes.cast(bptr, ctypes.c_void_p),
                      ctypes.cast(sptr, ctypes.c_void_p), n, _fmt(ab_dtype), _p(c), c_dtype,
                      _p(po), L, _p(_c(alpha, np.float32)), _p(_c(beta, np.float32)),
                      _p(_c(prob, np.float32)), act, geglu_alpha, clamp_min, clamp_max,
                      linear_offset, situ_beta1, situ_beta2, int(bool(gate_first)),
                      int(bool(mask_filter)),
                      _p(rr), nrows, _p(D), _p(dps), _p(dbs), _p(amax))
    valid = _valid_rows(po, m_rows, rr)
    out = {"D": D, "D_q": round_to(D, d_dtype) if d_dtype in (BF16, F16, F32) else None,
           "valid": valid, "amax": amax}
    dp_in = np.zeros(m_rows, np.float32) if dprob_in is None else np.asarray(dprob_in, np.float32)
    dp_in = dp_in if rr is None else dp_in[rr]
    out["dprob"] = dp_in.astype(np.float64) + dps
    if want_bias:
        out["dbias"] = decode_array(_c(dbias_in, np.uint16), BF16).reshape(L, 2 * n) + dbs
        out["dbias_q"] = round_to(out["dbias"], BF16)
    return out


# --------------------------------------------------------------------------
# grouped dgrad + dsReLU (MXFP8)
# --------------------------------------------------------------------------

def dsrelu(a, sfa, m_rows, k, b_list, sfb_list, n, c, c_dtype,
           padded_offsets, alpha, prob, d_dtype=BF16, dprob_in=None, rows=None, ab_dtype=E4M3):
    """Grouped block-scaled dgrad fused with dsReLU.

    a: uint8 FP8 codes (E4M3, or E5M2 with ab_dtype=E5M2; B alike)
    (m_rows, k); sfa: uint8 e8m0 (m_rows, k/32);
    b_list / sfb_list: per expert (n, k) codes and (n, k/32) scales;
    c: (m_rows, n) in c_dtype bits.
    Returns a dict with D (float64), D_q (rounded), dprob (float64:
    dprob_in + row sum) and amax (float64, per expert, from 0)."""
    po = _c(padded_offsets, np.int32)
    L = po.size
    a = _c(a, np.uint8).ravel()
    sfa = _c(sfa, np.uint8).ravel()
    bl = [_c(x, np.uint8).ravel() for x in b_list]
    sl = [_c(x, np.uint8).ravel() for x in sfb_list]
    bptr = (ctypes.c_void_p * L)(*[x.ctypes.data for x in bl])
    sptr = (ctypes.c_void_p * L)(*[x.ctypes.data for x in sl])
    c = _c(c, _DT_NP[c_dtype]).ravel()
    rr = None if rows is None else _c(rows, np.int64)
    nrows = m_rows if rr is None else rr.size
    D = np.zeros((nrows, n), np.float64)
    dps = np.zeros(nrows, np.float64)
    amax = np.zeros(L, np.float64)
    lib().orc_dsrelu(_p(a), _p(sfa), m_rows, k, ctypes.cast(bptr, ctypes.c_void_p),
                     ctypes.cast(sptr, ctypes.c_void_p), n, _fmt(ab_dtype), _p(c), c_dtype,
                     _p(po), L, _p(_c(alpha, np.float32)), _p(_c(prob, np.float32)),
                     _p(rr), nrows, _p(D), _p(dps), _p(amax))
    out = {"D": D, "D_q": round_to(D, d_dtype) if d_dtype in (BF16, F16, F32) else None,
           "amax": amax,
           "valid": _valid_rows(po, m_rows, rr)}
    dp_in = np.zeros(m_rows, np.float32) if dprob_in is None else np.asarray(dprob_in, np.float32)
    dp_in = dp_in if rr is None else dp_in[rr]
    out["dprob"] = dp_in.astype(np.float64) + dps
    return out
