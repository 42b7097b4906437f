"""ctypes binding of libgg_moe (include/gg_moe.h) -- argument marshalling only.

Each function takes torch tensors (device memory allocated by PyTorch) or
raw integers for pointers, converts them to the C arguments, calls the C
entry point of the same name and raises GGError on a non-GG_OK status.
Every step of the computation runs in the library's HIP kernels; if the
library has not been built, loading it raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgg_moe.so")

# enums of gg_moe.h
GG_BF16, GG_F16, GG_F32, GG_F8E4M3, GG_F8E5M2 = 0, 1, 2, 3, 4
GG_MAJOR_K, GG_MAJOR_M, GG_MAJOR_N = 0, 1, 2
GG_DSWIGLU, GG_DGEGLU, GG_DSITUGLU = 0, 1, 2
GG_FLAG_GATE_FIRST, GG_FLAG_GEGLU_MASK_FILTER, GG_FLAG_VALIDATE_OFFSETS = 1, 2, 4
GG_FLAG_TENSOR_RAGGED, GG_FLAG_STATIC_SCHED, GG_FLAG_AB_E5M2 = 8, 16, 32
GG_DEVERR_DECREASING, GG_DEVERR_GRANULE, GG_DEVERR_LAST, GG_DEVERR_SKIPPED = 1, 2, 4, 8
STATUS_NAMES = ["GG_OK", "GG_ERR_NULL", "GG_ERR_SHAPE", "GG_ERR_DTYPE", "GG_ERR_LAYOUT",
                "GG_ERR_ALIGN", "GG_ERR_MODE", "GG_ERR_WORKSPACE", "GG_ERR_UNSUPPORTED",
                "GG_ERR_DEVICE", "GG_ERR_HIP", "GG_ERR_OFFSETS", "GG_ERR_VALUE"]
EXPORTS = ["gg_abi_version", "gg_last_error", "gg_device_error", "gg_wgrad_workspace_size",
           "gg_wgrad", "gg_wgrad_noalloc", "gg_wgrad_mx", "gg_dglu_workspace_size", "gg_dglu", "gg_dglu_mx",
           "gg_dsrelu_workspace_size", "gg_dsrelu"]

_TORCH_DTYPE = {torch.bfloat16: GG_BF16, torch.float16: GG_F16, torch.float32: GG_F32,
                torch.float8_e4m3fn: GG_F8E4M3, torch.float8_e5m2: GG_F8E5M2}


class GGError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


_lib = None


def load_library(path=LIB_PATH):
    """Load libgg_moe.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           "python moe_grouped_gemm_offset_amd/build.py")
    L = ctypes.CDLL(path)
    P, I32, I64, U32, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float)
    L.gg_abi_version.restype = ctypes.c_int
    L.gg_abi_version.argtypes = []
    L.gg_last_error.restype = ctypes.c_char_p
    L.gg_last_error.argtypes = []
    L.gg_device_error.restype = ctypes.c_int
    L.gg_device_error.argtypes = [P, P, ctypes.POINTER(I32)]
    L.gg_wgrad_workspace_size.restype = SZ
    L.gg_wgrad_workspace_size.argtypes = [I32]
    L.gg_dglu_workspace_size.restype = SZ
    L.gg_dglu_workspace_size.argtypes = [I32, I32, I32]
    L.gg_dsrelu_workspace_size.restype = SZ
    L.gg_dsrelu_workspace_size.argtypes = [I32]
    L.gg_wgrad.restype = ctypes.c_int
    L.gg_wgrad.argtypes = [P, I32, P, I32, P, I32, I64, I32, I32, P, P, I32, I32, U32, P, SZ, P]
    L.gg_wgrad_noalloc.restype = ctypes.c_int
    L.gg_wgrad_noalloc.argtypes = [P, I32, P, I32, P, I32, I64, I32, I32, P, P, I32, I32, U32, P]
    L.gg_wgrad_mx.restype = ctypes.c_int
    L.gg_wgrad_mx.argtypes = [P, P, P, P, P, I32, I64, I32, I32, P, P, I32, I32, U32, P, SZ, P]
    L.gg_dglu.restype = ctypes.c_int
    L.gg_dglu.argtypes = [P, I64, I32, P, P, I32, I32, P, I32, P, I32, P, P, P, P, I32, P, P,
                          I32, F, F, F, F, U32, P, SZ, P]
    L.gg_dglu_mx.restype = ctypes.c_int
    L.gg_dglu_mx.argtypes = [P, P, I64, I32, P, P, P, P, I32, I32, P, I32, P, I32, P, P, P, P, I32, P,
                             P, P, P, I32, F, F, F, F, F, F, U32, P, SZ, P]
    L.gg_dsrelu.restype = ctypes.c_int
    L.gg_dsrelu.argtypes = [P, P, I64, I32, P, P, P, P, I32, I32, P, I32, P, I32, P, P, P, I32, P, P,
                            P, U32, P, SZ, P]
    _lib = L
    return L


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Fp8Out(ctypes.Structure):
    """gg_fp8_out of gg_moe.h (device pointers)."""
    _fields_ = [("d_col", ctypes.c_void_p), ("sfd_row", ctypes.c_void_p),
                ("sfd_col", ctypes.c_void_p), ("norm_const", ctypes.c_void_p)]


def _fp8_out(f):
    """A dict of tensors (sfd_row, norm_const and optionally d_col, sfd_col)
    as a gg_fp8_out, or None."""
    if f is None:
        return None
    return Fp8Out(_ptr(f.get("d_col")), _ptr(f.get("sfd_row")), _ptr(f.get("sfd_col")),
                  _ptr(f.get("norm_const")))


def _ref(s):
    return None if s is None else ctypes.addressof(s)


def _check(status):
    if status != 0:
        raise GGError(status, gg_last_error())


def gg_abi_version():
    return load_library().gg_abi_version()


def gg_last_error():
    return load_library().gg_last_error().decode()


def gg_wgrad_workspace_size(num_experts):
    return load_library().gg_wgrad_workspace_size(num_experts)


def gg_dglu_workspace_size(L, n, generate_dbias):
    return load_library().gg_dglu_workspace_size(L, n, int(bool(generate_dbias)))


def gg_dsrelu_workspace_size(L):
    return load_library().gg_dsrelu_workspace_size(L)


def _torch_stream(stream):
    """The torch stream object of a call's stream argument (None: the current
    stream; an int: the raw hipStream_t)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _workspace(ws, nbytes, like, stream):
    """The caller's workspace, or a new one allocated on the stream the call
    runs on: torch's caching allocator ties a freed block to the stream it
    was allocated on, so a workspace the caller drops is not handed to work
    on another stream while this call's kernels may still use it."""
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    with torch.cuda.stream(_torch_stream(stream)):
        t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=like.device)
    return t, t.numel()


def _ab(a, flags):
    """Operand codes given as a float8_e5m2 tensor add GG_FLAG_AB_E5M2 (uint8
    or float8_e4m3fn codes leave flags as they are)."""
    return flags | GG_FLAG_AB_E5M2 if a is not None and a.dtype == torch.float8_e5m2 else flags


def _sched(flags):
    """GG_SCHED=static in the environment adds GG_FLAG_STATIC_SCHED (a
    benchmarking override; GG_SCHED=dynamic or unset leaves flags alone)."""
    return flags | GG_FLAG_STATIC_SCHED if os.environ.get("GG_SCHED") == "static" else flags


def gg_device_error(workspace, stream=None):
    code = ctypes.c_int32(0)
    _check(load_library().gg_device_error(_ptr(workspace), _stream(stream), ctypes.byref(code)))
    return code.value


def gg_wgrad(a, a_major, b, b_major, offsets, tokens_sum, hidden, intermediate,
             wgrad_dense=None, wgrad_ptrs=None, wgrad_dtype=None, accumulate=False, flags=0,
             workspace=None, stream=None):
    """Grouped wgrad (gg_wgrad of gg_moe.h).  a_major: GG_MAJOR_K/GG_MAJOR_M,
    b_major: GG_MAJOR_K/GG_MAJOR_N.  Returns the workspace used."""
    L = load_library()
    E = offsets.numel()
    if wgrad_dtype is None:
        wgrad_dtype = _TORCH_DTYPE[wgrad_dense.dtype]
    ws, nbytes = _workspace(workspace, L.gg_wgrad_workspace_size(E), offsets, stream)
    _check(L.gg_wgrad(_ptr(a), a_major, _ptr(b), b_major, _ptr(offsets), E, tokens_sum, hidden,
                      intermediate, _ptr(wgrad_dense), _ptr(wgrad_ptrs), wgrad_dtype,
                      int(bool(accumulate)), _sched(flags), _ptr(ws), nbytes, _stream(stream)))
    return ws


def gg_wgrad_noalloc(a, a_major, b, b_major, offsets, tokens_sum, hidden, intermediate,
                     wgrad_dense=None, wgrad_ptrs=None, wgrad_dtype=None, accumulate=False, flags=0,
                     stream=None):
    """Grouped wgrad on the library's static scratch (gg_wgrad_noalloc of
    gg_moe.h): no workspace is allocated or passed."""
    L = load_library()
    E = offsets.numel()
    if wgrad_dtype is None:
        wgrad_dtype = _TORCH_DTYPE[wgrad_dense.dtype]
    _check(L.gg_wgrad_noalloc(_ptr(a), a_major, _ptr(b), b_major, _ptr(offsets), E, tokens_sum, hidden,
                              intermediate, _ptr(wgrad_dense), _ptr(wgrad_ptrs), wgrad_dtype,
                              int(bool(accumulate)), _sched(flags), _stream(stream)))


def gg_wgrad_mx(a, sfa, b, sfb, offsets, tokens_sum, hidden, intermediate, wgrad_dense=None,
                wgrad_ptrs=None, wgrad_dtype=None, accumulate=False, flags=0, workspace=None,
                stream=None):
    """Grouped MXFP8 wgrad (gg_wgrad_mx of gg_moe.h): FP8 codes (uint8 /
    float8_e4m3fn tensors: E4M3; float8_e5m2 tensors or GG_FLAG_AB_E5M2:
    E5M2) and E8M0 scales, both operands K-major.  Returns the workspace
    used."""
    L = load_library()
    E = offsets.numel()
    if wgrad_dtype is None:
        wgrad_dtype = _TORCH_DTYPE[wgrad_dense.dtype]
    ws, nbytes = _workspace(workspace, L.gg_wgrad_workspace_size(E), offsets, stream)
    _check(L.gg_wgrad_mx(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(offsets), E, tokens_sum,
                         hidden, intermediate, _ptr(wgrad_dense), _ptr(wgrad_ptrs), wgrad_dtype,
                         int(bool(accumulate)), _sched(_ab(a, flags)), _ptr(ws), nbytes,
                         _stream(stream)))
    return ws


def gg_dglu(a, b_dense, b_ptrs, b_major, n, c, padded_offsets, alpha, beta, prob, d_row, dprob,
            dbias=None, act=GG_DSWIGLU, geglu_alpha=1.702, clamp_min=-7.0, clamp_max=7.0,
            linear_offset=1.0, flags=0, workspace=None, stream=None):
    """Grouped dgrad + dSwiGLU/dGeGLU (gg_dglu of gg_moe.h).  Returns the
    workspace used."""
    L = load_library()
    nl = padded_offsets.numel()
    ws, nbytes = _workspace(workspace, L.gg_dglu_workspace_size(nl, n, dbias is not None), a, stream)
    _check(L.gg_dglu(_ptr(a), a.shape[0], a.shape[1], _ptr(b_dense), _ptr(b_ptrs), b_major, n,
                     _ptr(c), _TORCH_DTYPE[c.dtype], _ptr(padded_offsets), nl, _ptr(alpha),
                     _ptr(beta), _ptr(prob), _ptr(d_row), _TORCH_DTYPE[d_row.dtype], _ptr(dprob),
                     _ptr(dbias), act, geglu_alpha, clamp_min, clamp_max, linear_offset, flags,
                     _ptr(ws), nbytes, _stream(stream)))
    return ws


def gg_dglu_mx(a, sfa, b, sfb, b_ptrs, sfb_ptrs, n, c, padded_offsets, alpha, beta, prob, d_row,
               dprob, dbias=None, amax=None, fp8_out=None, act=GG_DSWIGLU, geglu_alpha=1.702, clamp_min=-7.0,
               clamp_max=7.0, linear_offset=1.0, situ_beta1=4.0, situ_beta2=25.0, flags=0,
               workspace=None, stream=None, b_major=GG_MAJOR_K):
    """Grouped MXFP8 dgrad + dSwiGLU/dGeGLU/dSiTU-GLU (gg_dglu_mx of
    gg_moe.h): a is an (m_rows, k) tensor of FP8 codes (uint8 or
    float8_e4m3fn: E4M3; float8_e5m2: E5M2, as for gg_wgrad_mx).  b / b_ptrs
    hold (n, k) codes per expert with b_major GG_MAJOR_K, (k, n) ones with
    GG_MAJOR_N.  c may be float8_e4m3fn / float8_e5m2.  With a float8_e4m3fn / float8_e5m2 d_row
    fp8_out is a dict of the other FP8 outputs (sfd_row, norm_const and
    optionally d_col, sfd_col).  Returns the workspace used."""
    q = _fp8_out(fp8_out)
    L = load_library()
    nl = padded_offsets.numel()
    ws, nbytes = _workspace(workspace, L.gg_dglu_workspace_size(nl, n, dbias is not None), a, stream)
    _check(L.gg_dglu_mx(_ptr(a), _ptr(sfa), a.shape[0], a.shape[1], _ptr(b), _ptr(sfb),
                        _ptr(b_ptrs), _ptr(sfb_ptrs), b_major, n, _ptr(c), _TORCH_DTYPE[c.dtype],
                        _ptr(padded_offsets), nl, _ptr(alpha), _ptr(beta), _ptr(prob),
                        _ptr(d_row), _TORCH_DTYPE[d_row.dtype], _ptr(dprob), _ptr(dbias),
                        _ptr(amax), _ref(q), act, geglu_alpha, clamp_min, clamp_max, linear_offset,
                        situ_beta1, situ_beta2, _ab(a, flags), _ptr(ws), nbytes, _stream(stream)))
    return ws


def gg_dsrelu(a, sfa, b, sfb, b_ptrs, sfb_ptrs, n, c, padded_offsets, alpha, prob, d_row, dprob,
              amax=None, fp8_out=None, flags=0, workspace=None, stream=None, b_major=GG_MAJOR_K):
    """Grouped MXFP8 dgrad + dsReLU (gg_dsrelu of gg_moe.h); operand, C and
    D dtypes and fp8_out as for gg_dglu_mx.  Returns the workspace used."""
    q = _fp8_out(fp8_out)
    L = load_library()
    nl = padded_offsets.numel()
    ws, nbytes = _workspace(workspace, L.gg_dsrelu_workspace_size(nl), a, stream)
    _check(L.gg_dsrelu(_ptr(a), _ptr(sfa), a.shape[0], a.shape[1], _ptr(b), _ptr(sfb),
                       _ptr(b_ptrs), _ptr(sfb_ptrs), b_major, n, _ptr(c), _TORCH_DTYPE[c.dtype],
                       _ptr(padded_offsets), nl, _ptr(alpha), _ptr(prob), _ptr(d_row),
                       _TORCH_DTYPE[d_row.dtype], _ptr(dprob), _ptr(amax), _ref(q), _ab(a, flags), _ptr(ws),
                       nbytes, _stream(stream)))
    return ws
