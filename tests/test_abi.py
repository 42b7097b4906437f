"""The C ABI without a GPU: the library loads, exports every function that
include/gg_moe.h declares, and rejects invalid arguments on the host (before
any device call) with the documented status codes.  Pointers here are fake
aligned addresses: validation never dereferences them."""
import ctypes
import os
import re

import pytest
import torch

from moe_grouped_gemm_offset_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gg_moe.h")

OK, NULL, SHAPE, DTYPE, LAYOUT, ALIGN, MODE, WORKSPACE, UNSUPPORTED, DEVICE, HIP, OFFSETS, VALUE = \
    range(13)

P = 1 << 20          # a fake 256-byte aligned device address
WS = 1 << 24


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(gg_\w+)\s*\(", src, re.M)))


def test_loads_and_exports_every_declared_symbol():
    lib = B.load_library()
    names = declared()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert B.gg_abi_version() == 3


def test_peak_probe_library():
    """The benchmark's MFMA rate probe is built beside the library, exports its
    one function and rejects invalid arguments without launching."""
    path = os.path.join(ROOT, "moe_grouped_gemm_offset_amd", "libgg_peak.so")
    lib = ctypes.CDLL(path)
    f = lib.gg_peak_mfma
    f.restype = ctypes.c_double
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(2, 1, 1, P, None) == -1.0
    assert f(0, 0, 1, P, None) == -1.0
    assert f(1, 1, 0, P, None) == -1.0
    assert f(0, 1, 1, None, None) == -1.0


def test_workspace_sizes():
    assert B.gg_wgrad_workspace_size(64) == 256 + 64 * 16
    assert B.gg_wgrad_workspace_size(1024) == 256 + 1024 * 16
    assert B.gg_dglu_workspace_size(32, 1536, 1) == 256 + 32 * 3072 * 4
    assert B.gg_dglu_workspace_size(32, 1536, 0) == 256
    assert B.gg_dsrelu_workspace_size(16) == 256


def wgrad(**kw):
    args = dict(a=P, a_major=0, b=P, b_major=2, offsets=P, E=4, T=1024, hidden=256, inter=256,
                dense=P, ptrs=None, dtype=2, acc=0, flags=0, ws=WS, wsb=4096, stream=None)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_wgrad(args["a"], args["a_major"], args["b"], args["b_major"], args["offsets"],
                        args["E"], args["T"], args["hidden"], args["inter"], args["dense"],
                        args["ptrs"], args["dtype"], args["acc"], args["flags"], args["ws"],
                        args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(offsets=None), NULL),
    (dict(ws=None), NULL),
    (dict(a=None), NULL),
    (dict(a_major=2), LAYOUT),
    (dict(b_major=1), LAYOUT),
    (dict(dtype=3), DTYPE),
    (dict(ptrs=P), MODE),
    (dict(dense=None), MODE),
    (dict(E=0), SHAPE),
    (dict(E=1025), SHAPE),
    (dict(T=-8), SHAPE),
    (dict(hidden=96), UNSUPPORTED),
    (dict(T=1020), ALIGN),
    (dict(a=P + 8), ALIGN),
    (dict(dense=P + 4), ALIGN),
    (dict(ws=WS + 16), ALIGN),
    (dict(wsb=100), WORKSPACE),
    (dict(flags=1), MODE),
    (dict(flags=32), MODE),
    (dict(T=1 << 22), UNSUPPORTED),
    (dict(hidden=1 << 20, inter=1 << 20, E=1024), UNSUPPORTED),
])
def test_wgrad_rejects(kw, status):
    assert wgrad(**kw) == status
    assert B.gg_last_error() != ""


def wgrad_noalloc(**kw):
    args = dict(a=P, a_major=0, b=P, b_major=2, offsets=P, E=4, T=1024, hidden=256, inter=256,
                dense=P, ptrs=None, dtype=2, acc=0, flags=0, stream=None)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_wgrad_noalloc(args["a"], args["a_major"], args["b"], args["b_major"],
                                args["offsets"], args["E"], args["T"], args["hidden"], args["inter"],
                                args["dense"], args["ptrs"], args["dtype"], args["acc"], args["flags"],
                                args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(E=1025), WORKSPACE),
    (dict(E=0), SHAPE),
    (dict(offsets=None), NULL),
    (dict(a=None), NULL),
    (dict(a_major=2), LAYOUT),
    (dict(dtype=3), DTYPE),
    (dict(ptrs=P), MODE),
    (dict(hidden=96), UNSUPPORTED),
    (dict(T=1020), ALIGN),
    (dict(flags=1), MODE),
])
def test_wgrad_noalloc_rejects(kw, status):
    """Host checks of the static-scratch entry, before any device call; its
    scratch holds the workspace of at most 1024 experts."""
    assert wgrad_noalloc(**kw) == status
    assert B.gg_last_error() != ""
    if kw.get("E") == 1025:
        assert "1024 experts" in B.gg_last_error()


def dglu(**kw):
    args = dict(a=P, M=1024, k=256, bd=P, bp=None, bm=0, n=256, c=P, cdt=0, po=P, L=4, alpha=P,
                beta=P, prob=P, d=P, ddt=0, dprob=P, dbias=None, act=0, flags=0, ws=WS, wsb=1 << 20)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_dglu(args["a"], args["M"], args["k"], args["bd"], args["bp"], args["bm"], args["n"],
                       args["c"], args["cdt"], args["po"], args["L"], args["alpha"], args["beta"],
                       args["prob"], args["d"], args["ddt"], args["dprob"], args["dbias"], args["act"],
                       1.702, -7.0, 7.0, 1.0, args["flags"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(po=None), NULL),
    (dict(alpha=None), NULL),
    (dict(bp=P), MODE),
    (dict(bd=None), MODE),
    (dict(bm=2), LAYOUT),
    (dict(bm=1, bd=None, bp=P), LAYOUT),
    (dict(cdt=3), DTYPE),
    (dict(act=2), MODE),
    (dict(act=3), MODE),
    (dict(n=48), SHAPE),
    (dict(k=96), UNSUPPORTED),
    (dict(L=0), SHAPE),
    (dict(L=1025), SHAPE),
    (dict(c=P + 2), ALIGN),
    (dict(flags=8), MODE),
    (dict(flags=32), MODE),
    (dict(dbias=P, wsb=256), WORKSPACE),
])
def test_dglu_rejects(kw, status):
    assert dglu(**kw) == status


def dsrelu(**kw):
    args = dict(a=P, sfa=P, M=1024, k=512, b=P, sfb=P, bp=None, sp=None, bm=0, n=256, c=P, cdt=0,
                po=P, L=4, alpha=P, prob=P, d=P, ddt=0, dprob=P, amax=P, fp8=None, flags=0, ws=WS,
                wsb=256)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_dsrelu(args["a"], args["sfa"], args["M"], args["k"], args["b"], args["sfb"],
                         args["bp"], args["sp"], args["bm"], args["n"], args["c"], args["cdt"], args["po"],
                         args["L"], args["alpha"], args["prob"], args["d"], args["ddt"], args["dprob"],
                         args["amax"], args["fp8"], args["flags"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sfa=None), NULL),
    (dict(b=None, sfb=None), MODE),
    (dict(bp=P, sp=P), MODE),
    (dict(sfb=None), MODE),
    (dict(k=192), UNSUPPORTED),
    (dict(n=40), SHAPE),
    (dict(bm=1), LAYOUT),
    (dict(bm=3), LAYOUT),
    (dict(ddt=5), DTYPE),
    (dict(cdt=5), DTYPE),
    (dict(ddt=4), NULL),               # FP8 D without fp8_out
    (dict(sfa=P + 1), ALIGN),
    (dict(wsb=16), WORKSPACE),
    (dict(flags=8), MODE),
    (dict(flags=64), MODE),
    (dict(flags=32), UNSUPPORTED),     # E5M2 operands with a 16/32-bit D
    (dict(flags=32, ddt=2), UNSUPPORTED),
])
def test_dsrelu_rejects(kw, status):
    assert dsrelu(**kw) == status


@pytest.mark.parametrize("entry", ["wgrad", "wgrad_noalloc", "dglu", "dsrelu", "dglu_mx"])
def test_static_sched_flag_accepted(entry):
    """GG_FLAG_STATIC_SCHED passes every entry's flag check: the call gets as
    far as it gets without it (the device check, where there is no GPU)."""
    if torch.cuda.is_available():
        pytest.skip("checks the no-device path")
    call = globals()[entry]
    assert call(flags=16) == call(flags=0) == DEVICE


def fp8_out(**kw):
    f = dict(d_col=P, sfd_row=P, sfd_col=P, norm_const=P)
    f.update(kw)
    return B.Fp8Out(f["d_col"], f["sfd_row"], f["sfd_col"], f["norm_const"])


@pytest.mark.parametrize("entry", ["dsrelu", "dglu_mx"])
@pytest.mark.parametrize("kw,status", [
    (dict(), None),
    (dict(d_col=None), MODE),
    (dict(sfd_col=None), MODE),
    (dict(d_col=None, sfd_col=None), None),
    (dict(sfd_row=None), NULL),
    (dict(norm_const=None), NULL),
    (dict(d_col=P + 8), ALIGN),
    (dict(norm_const=P + 2), ALIGN),
])
def test_fp8_out_checks(entry, kw, status):
    """FP8 outputs (GG_F8E4M3, GG_F8E5M2): fp8_out is required and checked;
    valid ones reach the device check (GG_ERR_DEVICE here, where there is no
    GPU)."""
    f = fp8_out(**kw)                  # kept alive across the calls below
    call = dsrelu if entry == "dsrelu" else dglu_mx
    got = call(ddt=3, fp8=ctypes.addressof(f))
    want = status if status is not None else (DEVICE if not torch.cuda.is_available() else OK)
    if status is None and torch.cuda.is_available():
        pytest.skip("checks the no-device path")
    assert got == want
    assert call(ddt=3, fp8=None) == NULL
    assert call(ddt=4, fp8=ctypes.addressof(f)) == got, "E5M2 outputs take the same checks"
    assert call(ddt=4, fp8=None) == NULL
    assert call(ddt=5, fp8=ctypes.addressof(f)) == DTYPE


def dglu_mx(**kw):
    args = dict(a=P, sfa=P, M=1024, k=512, b=P, sfb=P, bp=None, sp=None, bm=0, n=256, c=P, cdt=0,
                po=P, L=4, alpha=P, beta=P, prob=P, d=P, ddt=0, dprob=P, dbias=None, amax=P, fp8=None,
                act=0, flags=0, ws=WS, wsb=1 << 20, b1=4.0, b2=25.0)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_dglu_mx(args["a"], args["sfa"], args["M"], args["k"], args["b"], args["sfb"],
                          args["bp"], args["sp"], args["bm"], args["n"], args["c"], args["cdt"], args["po"],
                          args["L"], args["alpha"], args["beta"], args["prob"], args["d"],
                          args["ddt"], args["dprob"], args["dbias"], args["amax"], args["fp8"], args["act"],
                          1.702, -7.0, 7.0, 1.0, args["b1"], args["b2"], args["flags"], args["ws"],
                          args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sfa=None), NULL),
    (dict(beta=None), NULL),
    (dict(b=None, sfb=None), MODE),
    (dict(bp=P, sp=P), MODE),
    (dict(b=None, sfb=None, bp=P), MODE),
    (dict(act=3), MODE),
    (dict(flags=8), MODE),
    (dict(bm=1), LAYOUT),
    (dict(act=2, b1=0.0), VALUE),
    (dict(act=2, b2=-1.0), VALUE),
    (dict(act=2, b1=float("inf")), VALUE),
    (dict(act=2, b2=float("nan")), VALUE),
    (dict(k=192), UNSUPPORTED),
    (dict(n=1 << 21), UNSUPPORTED),
    (dict(n=40), SHAPE),
    (dict(cdt=5), DTYPE),
    (dict(ddt=5), DTYPE),
    (dict(flags=64), MODE),
    (dict(flags=32), UNSUPPORTED),     # E5M2 operands with a 16/32-bit D
    (dict(amax=P + 2), ALIGN),
    (dict(a=P + 8), ALIGN),
    (dict(dbias=P, wsb=256), WORKSPACE),
])
def test_dglu_mx_rejects(kw, status):
    assert dglu_mx(**kw) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_a_gpu_reports_device():
    assert wgrad() == DEVICE
    assert dglu() == DEVICE
    assert dsrelu() == DEVICE
    assert dglu_mx() == DEVICE
    assert dglu_mx(act=2) == DEVICE
    assert dglu_mx(act=0, b1=0.0) == DEVICE, "the dSiTU scales are ignored for other activations"
    assert dsrelu(bm=2) == DEVICE, "N-major B"
    assert dsrelu(bm=2, b=None, sfb=None, bp=P, sp=P) == DEVICE
    assert dglu_mx(bm=2) == DEVICE
    assert dglu_mx(bm=2, b=None, sfb=None, bp=P, sp=P, act=2) == DEVICE


def wgrad_mx(**kw):
    args = dict(a=P, sfa=P, b=P, sfb=P, offsets=P, E=4, T=1024, hidden=256, inter=256, dense=P,
                ptrs=None, dtype=2, acc=0, flags=0, ws=WS, wsb=4096)
    args.update(kw)
    lib = B.load_library()
    return lib.gg_wgrad_mx(args["a"], args["sfa"], args["b"], args["sfb"], args["offsets"],
                           args["E"], args["T"], args["hidden"], args["inter"], args["dense"],
                           args["ptrs"], args["dtype"], args["acc"], args["flags"], args["ws"],
                           args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sfa=None), NULL),
    (dict(dtype=3), DTYPE),
    (dict(dtype=4), DTYPE),
    (dict(T=1000), ALIGN),
    (dict(sfb=P + 2), ALIGN),
    (dict(flags=64), MODE),
    (dict(flags=1), MODE),
])
def test_wgrad_mx_rejects(kw, status):
    assert wgrad_mx(**kw) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
@pytest.mark.parametrize("entry,kw", [
    ("wgrad_mx", dict(flags=32)),
    ("wgrad_mx", dict(flags=32 | 8, dtype=0)),
    ("dsrelu", dict(cdt=3)),
    ("dsrelu", dict(cdt=4)),
    ("dglu_mx", dict(cdt=3)),
    ("dglu_mx", dict(cdt=4, act=2)),
])
def test_fp8_formats_accepted(entry, kw):
    """E5M2 operands (GG_FLAG_AB_E5M2) on gg_wgrad_mx, and FP8 C (E4M3,
    E5M2) on the block-scaled dgrad entries, pass the host checks."""
    assert globals()[entry](**kw) == DEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
@pytest.mark.parametrize("entry", ["dsrelu", "dglu_mx"])
@pytest.mark.parametrize("ddt", [3, 4])
def test_e5m2_operands_with_fp8_out(entry, ddt):
    """GG_FLAG_AB_E5M2 with an FP8 D (either format) passes the host checks;
    the non-block-scaled entries reject the flag."""
    f = fp8_out()
    assert globals()[entry](flags=32, ddt=ddt, fp8=ctypes.addressof(f)) == DEVICE
    assert globals()[entry](flags=32, ddt=ddt, cdt=4, fp8=ctypes.addressof(f)) == DEVICE
    assert wgrad(flags=32) == MODE
    assert dglu(flags=32) == MODE
    assert dglu(cdt=3) == DTYPE
