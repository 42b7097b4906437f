"""GPU parity of the FP8 (E4M3 and E5M2) outputs of gg_dsrelu and
gg_dglu_mx against the oracle's step 3 (orc_quant_fp8) applied to the
oracle's D, for E4M3 and E5M2 operands (GG_FLAG_AB_E5M2) and 16-bit or FP8
C.

The kernel's D (fp32 accumulation) and the oracle's D (double) differ by a
few fp32 ulps, so a block's scale exponent may differ where
norm_const * amax / fmax (448 for E4M3, 57344 for E5M2) lies within that
distance of a power of two, and a code may differ by one step where a value
lies that close to a rounding midpoint.  The tests check: every scale that
differs belongs to such a boundary block; at least 99% of the codes are
identical; and the dequantized outputs (code * 2^e / norm_const) are within
the format's bound of the oracle's exact D, normwise half a step of its
fraction bits (2^-4 for E4M3's 3, 2^-3 for E5M2's 2) plus the 1e-2 of the
16-bit outputs.  Rows past valid_m and their scales are not written.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth
from tests.parity_util import ORC_DT, normwise, say

pytestmark = pytest.mark.gpu

SENT = 0x7F                                   # NaN in both formats: "not written"
# per output format: code -> value table, largest value, normwise tolerance
FMT = {
    orc.E4M3: (torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy(),
               448.0, 2.0 ** -4 + 1e-2),
    orc.E5M2: (torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().double().numpy(),
               57344.0, 2.0 ** -3 + 1e-2),
}
TORCH_FP8 = {orc.E4M3: torch.float8_e4m3fn, orc.E5M2: torch.float8_e5m2}


def gg():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def outputs(M, W):
    P = (M + 31) // 32
    d_row = torch.full((M, W), SENT, dtype=torch.uint8, device="cuda")
    d_col = torch.full((M, W), SENT, dtype=torch.uint8, device="cuda")
    sfd_row = torch.full((M, W // 32), SENT, dtype=torch.uint8, device="cuda")
    sfd_col = torch.full((W, P), SENT, dtype=torch.uint8, device="cuda")
    return d_row, dict(d_col=d_col, sfd_row=sfd_row, sfd_col=sfd_col)


def check(name, got_row, fp8, D, nc, vm, fmt=orc.E4M3):
    """got_row / fp8: the kernel's outputs (CPU tensors) in format fmt; D:
    the oracle's float64 D of rows 0 .. vm-1."""
    table, fmax, tol = FMT[fmt]
    ref = orc.quant_fp8(D, nc, with_col=True, d_dtype=fmt)
    M, W = got_row.shape
    P = fp8["sfd_col"].shape[1]
    # untouched rows and scale blocks past valid_m
    assert torch.all(got_row[vm:] == SENT) and torch.all(fp8["d_col"][vm:] == SENT)
    assert torch.all(fp8["sfd_row"][vm:] == SENT) and torch.all(fp8["sfd_col"][:, vm // 32:] == SENT)
    for kind, codes, sfd, rq, rs in (
            ("row", got_row[:vm].numpy(), fp8["sfd_row"][:vm].numpy(), ref["q_row"], ref["sfd_row"]),
            ("col", fp8["d_col"][:vm].numpy(), fp8["sfd_col"][:, :vm // 32].numpy(), ref["q_col"],
             ref["sfd_col"])):
        if kind == "row":
            Db = D.reshape(vm, W // 32, 32)
            e = sfd.astype(np.int64) - 127
            deq = table[codes].reshape(vm, W // 32, 32) * np.exp2(e)[..., None] / nc
            deq = deq.reshape(vm, W)
        else:
            Db = D.T.reshape(W, vm // 32, 32)
            e = sfd.astype(np.int64) - 127
            deq = (table[codes.T].reshape(W, vm // 32, 32) * np.exp2(e)[..., None] / nc).reshape(W, vm).T
        amax = np.abs(Db.astype(np.float32)).max(axis=2).astype(np.float64)
        lg = np.log2(np.maximum(nc * amax / fmax, 1e-300))
        boundary = np.abs(lg - np.round(lg)) < 1e-4
        differ = sfd != rs
        assert not np.any(differ & ~boundary), f"{name} {kind}: {int(np.sum(differ & ~boundary))} scales differ"
        same = np.mean(codes == rq)
        err = normwise(deq, D)
        say(f"  {name} {kind}: codes identical {same:.5f}, scales differing {int(differ.sum())}, "
            f"dequantized normwise {err:.3e} (tol {tol:.3e})")
        assert same >= 0.99, f"{name} {kind}: only {same:.4f} of the codes agree"
        assert err <= tol


def dsrelu_inputs(seed, discrete=False, ab=orc.E4M3, c_dtype=torch.bfloat16):
    counts = [256, 512, 0, 256]
    return synth.dsrelu_inputs(4, 512, 320, counts, m_extra=64, seed=seed, discrete=discrete,
                               scale_spread=3, ab_dtype=TORCH_FP8[ab], c_dtype=c_dtype)


# (operand format, output format, C dtype, norm_const)
DSRELU_CASES = [
    (orc.E4M3, orc.E4M3, torch.bfloat16, 1.0),
    (orc.E4M3, orc.E4M3, torch.bfloat16, 0.25),
    (orc.E4M3, orc.E5M2, torch.bfloat16, 1.0),
    (orc.E5M2, orc.E4M3, torch.bfloat16, 0.25),
    (orc.E5M2, orc.E5M2, torch.bfloat16, 1.0),
    (orc.E5M2, orc.E5M2, torch.float8_e4m3fn, 1.0),
    (orc.E4M3, orc.E4M3, torch.float8_e5m2, 1.0),
    (orc.E5M2, orc.E5M2, torch.float32, 2.0),
    (orc.E5M2, orc.E4M3, torch.bfloat16, "n"),      # N-major B, norm_const 1
]


@pytest.mark.parametrize("ab,fmt,c_dtype,nc", DSRELU_CASES)
def test_dsrelu_fp8(ab, fmt, c_dtype, nc):
    b = gg()
    nmaj = nc == "n"
    nc = 1.0 if nmaj else nc
    inp = dsrelu_inputs(111, ab=ab, c_dtype=c_dtype)
    M, N, L = inp["M"], inp["N"], inp["L"]
    d_row, fp8 = outputs(M, N)
    ncd = torch.tensor([nc], dtype=torch.float32, device="cuda")
    dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
    amax = torch.zeros(L, dtype=torch.float32, device="cuda")
    say("dsrelu fp8 out: operands", ab, "D", fmt, "C", c_dtype, "norm_const", nc)
    ws = b.gg_dsrelu(inp["a"].cuda(), inp["sfa"].cuda(),
                     (inp["b_dense"].transpose(1, 2).contiguous() if nmaj else inp["b_dense"]).cuda()
                     .view(torch.uint8), inp["sfb_dense"].cuda(), None, None, N,
                     inp["c"].cuda(), inp["padded_offsets"].cuda(), inp["alpha"].cuda(),
                     inp["prob"].cuda(), d_row.view(TORCH_FP8[fmt]), dprob, amax,
                     fp8_out=dict(fp8, norm_const=ncd),
                     b_major=b.GG_MAJOR_N if nmaj else b.GG_MAJOR_K)
    torch.cuda.synchronize()
    assert b.gg_device_error(ws) == 0
    ref = orc.dsrelu(synth.bits(inp["a"]), synth.bits(inp["sfa"]), M, inp["K"],
                     [synth.bits(x) for x in inp["b_list"]], [synth.bits(x) for x in inp["sfb_list"]],
                     N, synth.bits(inp["c"]), ORC_DT[c_dtype], inp["padded_offsets"].numpy(),
                     inp["alpha"].numpy(), inp["prob"].numpy(), ab_dtype=ab)
    vm = inp["valid_m"]
    check("dsrelu", d_row.cpu(), {k: v.cpu() for k, v in fp8.items()}, ref["D"][:vm], nc, vm, fmt)
    got_dp = dprob.cpu().double().numpy()[:vm]
    assert normwise(got_dp, ref["dprob"][:vm]) <= 1e-3


FMT_CASES = [(orc.E4M3, orc.E4M3, torch.bfloat16), (orc.E4M3, orc.E5M2, torch.bfloat16),
             (orc.E5M2, orc.E5M2, torch.float8_e5m2), (orc.E5M2, orc.E4M3, torch.float8_e4m3fn)]


@pytest.mark.parametrize("ab,fmt,c_dtype", FMT_CASES)
@pytest.mark.parametrize("act,flags", [(orc.DSWIGLU, 0), (orc.DGEGLU, 1), (orc.DSITUGLU, 0)])
@pytest.mark.parametrize("with_col", [True, False])
def test_dglu_mx_fp8(act, flags, with_col, ab, fmt, c_dtype):
    if not with_col and (ab, fmt) != (orc.E4M3, orc.E4M3):
        pytest.skip("row-only output: one format case is enough")
    b = gg()
    counts = [256, 512, 0, 256]
    inp = synth.dglu_mx_inputs(4, 512, 320, counts, c_std=4.0, m_extra=64, seed=112,
                               discrete=True, scale_spread=3, ab_dtype=TORCH_FP8[ab],
                               c_dtype=c_dtype)
    M, N, L = inp["M"], inp["N"], inp["L"]
    d_row, fp8 = outputs(M, 2 * N)
    if not with_col:
        fp8["d_col"] = fp8["sfd_col"] = None
    nc = 2.0
    ncd = torch.tensor([nc], dtype=torch.float32, device="cuda")
    dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
    amax = torch.zeros(L, 2, dtype=torch.float32, device="cuda")
    kb = [x.cuda().view(torch.uint8) for x in inp["b_list"]]
    ks = [x.cuda() for x in inp["sfb_list"]]
    bp = torch.tensor([x.data_ptr() for x in kb], dtype=torch.int64, device="cuda")
    sp = torch.tensor([x.data_ptr() for x in ks], dtype=torch.int64, device="cuda")
    say("dglu_mx fp8 out", act, flags, "with D_col" if with_col else "row only", "operands", ab,
        "D", fmt, "C", c_dtype)
    ws = b.gg_dglu_mx(inp["a"].cuda(), inp["sfa"].cuda(), None, None, bp, sp, N,
                      inp["c"].cuda(), inp["padded_offsets"].cuda(), inp["alpha"].cuda(),
                      inp["beta"].cuda(), inp["prob"].cuda(), d_row.view(TORCH_FP8[fmt]), dprob,
                      amax=amax, fp8_out=dict(fp8, norm_const=ncd), act=act, flags=flags)
    torch.cuda.synchronize()
    assert b.gg_device_error(ws) == 0
    ref = orc.dglu_mx(synth.bits(inp["a"]), synth.bits(inp["sfa"]), M, inp["K"],
                      [synth.bits(x) for x in inp["b_list"]], [synth.bits(x) for x in inp["sfb_list"]],
                      N, synth.bits(inp["c"]), ORC_DT[c_dtype], inp["padded_offsets"].numpy(),
                      inp["alpha"].numpy(), inp["beta"].numpy(), inp["prob"].numpy(), act=act,
                      gate_first=bool(flags & 1), ab_dtype=ab)
    vm = inp["valid_m"]
    if with_col:
        check("dglu_mx", d_row.cpu(), {k: v.cpu() for k, v in fp8.items()}, ref["D"][:vm], nc, vm,
              fmt)
    else:
        q = orc.quant_fp8(ref["D"][:vm], nc, with_col=False)
        got = d_row.cpu().numpy()
        assert np.all(got[vm:] == SENT)
        assert np.mean(got[:vm] == q["q_row"]) >= 0.99
    amax_ref = ref["amax"]
    assert np.max(np.abs(amax.cpu().numpy() - amax_ref) / np.maximum(amax_ref, 1e-30)) <= 1e-3
