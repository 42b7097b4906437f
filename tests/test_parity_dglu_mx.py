"""GPU parity of gg_dglu_mx against the oracle (through the C ABI).

Small cases span several tiles, a partial N tile, an empty group, rows past
valid_m, per-row scale spreads, dense and discrete (b_ptrs / sfb_ptrs) B,
all three activations (dSiTU-GLU with default and small tanh scales), the
gate-first and mask-filter flags, dbias, and C/D dtypes; the MoE-scale
workload (L 32, K 4096, N 1536, M 32768, discrete B) runs at full size in
the bench's launch configuration and is checked against the oracle on
sampled rows of every group and on every row and the amax halves of its
256-row groups.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth
from tests.parity_util import ORC_DT, TOL, assert_close, normwise, say, values

pytestmark = pytest.mark.gpu


def gg():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def column_maps(N, gate_first=False):
    n = np.arange(N)
    p, j = n // 32, n % 32
    cin = 64 * p + (32 if gate_first else 0) + j
    cgt = 64 * p + (0 if gate_first else 32) + j
    return cin, cgt


def run_gpu(inp, d_dtype=torch.bfloat16, with_amax=True, dbias=False, act=orc.DSWIGLU, flags=0,
            situ=(4.0, 25.0), b_major="k"):
    """b_major "n" hands the kernel B's codes N-major ((N, K) per expert
    transposed to (K, N), the same values; the oracle reads the K-major
    ones); the scales keep their (N, K/32) layout."""
    b = gg()
    dev = lambda x: x.cuda()
    nmaj = b_major == "n"
    lay = (lambda x: x.transpose(-1, -2).contiguous()) if nmaj else (lambda x: x)
    M, N, L = inp["M"], inp["N"], inp["L"]
    a = dev(inp["a"]).view(torch.uint8)
    keep = []
    if inp["b_dense"] is not None:
        bd, sd = lay(dev(inp["b_dense"]).view(torch.uint8)), dev(inp["sfb_dense"])
        bp = sp = None
    else:
        kb = [lay(dev(x).view(torch.uint8)) for x in inp["b_list"]]
        ks = [dev(x) for x in inp["sfb_list"]]
        keep += kb + ks
        bp = torch.tensor([x.data_ptr() for x in kb], dtype=torch.int64, device="cuda")
        sp = torch.tensor([x.data_ptr() for x in ks], dtype=torch.int64, device="cuda")
        bd = sd = None
    d = torch.full((M, 2 * N), float("nan"), dtype=d_dtype, device="cuda")
    dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
    amax = torch.full((L, 2), -1.0, dtype=torch.float32, device="cuda") if with_amax else None
    db = torch.zeros(L, 2 * N, dtype=torch.bfloat16, device="cuda") if dbias else None
    ws = b.gg_dglu_mx(a, dev(inp["sfa"]), bd, sd, bp, sp, N, dev(inp["c"]),
                      dev(inp["padded_offsets"]), dev(inp["alpha"]), dev(inp["beta"]),
                      dev(inp["prob"]), d, dprob, dbias=db, amax=amax, act=act, flags=flags,
                      situ_beta1=situ[0], situ_beta2=situ[1],
                      b_major=b.GG_MAJOR_N if nmaj else b.GG_MAJOR_K)
    torch.cuda.synchronize()
    err = b.gg_device_error(ws)
    return dict(d=d.cpu(), dprob=dprob.cpu(), amax=(amax.cpu() if with_amax else None),
                dbias=(db.cpu() if dbias else None), err=err)


def run_oracle(inp, d_dtype=torch.bfloat16, rows=None, dbias=False, act=orc.DSWIGLU, flags=0,
               situ=(4.0, 25.0)):
    L, N = inp["L"], inp["N"]
    return orc.dglu_mx(synth.bits(inp["a"]), synth.bits(inp["sfa"]), inp["M"], inp["K"],
                       [synth.bits(x) for x in inp["b_list"]],
                       [synth.bits(x) for x in inp["sfb_list"]], N, synth.bits(inp["c"]),
                       ORC_DT[inp["c"].dtype], inp["padded_offsets"].numpy(),
                       inp["alpha"].numpy(), inp["beta"].numpy(), inp["prob"].numpy(), act=act,
                       situ_beta1=situ[0], situ_beta2=situ[1], gate_first=bool(flags & 1),
                       mask_filter=bool(flags & 2),
                       d_dtype=ORC_DT[d_dtype], rows=rows,
                       dbias_in=np.zeros((L, 2 * N), np.uint16) if dbias else None)


def small(seed, discrete=False, c_dtype=torch.bfloat16, spread=3, c_std=2.0):
    counts = [256, 512, 0, 256]
    return synth.dglu_mx_inputs(4, 512, 320, counts, c_std=c_std, c_dtype=c_dtype, m_extra=64,
                                seed=seed, discrete=discrete, scale_spread=spread)


def check(inp, got, ref, d_dtype=orc.BF16):
    vm = inp["valid_m"]
    assert got["err"] == 0
    assert_close(values(got["d"][:vm]), ref["D"][:vm], d_dtype, "D_row")
    assert torch.all(torch.isnan(got["d"][vm:])), "rows past valid_m are not written"
    assert_close(values(got["dprob"][:vm]), ref["dprob"][:vm], orc.F32, "dprob")
    assert torch.all(got["dprob"][vm:] == 0)
    start = 0
    for g, c in enumerate(inp["counts"]):
        if c:
            e = normwise(values(got["d"][start:start + c]), ref["D"][start:start + c])
            assert e <= TOL[d_dtype], f"group {g}: {e:.3e}"
        start += c


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU, orc.DSITUGLU])
@pytest.mark.parametrize("discrete", [False, True])
def test_small(discrete, act):
    inp = small(81, discrete, c_std=4.0 if act == orc.DGEGLU else 2.0)
    say("dglu_mx small", "discrete" if discrete else "dense", ["dswiglu", "dgeglu", "dsituglu"][act])
    got = run_gpu(inp, act=act)
    ref = run_oracle(inp, act=act)
    check(inp, got, ref)
    amax = got["amax"].numpy()
    assert np.all(amax[2] == 0.0), "an empty expert's amax is 0"
    assert_close(amax.ravel(), ref["amax"].ravel(), orc.F32, "amax")
    for g in (0, 1, 3):
        for h in range(2):
            assert abs(amax[g, h] - ref["amax"][g, h]) <= 1e-3 * ref["amax"][g, h], (g, h)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_flags(flags):
    inp = small(82, True, c_std=4.0)
    got = run_gpu(inp, act=orc.DGEGLU, flags=flags)
    ref = run_oracle(inp, act=orc.DGEGLU, flags=flags)
    check(inp, got, ref)
    assert_close(got["amax"].numpy().ravel(), ref["amax"].ravel(), orc.F32, "amax")


def test_dbias():
    inp = small(83, True)
    got = run_gpu(inp, dbias=True)
    ref = run_oracle(inp, dbias=True)
    check(inp, got, ref)
    assert_close(values(got["dbias"]), ref["dbias"], orc.BF16, "dbias")
    assert torch.all(got["dbias"][2] == 0), "an empty expert's dbias stays 0"


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU, orc.DSITUGLU])
@pytest.mark.parametrize("discrete", [False, True])
def test_n_major(discrete, act):
    """N-major B ("Parameters / Input tensor B (dense mode)": K-major or
    N-major), dense and discrete, all three activations, with dbias."""
    inp = small(86, discrete, c_std=4.0 if act == orc.DGEGLU else 2.0)
    say("dglu_mx N-major", "discrete" if discrete else "dense", act)
    got = run_gpu(inp, act=act, dbias=True, b_major="n")
    ref = run_oracle(inp, act=act, dbias=True)
    check(inp, got, ref)
    assert_close(values(got["dbias"]), ref["dbias"], orc.BF16, "dbias")
    assert_close(got["amax"].numpy().ravel(), ref["amax"].ravel(), orc.F32, "amax")


@pytest.mark.parametrize("c_dtype", [torch.float8_e4m3fn, torch.float8_e5m2])
@pytest.mark.parametrize("act,d_dtype", [(orc.DSWIGLU, torch.bfloat16), (orc.DGEGLU, torch.float32),
                                         (orc.DSITUGLU, torch.float16)])
def test_fp8_c(c_dtype, act, d_dtype):
    """An FP8 C (the dGLU page's "Input tensor C" dtypes) is read as its
    exact value, with dbias."""
    inp = small(85, True, c_dtype=c_dtype, c_std=4.0 if act == orc.DGEGLU else 2.0)
    say("dglu_mx fp8 C", c_dtype, "act", act, "D", d_dtype)
    got = run_gpu(inp, d_dtype, act=act, dbias=True)
    ref = run_oracle(inp, d_dtype, act=act, dbias=True)
    check(inp, got, ref, ORC_DT[d_dtype])
    assert_close(values(got["dbias"]), ref["dbias"], orc.BF16, "dbias")
    assert_close(got["amax"].numpy().ravel(), ref["amax"].ravel(), orc.F32, "amax")


@pytest.mark.parametrize("c_dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("d_dtype", [torch.float16, torch.float32])
def test_dtypes(c_dtype, d_dtype):
    inp = small(84, c_dtype=c_dtype)
    got = run_gpu(inp, d_dtype, act=orc.DGEGLU)
    ref = run_oracle(inp, d_dtype, act=orc.DGEGLU)
    check(inp, got, ref, ORC_DT[d_dtype])


@pytest.mark.parametrize("situ", [(4.0, 25.0), (1.0, 2.0)])
@pytest.mark.parametrize("c_dtype", [torch.bfloat16, torch.float32])
def test_situ(c_dtype, situ):
    """dSiTU-GLU with the page's default scales and with small ones (tanh
    saturates), C drawn N(0, 4); fp32 D so the 1e-3 tolerance applies."""
    inp = small(86, True, c_dtype=c_dtype, c_std=4.0)
    got = run_gpu(inp, torch.float32, act=orc.DSITUGLU, situ=situ, dbias=True)
    ref = run_oracle(inp, torch.float32, act=orc.DSITUGLU, situ=situ, dbias=True)
    check(inp, got, ref, orc.F32)
    assert_close(values(got["dbias"]), ref["dbias"], orc.BF16, "dbias")
    assert_close(got["amax"].numpy().ravel(), ref["amax"].ravel(), orc.F32, "amax")


def test_unit_scales_no_amax():
    inp = small(85, spread=0)
    inp["sfa"] = torch.full_like(inp["sfa"], 127)
    got = run_gpu(inp, with_amax=False)
    ref = run_oracle(inp)
    check(inp, got, ref)


def test_workload_sampled():
    """The block-scaled dGLU workload at full size (L 32, K 4096, N 1536,
    M 32768, discrete B and SFB): the first and last rows of every group and
    every row of its 256-row groups against the oracle; those groups' amax
    halves equal the oracle's, every other group's are at least the oracle's
    |D| on its listed rows."""
    w = synth.WORKLOADS["dglu_mxfp8"]
    counts = synth.workload_counts("dglu_mxfp8")
    inp = synth.dglu_mx_inputs(w["L"], w["K"], w["N"], counts, c_std=w["c_std"], seed=w["seed"],
                               device="cuda", discrete=w["discrete"])
    say("dglu_mxfp8 counts", counts.tolist())
    got = run_gpu(inp)
    assert got["err"] == 0
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cpu["b_list"] = [x.cpu() for x in inp["b_list"]]
    cpu["sfb_list"] = [x.cpu() for x in inp["sfb_list"]]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    whole = [g for g, c in enumerate(counts) if c == 256]
    assert whole
    rows = set()
    for g, (s, c) in enumerate(zip(starts, counts)):
        if g in whole:
            rows.update(range(s, s + c))
        elif c:
            rows.update([s, s + c - 1])
    rows = np.array(sorted(rows), np.int64)
    ref = run_oracle(cpu, rows=rows)
    assert_close(values(got["d"][rows]), ref["D"], orc.BF16, "D_row (listed rows)")
    assert_close(values(got["dprob"][rows]), ref["dprob"], orc.F32, "dprob (listed rows)")
    amax = got["amax"].numpy().astype(np.float64)
    for g, c in enumerate(counts):
        for h in range(2):
            if g in whole:
                assert abs(amax[g, h] - ref["amax"][g, h]) <= 1e-3 * ref["amax"][g, h], \
                    (g, h, amax[g, h], ref["amax"][g, h])
            elif c:
                assert amax[g, h] >= ref["amax"][g, h] * (1 - 1e-3), (g, h, amax[g, h], ref["amax"][g, h])
