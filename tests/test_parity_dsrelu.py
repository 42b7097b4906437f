"""GPU parity of gg_dsrelu against the oracle (through the C ABI).

Small cases span several tiles, a partial N tile, an empty group, rows past
valid_m, per-row scale spreads, dense and discrete B, and C/D dtypes; the
MoE-scale workload (L 16, K 7168, N 2048, M 65536) runs at full size in the
bench's launch configuration and is checked against the oracle on sampled
rows of every group and on every row and the Amax of a smallest group.
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


def run_gpu(inp, d_dtype=torch.bfloat16, with_amax=True, b_major="k"):
    """b_major "n" hands the kernel B's codes N-major: each expert's (N, K)
    codes transposed to (K, N), the same values (the oracle reads the K-major
    ones); the scales keep their (N, K/32) layout."""
    b = gg()
    dev = lambda x: x.cuda()
    nmaj = b_major == "n"
    lay = (lambda x: x.transpose(-1, -2).contiguous()) if nmaj else (lambda x: x)
    M, N, L = inp["M"], inp["N"], inp["L"]
    a = dev(inp["a"]).view(torch.uint8)
    if inp["b_dense"] is not None:
        bd, sd = lay(dev(inp["b_dense"]).view(torch.uint8)), dev(inp["sfb_dense"])
        bp = sp = None
    else:
        kb = [lay(dev(x).view(torch.uint8)) for x in inp["b_list"]]
        ks = [dev(x) for x in inp["sfb_list"]]
        bp = torch.tensor([x.data_ptr() for x in kb], dtype=torch.int64, device="cuda")
        sp = torch.tensor([x.data_ptr() for x in ks], dtype=torch.int64, device="cuda")
        bd = sd = None
    d = torch.full((M, N), float("nan"), dtype=d_dtype, device="cuda")
    dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
    amax = torch.full((L,), -1.0, dtype=torch.float32, device="cuda") if with_amax else None
    ws = b.gg_dsrelu(a, dev(inp["sfa"]), bd, sd, bp, sp, N, dev(inp["c"]), dev(inp["padded_offsets"]),
                     dev(inp["alpha"]), dev(inp["prob"]), d, dprob, amax,
                     b_major=b.GG_MAJOR_N if nmaj else b.GG_MAJOR_K)
    torch.cuda.synchronize()
    err = b.gg_device_error(ws)
    if not inp["b_dense"] is None:
        pass
    return d.cpu(), dprob.cpu(), (amax.cpu() if with_amax else None), err


def run_oracle(inp, d_dtype=torch.bfloat16, rows=None):
    return orc.dsrelu(synth.bits(inp["a"]), synth.bits(inp["sfa"]), inp["M"], inp["K"],
                      [synth.bits(x) for x in inp["b_list"]], [synth.bits(x) for x in inp["sfb_list"]],
                      inp["N"], synth.bits(inp["c"]), ORC_DT[inp["c"].dtype],
                      inp["padded_offsets"].numpy(), inp["alpha"].numpy(), inp["prob"].numpy(),
                      d_dtype=ORC_DT[d_dtype], rows=rows)


def small(seed, discrete=False, c_dtype=torch.bfloat16, spread=3):
    counts = [256, 512, 0, 256]
    return synth.dsrelu_inputs(4, 512, 320, counts, c_dtype=c_dtype, m_extra=64, seed=seed,
                               discrete=discrete, scale_spread=spread)


@pytest.mark.parametrize("discrete", [False, True])
def test_small(discrete):
    inp = small(61, discrete)
    say("dsrelu small", "discrete" if discrete else "dense")
    d, dprob, amax, err = run_gpu(inp)
    assert err == 0
    ref = run_oracle(inp)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], orc.BF16, "D_row")
    assert torch.all(torch.isnan(d[vm:]))
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, "dprob")
    assert torch.all(dprob[vm:] == 0)
    assert_close(amax.numpy(), ref["amax"], orc.F32, "amax")
    assert amax[2] == 0.0, "an empty expert's amax is 0"
    start = 0
    for g, c in enumerate(inp["counts"]):
        if c:
            e = normwise(values(d[start:start + c]), ref["D"][start:start + c])
            assert e <= TOL[orc.BF16], f"group {g}: {e:.3e}"
            assert abs(amax[g].item() - ref["amax"][g]) <= 1e-3 * ref["amax"][g]
        start += c


@pytest.mark.parametrize("c_dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("d_dtype", [torch.float16, torch.float32])
def test_dtypes(c_dtype, d_dtype):
    inp = small(62, c_dtype=c_dtype)
    d, dprob, amax, err = run_gpu(inp, d_dtype)
    ref = run_oracle(inp, d_dtype)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], ORC_DT[d_dtype], "D_row")
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, "dprob")


@pytest.mark.parametrize("c_dtype", [torch.float8_e4m3fn, torch.float8_e5m2])
@pytest.mark.parametrize("d_dtype", [torch.bfloat16, torch.float32])
def test_fp8_c(c_dtype, d_dtype):
    """An FP8 C (the dsReLU page's "Input tensor C" dtypes) is read as its
    exact value."""
    inp = small(64, c_dtype=c_dtype, discrete=True)
    say("dsrelu fp8 C", c_dtype, "D", d_dtype)
    d, dprob, amax, err = run_gpu(inp, d_dtype)
    assert err == 0
    ref = run_oracle(inp, d_dtype)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], ORC_DT[d_dtype], "D_row")
    assert torch.all(torch.isnan(d[vm:]))
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, "dprob")
    assert_close(amax.numpy(), ref["amax"], orc.F32, "amax")


def test_unit_scales_no_amax():
    inp = small(63, spread=0)
    inp["sfa"] = torch.full_like(inp["sfa"], 127)
    d, dprob, amax, err = run_gpu(inp, with_amax=False)
    ref = run_oracle(inp)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], orc.BF16, "D_row")


@pytest.mark.parametrize("b_major", ["k", "n"])
def test_workload_sampled(b_major):
    """The dsReLU workload at full size (L 16, K 7168, N 2048, M 65536), with
    dense K-major B (the bench's launch) and with discrete N-major B (the
    page's FP8 discrete b_major "n"): the first and last rows of every group
    and every row of a smallest group (2816 rows) against the oracle; that
    group's Amax equals the oracle's, and every other group's Amax is at
    least the oracle's |D| on its listed rows."""
    w = synth.WORKLOADS["dsrelu_mxfp8"]
    counts = synth.workload_counts("dsrelu_mxfp8")
    inp = synth.dsrelu_inputs(w["L"], w["K"], w["N"], counts, seed=w["seed"], device="cuda",
                              discrete=b_major == "n")
    say("dsrelu_mxfp8 counts", counts.tolist(), "B", b_major)
    d, dprob, amax, err = run_gpu(inp, b_major=b_major)
    assert err == 0
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cpu["b_list"] = [x.cpu() for x in inp["b_list"]]
    cpu["sfb_list"] = [x.cpu() for x in inp["sfb_list"]]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    small_g = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
    rows = set()
    for g, (s, c) in enumerate(zip(starts, counts)):
        if g == small_g:
            rows.update(range(s, s + c))
        elif c:
            rows.update([s, s + c - 1])
    rows = np.array(sorted(rows), np.int64)
    say(f"  oracle on {rows.size} rows (all {counts[small_g]} of group {small_g})")
    ref = run_oracle(cpu, rows=rows)
    assert_close(values(d[rows]), ref["D"], orc.BF16, "D_row (listed rows)")
    assert_close(values(dprob[rows]), ref["dprob"], orc.F32, "dprob (listed rows)")
    got = amax.numpy().astype(np.float64)
    want = ref["amax"][small_g]
    say(f"  amax of group {small_g}: {got[small_g]:.6e} vs oracle {want:.6e}")
    assert abs(got[small_g] - want) <= 1e-3 * want
    for g, c in enumerate(counts):
        if c and g != small_g:
            assert got[g] >= ref["amax"][g] * (1 - 1e-3), (g, got[g], ref["amax"][g])


@pytest.mark.parametrize("case", range(6))
def test_random_shapes(case):
    """Seeded random shapes: K a multiple of 128 from 128 to 2048 (1-16 load
    units, scale groups cut short), compact N a multiple of 32 up to 640
    (partial N tiles), 1-6 groups of 256-multiple rows (some empty), rows
    past valid_m, dense or discrete B, spread scales; every row, dprob and
    amax against the oracle."""
    rng = np.random.default_rng(700 + case)
    K = int(rng.integers(1, 17)) * 128
    N = int(rng.integers(1, 21)) * 32
    L = int(rng.integers(1, 7))
    counts = [int(c) * 256 for c in rng.integers(0, 3, size=L)]
    if sum(counts) == 0:
        counts[0] = 256
    inp = synth.dsrelu_inputs(L, K, N, counts, m_extra=64 * (case % 2), seed=700 + case,
                              discrete=bool(case % 2), scale_spread=3)
    say("dsrelu random", case, "K", K, "N", N, "L", L, counts)
    d, dprob, amax, err = run_gpu(inp)
    assert err == 0
    ref = run_oracle(inp)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], orc.BF16, "D_row")
    assert torch.all(torch.isnan(d[vm:]))
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, "dprob")
    for g, c in enumerate(counts):
        if c == 0:
            assert amax[g] == 0.0, "an empty expert's amax is 0"
        else:
            assert abs(amax[g].item() - ref["amax"][g]) <= 1e-3 * ref["amax"][g]


@pytest.mark.parametrize("case", range(4))
def test_n_major(case):
    """N-major B (the page's FP8 b_major "n"), dense and discrete, partial N
    tiles (N not a multiple of 256), K of one to several load units, with
    C/D dtypes varied: every row, dprob and amax against the oracle."""
    rng = np.random.default_rng(800 + case)
    K = [128, 512, 1152, 2048][case]
    N = [32, 320, 544, 256][case]
    L = [1, 4, 3, 5][case]
    counts = [int(c) * 256 for c in rng.integers(0, 3, size=L)]
    if sum(counts) == 0:
        counts[0] = 256
    c_dtype = [torch.bfloat16, torch.float32, torch.float8_e4m3fn, torch.float16][case]
    d_dtype = [torch.bfloat16, torch.float16, torch.bfloat16, torch.float32][case]
    inp = synth.dsrelu_inputs(L, K, N, counts, c_dtype=c_dtype, m_extra=64 * (case % 2),
                              seed=800 + case, discrete=bool(case % 2), scale_spread=3)
    say("dsrelu N-major", case, "K", K, "N", N, "L", L, counts, c_dtype, d_dtype)
    d, dprob, amax, err = run_gpu(inp, d_dtype, b_major="n")
    assert err == 0
    ref = run_oracle(inp, d_dtype)
    vm = inp["valid_m"]
    assert_close(values(d[:vm]), ref["D"][:vm], ORC_DT[d_dtype], "D_row")
    assert torch.all(torch.isnan(d[vm:]))
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, "dprob")
    for g, c in enumerate(counts):
        if c == 0:
            assert amax[g] == 0.0
        else:
            assert abs(amax[g].item() - ref["amax"][g]) <= 1e-3 * ref["amax"][g]
