"""Pins of the oracle's grouped block-scaled (MXFP8) dgrad + dGLU (no GPU).

"Grouped GEMM + dGLU (SM100)", "Block-scaled contract / Equations": the
contraction R_g = alpha_g^2 * sum_k deq(A[m,k]) deq(B_g[n,k]) takes E4M3
codes times the E8M0 scale of their 32-value K block, and the dSwiGLU /
dGeGLU epilogue of the BF16 contract follows; "Shapes" gives the amax of a
bf16/fp16 output the shape (L, 2, 1), read here as max |D| over the input
gradient columns (index 0) and over the gate gradient columns (index 1) of
each expert's rows.

Pinned by:
* unit scales and integer values (exact in E4M3 and in bf16) reducing the op
  to the BF16-contract oracle, whose own pins tie it to finite differences;
* finite differences of the forward f = sum_n prob * R * act(gate, input),
  with R from a library matmul of torch-decoded, scale-expanded operands;
* the exact scale-shift invariance: adding j to every scale byte of a row of
  A multiplies that row of D, and its dprob, by 2^j;
* amax equal to the maxima of |D| over the two column sets of each group,
  with the sets swapping under gate-first, and over the listed rows only.

dSiTU-GLU (the page's "Equations": T_g = b1 tanh(G/b1) sigmoid(G),
T_u = b2 tanh(U/b2); gradients R prob T_u dT_g/dG and R prob T_g dT_u/dU,
dprob the row sum of R T_g T_u) is pinned by finite differences of
f = sum prob R T_g T_u, by its limit b1, b2 -> infinity, where T_g -> SiLU(G)
and T_u -> U make it dSwiGLU, and by the oddness of T_u (negating every
input negates the gate gradient and dprob and leaves the input gradient).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth

GA, LO, CLO, CHI = 1.702, 1.0, -7.0, 7.0


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def act_swiglu(g, u):
    return g * sig(g) * u


def act_geglu(g, u):
    gc = np.minimum(g, CHI)
    uc = np.clip(u, CLO, CHI)
    return gc * sig(GA * gc) * (uc + LO)


def column_maps(N, gate_first=False):
    n = np.arange(N)
    p, j = n // 32, n % 32
    cin = 64 * p + (32 if gate_first else 0) + j
    cgt = 64 * p + (0 if gate_first else 32) + j
    return cin, cgt


def run(inp, **kw):
    cdt = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16}[inp["c"].dtype]
    return orc.dglu_mx(synth.bits(inp["a"]), synth.bits(inp["sfa"]), inp["M"], inp["K"],
                       [synth.bits(b) for b in inp["b_list"]],
                       [synth.bits(s) for s in inp["sfb_list"]], inp["N"],
                       synth.bits(inp["c"]), cdt, inp["padded_offsets"].numpy(),
                       inp["alpha"].numpy(), inp["beta"].numpy(), inp["prob"].numpy(), **kw)


def small(seed, counts=(5, 0, 3, 4), N=64, K=96, m_extra=2, spread=3, c_std=2.0, **kw):
    inp = synth.dglu_mx_inputs(len(counts), K, N, counts, c_std=c_std, c_dtype=torch.float32,
                               m_extra=m_extra, seed=seed, scale_spread=spread, **kw)
    inp["beta"] = torch.ones_like(inp["beta"])   # X = C exactly
    return inp


def library_R(inp):
    """R (M, N) via numpy matmuls of torch-decoded, scale-expanded operands."""
    def deq(q, s):
        v = q.float().double().numpy()
        return v * np.repeat(np.exp2(s.double().numpy() - 127.0), 32, axis=1)
    A = deq(inp["a"], inp["sfa"])
    R = np.zeros((inp["M"], inp["N"]))
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        B = deq(inp["b_list"][g], inp["sfb_list"][g])
        al = float(inp["alpha"][g])
        R[start:start + cnt] = (al * al) * (A[start:start + cnt] @ B.T)
        start += cnt
    return R


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU])
def test_unit_scales_reduce_to_bf16_contract(act):
    """Integer operands in [-2, 2] with every scale byte 127: deq is the
    integer itself, so the block-scaled op must equal the BF16 contract on
    the same integers, bit for bit (all products and sums are exact)."""
    inp = small(71, ints=True, spread=0, c_std=4.0)
    ones = lambda s: torch.full_like(s, 127)
    inp["a"] = inp["a"].float().mul(torch.exp2(inp["sfa"].float() - 127).repeat_interleave(32, 1)) \
        .to(torch.float8_e4m3fn)
    inp["b_list"] = [b.float().mul(torch.exp2(s.float() - 127).repeat_interleave(32, 1))
                     .to(torch.float8_e4m3fn) for b, s in zip(inp["b_list"], inp["sfb_list"])]
    inp["sfa"] = ones(inp["sfa"])
    inp["sfb_list"] = [ones(s) for s in inp["sfb_list"]]
    assert set(np.unique(inp["a"].float().numpy())) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    L, N = inp["L"], inp["N"]
    dbias_in = np.zeros((L, 2 * N), np.uint16)
    mx = run(inp, act=act, dbias_in=dbias_in)
    ref = orc.dglu(synth.bits(inp["a"].float().to(torch.bfloat16)), inp["M"], inp["K"],
                   [synth.bits(b.float().to(torch.bfloat16)) for b in inp["b_list"]], 0, N,
                   synth.bits(inp["c"]), orc.F32, inp["padded_offsets"].numpy(),
                   inp["alpha"].numpy(), inp["beta"].numpy(), inp["prob"].numpy(),
                   act=act, dbias_in=dbias_in)
    assert np.array_equal(mx["D"], ref["D"])
    assert np.array_equal(mx["dprob"], ref["dprob"])
    assert np.array_equal(mx["dbias"], ref["dbias"])
    assert np.any(mx["D"] != 0)


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU])
def test_finite_differences(act):
    inp = small(72, c_std=4.0 if act == orc.DGEGLU else 2.0)
    out = run(inp, act=act, mask_filter=True)
    R = library_R(inp)
    X = inp["c"].double().numpy()
    prob = inp["prob"].double().numpy()
    N = inp["N"]
    cin, cgt = column_maps(N)
    f = act_swiglu if act == orc.DSWIGLU else act_geglu
    checked = 0
    for m in range(inp["valid_m"]):
        for n in range(N):
            g, u = X[m, cgt[n]], X[m, cin[n]]
            for which, x0, col in (("g", g, cgt[n]), ("u", u, cin[n])):
                h = 1e-5 * max(1.0, abs(x0))
                if act == orc.DGEGLU and (abs(x0 - CHI) < 10 * h or abs(x0 - CLO) < 10 * h):
                    continue
                if which == "g":
                    fd = (f(g + h, u) - f(g - h, u)) / (2 * h)
                else:
                    fd = (f(g, u + h) - f(g, u - h)) / (2 * h)
                want = prob[m] * R[m, n] * fd
                got = out["D"][m, col]
                assert abs(got - want) <= 1e-6 * max(abs(want), abs(prob[m] * R[m, n]), 1e-12), \
                    (m, n, which, got, want)
                checked += 1
        want_dp = np.sum(R[m] * f(X[m, cgt], X[m, cin]))
        assert abs(out["dprob"][m] - want_dp) <= 1e-9 * max(1.0, np.sum(np.abs(R[m]))), m
    assert checked > 1000
    # rows past valid_m and their dprob are untouched
    vm = inp["valid_m"]
    assert np.all(out["D"][vm:] == 0) and np.all(out["dprob"][vm:] == 0)


def test_scales_vary():
    inp = small(72)
    s = inp["sfa"].numpy()
    assert len(np.unique(s)) >= 5


@pytest.mark.parametrize("j", [-3, 5])
def test_scale_shift_invariance(j):
    inp = small(73)
    base = run(inp, act=orc.DSWIGLU)
    row = 6   # a row of group 2 (counts 5, 0, 3, 4)
    sfa = inp["sfa"].clone()
    sfa[row] = (sfa[row].int() + j).to(torch.uint8)
    shifted = run(dict(inp, sfa=sfa), act=orc.DSWIGLU)
    assert np.array_equal(shifted["D"][row], base["D"][row] * 2.0 ** j)
    assert shifted["dprob"][row] == base["dprob"][row] * 2.0 ** j
    others = np.arange(inp["M"]) != row
    assert np.array_equal(shifted["D"][others], base["D"][others])


@pytest.mark.parametrize("gate_first", [False, True])
@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU])
def test_amax_halves(gate_first, act):
    inp = small(74, c_std=4.0)
    out = run(inp, act=act, gate_first=gate_first)
    D = out["D"]
    cin, cgt = column_maps(inp["N"], gate_first)
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        blk = np.abs(D[start:start + cnt])
        want_in = blk[:, cin].max() if cnt else 0.0
        want_gt = blk[:, cgt].max() if cnt else 0.0
        assert out["amax"][g, 0] == want_in and out["amax"][g, 1] == want_gt, g
        start += cnt
    assert out["amax"][1, 0] == 0 and out["amax"][1, 1] == 0   # empty group
    assert np.all(out["amax"][[0, 2, 3]] > 0)


def test_amax_over_listed_rows():
    inp = small(75)
    full = run(inp)
    rows = np.array([0, 4, 8, 11], np.int64)
    part = run(inp, rows=rows)
    assert np.array_equal(part["D"], full["D"][rows])
    cin, cgt = column_maps(inp["N"])
    starts = np.concatenate([[0], np.cumsum(inp["counts"])[:-1]])
    for g, (s, c) in enumerate(zip(starts, inp["counts"])):
        sel = [r for r in rows if s <= r < s + c]
        if not sel:
            assert np.all(part["amax"][g] == 0)
            continue
        blk = np.abs(full["D"][sel])
        assert part["amax"][g, 0] == blk[:, cin].max()
        assert part["amax"][g, 1] == blk[:, cgt].max()


def act_situ(g, u, b1=4.0, b2=25.0):
    return b1 * np.tanh(g / b1) * sig(g) * (b2 * np.tanh(u / b2))


def test_situ_finite_differences():
    inp = small(76, c_std=4.0)
    out = run(inp, act=orc.DSITUGLU)
    R = library_R(inp)
    X = inp["c"].double().numpy()
    prob = inp["prob"].double().numpy()
    N = inp["N"]
    cin, cgt = column_maps(N)
    checked = 0
    for m in range(inp["valid_m"]):
        for n in range(N):
            g, u = X[m, cgt[n]], X[m, cin[n]]
            for which, x0, col in (("g", g, cgt[n]), ("u", u, cin[n])):
                h = 1e-5 * max(1.0, abs(x0))
                if which == "g":
                    fd = (act_situ(g + h, u) - act_situ(g - h, u)) / (2 * h)
                else:
                    fd = (act_situ(g, u + h) - act_situ(g, u - h)) / (2 * h)
                want = prob[m] * R[m, n] * fd
                got = out["D"][m, col]
                assert abs(got - want) <= 1e-6 * max(abs(want), abs(prob[m] * R[m, n]), 1e-12), \
                    (m, n, which, got, want)
                checked += 1
        want_dp = np.sum(R[m] * act_situ(X[m, cgt], X[m, cin]))
        assert abs(out["dprob"][m] - want_dp) <= 1e-9 * max(1.0, np.sum(np.abs(R[m]))), m
    assert checked > 1000


def test_situ_large_scales_reduce_to_dswiglu():
    inp = small(77)
    situ = run(inp, act=orc.DSITUGLU, situ_beta1=1e7, situ_beta2=1e7)
    swi = run(inp, act=orc.DSWIGLU)
    vm = inp["valid_m"]
    np.testing.assert_allclose(situ["D"][:vm], swi["D"][:vm], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(situ["dprob"][:vm], swi["dprob"][:vm], rtol=1e-9, atol=1e-12)


def test_situ_input_oddness():
    inp = small(78)
    N = inp["N"]
    cin, cgt = column_maps(N)
    base = run(inp, act=orc.DSITUGLU)
    c = inp["c"].clone()
    c[:, cin] = -c[:, cin]
    flip = run(dict(inp, c=c), act=orc.DSITUGLU)
    vm = inp["valid_m"]
    assert np.array_equal(flip["D"][:vm][:, cgt], -base["D"][:vm][:, cgt])
    assert np.array_equal(flip["D"][:vm][:, cin], base["D"][:vm][:, cin])
    assert np.array_equal(flip["dprob"][:vm], -base["dprob"][:vm])
