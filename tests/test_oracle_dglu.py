"""Pins of the oracle's grouped dgrad + dSwiGLU / dGeGLU (no GPU).

"Grouped GEMM + dGLU (SM100)", "BF16 contract / Tensors, layouts, and
equation": R_g = alpha_g^2 A_g B_g^T and X_g = beta_g C_g over the rows of
group g; X is split into alternating 32-wide blocks; D holds the gradient
with respect to those blocks, dprob the row sum of R times the unscaled
activation, dbias the per-expert row reduction of D.

Pinned by:
* finite differences of the forward that these gradients belong to,
  f = sum_n prob * R * act(gate, input), with the textbook activations
  SwiGLU act = gate * sigmoid(gate) * input and the clamped GeGLU
  act = gc * sigmoid(1.702 gc) * (uc + 1) (gc = min(gate, 7),
  uc = clamp(input, -7, 7));
* a closed form that reduces the fused op to a library GEMM
  (beta = 1, gate = 0, input = 1: D_gate = prob * R / 2, D_input = 0,
  dprob = 0, dbias_gate = sum of prob * R / 2);
* layout invariants (dense vs discrete, K- vs N-major B, gate-first swap,
  beta folded into C).
The page's "value-bearing" GeGLU filters (the derivative times the raw value
inside the clamp) are pinned only by the page text: the test checks that the
value variant equals the mask variant times the raw value.
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


def logical_R(inp):
    """R (M, N) float64 from numpy matmuls of the logical operands."""
    A = inp["a"].double().numpy()
    M, N = inp["M"], inp["N"]
    R = np.zeros((M, N))
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        Bg = inp["b_list"][g].double().numpy()
        if inp["b_major"] == "n":
            Bg = Bg.T
        al = float(inp["alpha"][g])
        R[start:start + cnt] = (al * al) * (A[start:start + cnt] @ Bg.T)
        start += cnt
    return R


def column_maps(N, gate_first=False):
    n = np.arange(N)
    p, j = n // 32, n % 32
    cin = 64 * p + (32 if gate_first else 0) + j
    cgt = 64 * p + (0 if gate_first else 32) + j
    return cin, cgt


def run(inp, **kw):
    b_major = 0 if inp["b_major"] == "k" else 1
    cdt = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16}[inp["c"].dtype]
    return orc.dglu(synth.bits(inp["a"]), inp["M"], inp["K"],
                    [synth.bits(b) for b in inp["b_list"]], b_major, inp["N"],
                    synth.bits(inp["c"]), cdt, inp["padded_offsets"].numpy(),
                    inp["alpha"].numpy(), inp["beta"].numpy(), inp["prob"].numpy(), **kw)


def small(seed, c_std=2.0, counts=(5, 0, 3, 4), m_extra=2, N=64, K=24, **kw):
    inp = synth.dglu_inputs(len(counts), K, N, counts, a_std=0.3, b_std=0.3, c_std=c_std,
                            c_dtype=torch.float32, m_extra=m_extra, seed=seed, **kw)
    inp["beta"] = torch.ones_like(inp["beta"])   # X = C exactly
    return inp


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU])
def test_finite_differences(act):
    inp = small(21, c_std=4.0 if act == orc.DGEGLU else 2.0)
    out = run(inp, act=act, mask_filter=True)
    R = logical_R(inp)
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
        # f is linear in prob: d f / d prob = sum_n R * act
        want_dp = np.sum(R[m] * f(X[m, cgt], X[m, cin]))
        assert abs(out["dprob"][m] - want_dp) <= 1e-9 * max(1.0, np.sum(np.abs(R[m]))), m
    assert checked > 1000


def test_geglu_clamps_are_exercised():
    inp = small(21, c_std=4.0)
    X = inp["c"].double().numpy()[: inp["valid_m"]]
    assert np.mean(X > 7) > 0.02 and np.mean(X < -7) > 0.02


def test_geglu_value_filters_are_mask_times_raw():
    inp = small(22, c_std=4.0)
    val = run(inp, act=orc.DGEGLU)["D"]
    msk = run(inp, act=orc.DGEGLU, mask_filter=True)["D"]
    X = inp["c"].double().numpy()
    vm = inp["valid_m"]
    inside = (X[:vm] <= 7) & (X[:vm] >= -7)
    cin, cgt = column_maps(inp["N"])
    is_gate = np.zeros(X.shape[1], bool)
    is_gate[cgt] = True
    # a gate passes its filter whenever it is <= 7 (no lower bound)
    passes = np.where(is_gate[None, :], X[:vm] <= 7, inside)
    assert np.array_equal(val[:vm][passes], msk[:vm][passes] * X[:vm][passes])
    assert np.all(val[:vm][~passes] == 0) and np.all(msk[:vm][~passes] == 0)


@pytest.mark.parametrize("gate_first", [False, True])
def test_closed_form_gemm(gate_first):
    """beta = 1, gate = 0, input = 1: s = 1/2, so D_gate = prob R / 2,
    D_input = 0, dprob = 0 and dbias_gate[g] = sum_{m in g} prob R / 2."""
    inp = small(23)
    N, M, L = inp["N"], inp["M"], inp["L"]
    cin, cgt = column_maps(N, gate_first)
    c = torch.zeros(M, 2 * N)
    c[:, cin] = 1.0
    inp["c"] = c
    dbias_in = np.zeros((L, 2 * N), np.uint16)
    out = run(inp, gate_first=gate_first, dbias_in=dbias_in)
    R = logical_R(inp)
    prob = inp["prob"].double().numpy()
    vm = inp["valid_m"]
    np.testing.assert_allclose(out["D"][:vm][:, cgt], prob[:vm, None] * R[:vm] / 2,
                               rtol=1e-12, atol=1e-15)
    assert np.all(out["D"][:, cin] == 0)
    assert np.all(out["dprob"] == 0)
    # rows past valid_m are untouched
    assert np.all(out["D"][vm:] == 0)
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        want = 0.5 * (prob[start:start + cnt] @ R[start:start + cnt])
        np.testing.assert_allclose(out["dbias"][g][cgt], want, rtol=1e-12, atol=1e-15)
        assert np.all(out["dbias"][g][cin] == 0)
        start += cnt


def test_beta_scales_c_in_fp32():
    inp = small(24)
    inp["beta"] = synth.uniform((inp["L"],), 0.5, 1.5, torch.Generator().manual_seed(5), "cpu")
    a = run(inp, act=orc.DGEGLU)
    # fold beta into C with one fp32 product per element, beta = 1
    c = inp["c"].clone()
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        c[start:start + cnt] = (c[start:start + cnt] * inp["beta"][g]).float()
        start += cnt
    inp2 = dict(inp, c=c, beta=torch.ones_like(inp["beta"]))
    b = run(inp2, act=orc.DGEGLU)
    vm = inp["valid_m"]
    assert np.array_equal(a["D"][:vm], b["D"][:vm])
    assert np.array_equal(a["dprob"][:vm], b["dprob"][:vm])


def test_discrete_and_n_major_b_match_dense():
    inp = small(25)
    dense = run(inp, act=orc.DSWIGLU)
    inp_n = dict(inp, b_list=[b.t().contiguous() for b in inp["b_list"]], b_major="n")
    nmaj = run(inp_n, act=orc.DSWIGLU)
    assert np.array_equal(dense["D"], nmaj["D"])
    assert np.array_equal(dense["dprob"], nmaj["dprob"])


def test_gate_first_is_a_column_swap():
    inp = small(26)
    N = inp["N"]
    a = run(inp, act=orc.DSWIGLU)
    cin, cgt = column_maps(N)
    c = inp["c"].clone()
    c[:, cin], c[:, cgt] = inp["c"][:, cgt], inp["c"][:, cin]
    b = run(dict(inp, c=c), act=orc.DSWIGLU, gate_first=True)
    assert np.array_equal(a["D"][:, cin], b["D"][:, cgt])
    assert np.array_equal(a["D"][:, cgt], b["D"][:, cin])
    assert np.array_equal(a["dprob"], b["dprob"])


def test_accumulating_outputs_and_empty_group():
    inp = small(27)
    L, N = inp["L"], inp["N"]
    dbias_in = synth.bits(synth.normal((L, 2 * N), 1.0, torch.Generator().manual_seed(3), "cpu"))
    dprob_in = np.random.default_rng(4).standard_normal(inp["M"]).astype(np.float32)
    base = run(inp, act=orc.DSWIGLU, dbias_in=np.zeros((L, 2 * N), np.uint16))
    acc = run(inp, act=orc.DSWIGLU, dbias_in=dbias_in, dprob_in=dprob_in)
    np.testing.assert_array_equal(acc["dbias"], orc.decode_array(dbias_in, orc.BF16) + base["dbias"])
    np.testing.assert_array_equal(acc["dprob"], dprob_in.astype(np.float64) + base["dprob"])
    # group 1 is empty: its dbias stays what the caller passed
    assert np.all(base["dbias"][1] == 0)
    assert np.array_equal(acc["dbias_q"][1], dbias_in[1])


def test_row_sampling_matches_full():
    inp = small(28)
    full = run(inp, act=orc.DGEGLU)
    rows = np.array([11, 0, 5, 13], np.int64)
    part = run(inp, act=orc.DGEGLU, rows=rows)
    assert np.array_equal(part["D"], full["D"][rows])
    assert np.array_equal(part["dprob"], full["dprob"][rows])
