"""Pins of the oracle's grouped wgrad (no GPU).

"Grouped GEMM + WGrad (Unified)", section "Operation": expert e contracts over
its token slice [begin, end) with begin = offsets[e-1] (0 for e = 0) and
end = offsets[e]; accumulate adds to the existing output, overwrite replaces
it and an empty expert gives zero.  Section "BF16 contract" fixes the strides
of the K-/M-major A and K-/N-major B.

The oracle is pinned against (i) an independent numpy formulation with token
masks, (ii) numpy.matmul for one expert, (iii) the invariant that the experts
sum to the dense product, (iv) exact-integer inputs, (v) the empty-expert and
accumulate rules.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth


def logical(inp):
    """Logical A (hidden, T) and B (T, inter) as float64 via torch's cast."""
    a = inp["a"].double().numpy()
    b = inp["b"].double().numpy()
    A = a if inp["a_major"] == "k" else a.T
    B = b if inp["b_major"] == "n" else b.T
    return A, B


def run(inp, **kw):
    return orc.wgrad(synth.bits(inp["a"]), 0 if inp["a_major"] == "k" else 1,
                     synth.bits(inp["b"]), 0 if inp["b_major"] == "k" else 1,
                     inp["offsets"].numpy(), inp["hidden"], inp["inter"],
                     inp["tokens_sum"], **kw)


@pytest.mark.parametrize("a_major", ["k", "m"])
@pytest.mark.parametrize("b_major", ["k", "n"])
@pytest.mark.parametrize("counts", [[7], [3, 0, 5], [0, 4, 1, 0, 6]])
def test_masked_formulation(a_major, b_major, counts):
    inp = synth.wgrad_inputs(12, 10, counts, a_major, b_major, seed=11)
    exact, _ = run(inp)
    A, B = logical(inp)
    T = inp["tokens_sum"]
    ends = np.cumsum(counts)
    starts = ends - np.asarray(counts)
    want = np.zeros_like(exact)
    for e in range(len(counts)):
        mask = np.zeros(T)
        mask[starts[e]:ends[e]] = 1.0
        want[e] = np.einsum("ht,t,ti->hi", A, mask, B)
    np.testing.assert_allclose(exact, want, rtol=1e-12, atol=1e-12)


def test_single_expert_is_matmul():
    inp = synth.wgrad_inputs(33, 17, [40], "m", "n", seed=12)
    exact, _ = run(inp)
    A, B = logical(inp)
    np.testing.assert_allclose(exact[0], A @ B, rtol=1e-12, atol=1e-12)


def test_experts_sum_to_dense_product():
    inp = synth.wgrad_inputs(16, 24, [5, 0, 9, 2, 0, 8], "k", "k", seed=13)
    exact, _ = run(inp)
    A, B = logical(inp)
    np.testing.assert_allclose(exact.sum(0), A @ B, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("dtype", [orc.F32, orc.BF16, orc.F16])
def test_exact_integers(dtype):
    # values in [-2, 2] over <= 64 tokens: every partial sum is an integer
    # of magnitude <= 256, exact in double and in every output dtype.
    inp = synth.wgrad_inputs(8, 8, [16, 0, 32, 16], "k", "n", seed=14, ints=True)
    exact, res = run(inp, out_dtype=dtype)
    A, B = logical(inp)
    assert np.all(exact == np.round(exact))
    got = orc.decode_array(res, dtype)
    assert np.array_equal(got, exact)
    assert np.array_equal(exact[2], A[:, 16:48] @ B[16:48, :])


@pytest.mark.parametrize("dtype", [orc.F32, orc.BF16])
def test_empty_expert_and_accumulate(dtype):
    counts = [8, 0, 16, 8]
    inp = synth.wgrad_inputs(8, 8, counts, "k", "n", seed=15, ints=True)
    tdt = {orc.F32: torch.float32, orc.BF16: torch.bfloat16}[dtype]
    old = synth.bits(synth.wgrad_initial(4, 8, 8, tdt, seed=16))
    ex_ow, ow = run(inp, out_dtype=dtype)
    ex_acc, acc = run(inp, out_dtype=dtype, accumulate=True, old=old)
    # overwrite: the empty expert is exactly zero
    assert np.all(orc.decode_array(ow[1], dtype) == 0.0)
    # accumulate: the empty expert's slice is left bit-identical
    assert np.array_equal(acc[1], old[1])
    # accumulate onto zeros equals overwrite bit-exactly
    zeros = np.zeros_like(old)
    _, acc0 = run(inp, out_dtype=dtype, accumulate=True, old=zeros)
    assert np.array_equal(acc0, ow)
    # accumulate adds exactly the overwrite result (in double)
    np.testing.assert_array_equal(ex_acc - orc.decode_array(old, dtype), ex_ow)
    if dtype == orc.F32:
        # x + x is exact in fp32: accumulating onto the overwrite result
        # doubles it bit-exactly
        _, twice = run(inp, out_dtype=dtype, accumulate=True, old=ow)
        assert np.array_equal(twice, (2.0 * ow.astype(np.float64)).astype(np.float32))


def test_row_sampling_matches_full():
    inp = synth.wgrad_inputs(20, 6, [4, 4, 0, 8], "m", "n", seed=17)
    full, _ = run(inp)
    rows = np.array([19, 0, 7], np.int32)
    part, _ = run(inp, hrows=rows)
    assert np.array_equal(part, full[:, rows, :])
