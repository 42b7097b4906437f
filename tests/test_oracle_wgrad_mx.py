"""Pins of the oracle's block-scaled (MXFP8) grouped wgrad (no GPU).

"Grouped GEMM + WGrad (Unified)", "Operation" and "Block-scaled contract":
Wgrad[e] = A[:, begin:end] @ B[begin:end, :] on dequantized operands, with
one E8M0 scale per 32 tokens (the reduction axis) of every row of A (hidden,
T) and of B stored K-major as (inter, T).

Pinned by:
* integer operands with unit scales equal to the BF16 oracle bit for bit
  (whose own pins tie it to numpy and to the A @ B identity);
* a library matmul of torch-decoded, scale-expanded operands per expert;
* the sum over experts equal to the ungrouped product, an empty expert zero;
* exact scale shifts: j added to every scale of a row of A (of B) multiplies
  that row (column) of every expert's result by 2^j; j added to one 32-token
  scale block changes only the expert that owns those tokens.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth


def run(inp, **kw):
    return orc.wgrad_mx(synth.bits(inp["a"]), synth.bits(inp["sfa"]), synth.bits(inp["b"]),
                        synth.bits(inp["sfb"]), inp["offsets"].numpy(), inp["hidden"],
                        inp["inter"], inp["tokens_sum"], **kw)


def deq(q, s):
    return q.float().double().numpy() * np.repeat(np.exp2(s.double().numpy() - 127.0), 32, axis=1)


def small(seed, counts=(64, 0, 96, 32), hidden=24, inter=40, spread=3, **kw):
    return synth.wgrad_mx_inputs(hidden, inter, counts, seed=seed, scale_spread=spread, **kw)


def test_unit_scales_reduce_to_bf16():
    inp = small(91, ints=True, spread=0)
    a = deq(inp["a"], inp["sfa"])
    b = deq(inp["b"], inp["sfb"])
    assert set(np.unique(a)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    inp["a"] = torch.from_numpy(a).float().to(torch.float8_e4m3fn)
    inp["b"] = torch.from_numpy(b).float().to(torch.float8_e4m3fn)
    inp["sfa"] = torch.full_like(inp["sfa"], 127)
    inp["sfb"] = torch.full_like(inp["sfb"], 127)
    exact, res = run(inp)
    a16 = synth.bits(torch.from_numpy(a).to(torch.bfloat16))
    b16 = synth.bits(torch.from_numpy(b).to(torch.bfloat16))
    ref_exact, ref_res = orc.wgrad(a16, 0, b16, 0, inp["offsets"].numpy(), inp["hidden"],
                                   inp["inter"], inp["tokens_sum"])
    assert np.array_equal(exact, ref_exact) and np.array_equal(res, ref_res)
    assert np.any(exact != 0)


def test_library_matmul_per_expert():
    inp = small(92)
    exact, res = run(inp)
    A, B = deq(inp["a"], inp["sfa"]), deq(inp["b"], inp["sfb"])
    start = 0
    for e, c in enumerate(inp["counts"]):
        want = A[:, start:start + c] @ B[:, start:start + c].T
        np.testing.assert_allclose(exact[e], want, rtol=1e-12, atol=1e-12 * np.abs(want).max(initial=1))
        start += c
    assert np.all(exact[1] == 0) and np.all(res[1] == 0), "an empty expert gives zero"
    np.testing.assert_allclose(exact.sum(0), A @ B.T, rtol=1e-12, atol=1e-9)


def test_scale_shifts():
    inp = small(93)
    base, _ = run(inp)
    sfa = inp["sfa"].clone()
    sfa[5] = (sfa[5].int() + 3).to(torch.uint8)
    got, _ = run(dict(inp, sfa=sfa))
    assert np.array_equal(got[:, 5], base[:, 5] * 8.0)
    assert np.array_equal(np.delete(got, 5, axis=1), np.delete(base, 5, axis=1))
    sfb = inp["sfb"].clone()
    sfb[7] = (sfb[7].int() - 2).to(torch.uint8)
    got, _ = run(dict(inp, sfb=sfb))
    assert np.array_equal(got[:, :, 7], base[:, :, 7] * 0.25)
    # one 32-token block (tokens 64..95: the first block of expert 2)
    sfb = inp["sfb"].clone()
    sfb[:, 2] = (sfb[:, 2].int() + 1).to(torch.uint8)
    got, _ = run(dict(inp, sfb=sfb))
    assert np.array_equal(got[[0, 1, 3]], base[[0, 1, 3]])
    assert not np.array_equal(got[2], base[2])


def test_accumulate_and_rows():
    inp = small(94)
    E, H, I = len(inp["counts"]), inp["hidden"], inp["inter"]
    old = synth.bits(synth.wgrad_initial(E, H, I, torch.float32, 5))
    exact, res = run(inp, out_dtype=orc.F32, accumulate=True, old=old)
    over, _ = run(inp)
    np.testing.assert_allclose(exact, over + old.astype(np.float64), rtol=0, atol=0)
    rows = np.array([0, 7, 23], np.int32)
    part, _ = run(inp, hrows=rows)
    assert np.array_equal(part, over[:, rows])


def test_ragged_relayout_is_data_movement():
    """to_ragged (the tensor_ragged storage used by the GPU tests) only moves
    values: expert e's block, read back with pitch counts[e], is the slice."""
    inp = small(95)
    flat = synth.to_ragged(inp["a"].view(torch.uint8), inp["counts"])
    start, off = 0, 0
    for c in inp["counts"]:
        blk = flat[off:off + inp["hidden"] * c].reshape(inp["hidden"], c)
        assert torch.equal(blk, inp["a"].view(torch.uint8)[:, start:start + c])
        start += c
        off += inp["hidden"] * c
    sflat = synth.to_ragged(inp["sfa"], inp["counts"], per=32)
    assert sflat.numel() == inp["sfa"].numel()
