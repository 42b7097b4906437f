"""gg_wgrad_noalloc (the wgrad entry on the library's static scratch, for
callers that cannot allocate) against gg_wgrad with a caller workspace
(GPU, through the C ABI).

Both run the same kernels, so their outputs must agree bit for bit.  The
calls come in a row on one GPU, each later one on a smaller problem than the
first, so each must clear and rewrite the scratch the previous one left
behind: the work-queue counters and the expert order.  The first call
covers an MoE-like shape with Zipf-skewed token counts (empty experts
included) and pointer outputs; later ones overwrite and accumulate into
dense bf16 / fp32 outputs with both A majors.
"""
import numpy as np
import pytest
import torch

from moe_grouped_gemm_offset_amd import synth
from tests.parity_util import say

pytestmark = pytest.mark.gpu


def gg():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def both(b, inp, out_dtype, accumulate=False, pointers=False, seed=0):
    """(gg_wgrad result, gg_wgrad_noalloc result) for the same inputs."""
    E = len(inp["counts"])
    h, i, T = inp["hidden"], inp["inter"], inp["tokens_sum"]
    am = b.GG_MAJOR_K if inp["a_major"] == "k" else b.GG_MAJOR_M
    bm = b.GG_MAJOR_N if inp["b_major"] == "n" else b.GG_MAJOR_K
    args = (inp["a"], am, inp["b"], bm, inp["offsets"], T, h, i)
    init = synth.wgrad_initial(E, h, i, out_dtype, seed=seed, device="cuda")
    res = []
    for fn in (b.gg_wgrad, b.gg_wgrad_noalloc):
        if pointers:
            outs = [init[e].clone() if accumulate else torch.empty(h, i, dtype=out_dtype, device="cuda")
                    for e in range(E)]
            ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device="cuda")
            fn(*args, wgrad_ptrs=ptrs, wgrad_dtype=b._TORCH_DTYPE[out_dtype], accumulate=accumulate)
            torch.cuda.synchronize()
            res.append(torch.stack(outs))
        else:
            out = init.clone() if accumulate else torch.full((E, h, i), float("nan"), dtype=out_dtype,
                                                             device="cuda")
            fn(*args, wgrad_dense=out, accumulate=accumulate)
            torch.cuda.synchronize()
            res.append(out)
    return res


def same(x, y):
    return torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                       y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


def test_noalloc_matches_workspace_entry():
    b = gg()
    # first call: 48 experts, 16384 Zipf(1.2) tokens, hidden 1024, intermediate
    # 512, M-major A, fp32 pointer outputs, overwrite
    counts = synth.zipf_groups(16384, 48, 1.2, seed=41)
    assert (counts == 0).any()
    inp = synth.wgrad_inputs(1024, 512, counts, a_major="m", b_major="n", seed=41, device="cuda")
    say("noalloc call 1: 48 experts, counts", (counts // 256).tolist())
    ref, got = both(b, inp, torch.float32, pointers=True)
    assert same(ref, got)
    # later calls, each smaller than the first
    cases = [
        ([256, 0, 512, 256], 256, 256, "k", torch.bfloat16, False),
        ([512, 256, 0], 512, 256, "m", torch.float32, True),
        ([256], 256, 512, "k", torch.bfloat16, True),
    ]
    for n, (cnt, h, i, am, dt, acc) in enumerate(cases):
        say(f"noalloc call {n + 2}: counts {cnt}, hidden {h}, inter {i}, A {am}-major, {dt}, "
            f"{'accumulate' if acc else 'overwrite'}")
        inp = synth.wgrad_inputs(h, i, cnt, a_major=am, b_major="n", seed=50 + n, device="cuda")
        ref, got = both(b, inp, dt, accumulate=acc, seed=60 + n)
        assert same(ref, got)
        if not acc:
            for e, c in enumerate(cnt):
                if c == 0:
                    assert torch.all(got[e] == 0)


def test_noalloc_validates_offsets():
    """With GG_FLAG_VALIDATE_OFFSETS the entry rejects malformed offsets on
    the host (its device error word is not readable) and leaves the output
    untouched."""
    b = gg()
    inp = synth.wgrad_inputs(256, 256, [256] * 4, seed=70, device="cuda")
    out = torch.full((4, 256, 256), float("nan"), dtype=torch.float32, device="cuda")
    bad = torch.tensor([512, 256, 768, 1024], dtype=torch.int32, device="cuda")
    with pytest.raises(b.GGError) as ex:
        b.gg_wgrad_noalloc(inp["a"], b.GG_MAJOR_K, inp["b"], b.GG_MAJOR_N, bad, 1024, 256, 256,
                           wgrad_dense=out, flags=b.GG_FLAG_VALIDATE_OFFSETS)
    assert ex.value.status == 11
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(out))
