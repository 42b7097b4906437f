"""Calls queued on a caller-given stream, with the workspace left to the
binding and dropped by the caller at once (GPU).

The binding allocates such a workspace on the call's stream.  torch's
caching allocator ties a freed block to the stream it was allocated on, so
work queued afterwards on another stream cannot receive the block while the
call's kernels may still use it (for gg_wgrad it holds the work-queue
counters of the persistent kernel, for gg_dglu the dbias accumulators).
The tests check that a same-size allocation on the current stream gets a
different block, and that the side-stream results equal those of the same
call on the current stream.
"""
import pytest
import torch

from moe_grouped_gemm_offset_amd import synth

pytestmark = pytest.mark.gpu


def gg():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def test_wgrad_side_stream():
    b = gg()
    inp = synth.wgrad_inputs(256, 512, [256, 0, 512, 256], a_major="m", b_major="n", seed=91,
                             device="cuda")
    args = (inp["a"], b.GG_MAJOR_M, inp["b"], b.GG_MAJOR_N, inp["offsets"], inp["tokens_sum"], 256, 512)
    ref = torch.empty(4, 256, 512, dtype=torch.float32, device="cuda")
    b.gg_wgrad(*args, wgrad_dense=ref)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws = b.gg_wgrad(*args, wgrad_dense=out, stream=side)
    ptr, nbytes = ws.data_ptr(), ws.numel()
    del ws
    other = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert other.data_ptr() != ptr, "the dropped workspace went to the current stream"
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_dglu_side_stream_dbias():
    b = gg()
    inp = synth.dglu_inputs(3, 256, 320, [256, 512, 256], c_std=4.0, seed=92, device="cuda")
    M, N, L = inp["M"], inp["N"], inp["L"]

    def call(stream):
        d = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
        dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
        dbias = torch.zeros(L, 2 * N, dtype=torch.bfloat16, device="cuda")
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        ws = b.gg_dglu(inp["a"], inp["b_dense"], None, b.GG_MAJOR_K, N, inp["c"], inp["padded_offsets"],
                       inp["alpha"], inp["beta"], inp["prob"], d, dprob, dbias, act=b.GG_DGEGLU,
                       stream=stream)
        return d, dprob, dbias, ws

    ref = call(None)[:3]
    side = torch.cuda.Stream()
    d, dprob, dbias, ws = call(side)
    ptr, nbytes = ws.data_ptr(), ws.numel()
    del ws
    other = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert other.data_ptr() != ptr, "the dropped workspace went to the current stream"
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), ref[0].view(torch.int16))
    # dprob adds per-tile partial sums atomically, in no fixed order
    assert float((dprob - ref[1]).norm() / ref[1].norm()) <= 1e-6
    assert float((dbias.float() - ref[2].float()).norm() / ref[2].float().norm()) <= 2.0 ** -8
