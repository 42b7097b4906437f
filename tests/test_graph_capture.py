"""GPU: every entry point can be captured into a HIP graph and replayed.

The library allocates nothing and issues no memset: the per-call set-up
(error word, work-queue counters of the persistent wgrad kernel, dbias and
amax accumulators) is a kernel of its own, so a captured call replays its
whole sequence.  Each graph is replayed three times, with eager work and a
synchronisation between replays, and every replay is checked against the
eager result of the same call: bit for bit where the kernels are
deterministic (wgrad outputs, D_row, amax), to the parity tolerance where
rows are summed with atomics in varying order (dprob, dbias).
"""
import numpy as np
import pytest
import torch

from moe_grouped_gemm_offset_amd import synth
from tests.parity_util import normwise, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def lib():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def capture(fn):
    """fn() once eagerly (warm-up on a side stream, as graph capture wants),
    then captured; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def eager_noise():
    x = torch.randn(1 << 20, device="cuda")
    (x * 2.0).sum().item()
    torch.cuda.synchronize()


def test_wgrad_graph_replays():
    b = lib()
    counts = np.array([512, 0, 256, 768, 256], np.int64)
    inp = synth.wgrad_inputs(512, 768, counts, "m", "n", seed=61, device="cuda")
    E = len(counts)
    out = torch.empty(E, 512, 768, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(b.gg_wgrad_workspace_size(E), dtype=torch.uint8, device="cuda")

    def call():
        b.gg_wgrad(inp["a"], b.GG_MAJOR_M, inp["b"], b.GG_MAJOR_N, inp["offsets"],
                   inp["tokens_sum"], 512, 768, wgrad_dense=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = capture(call)
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        say("wgrad replay", r)
        assert torch.equal(out, want), f"replay {r} differs from the eager call"
        assert b.gg_device_error(ws) == 0


def test_dglu_graph_replays():
    b = lib()
    d = synth.dglu_inputs(4, 256, 256, [256, 512, 0, 256], c_std=4.0, seed=62, device="cuda")
    M, N, L = d["M"], d["N"], d["L"]
    dr = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    dp = torch.zeros(M, dtype=torch.float32, device="cuda")
    db = torch.zeros(L, 2 * N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(b.gg_dglu_workspace_size(L, N, 1), dtype=torch.uint8, device="cuda")

    def call():
        b.gg_dglu(d["a"], d["b_dense"], None, b.GG_MAJOR_K, N, d["c"], d["padded_offsets"],
                  d["alpha"], d["beta"], d["prob"], dr, dp, db, act=b.GG_DGEGLU, workspace=ws)

    call()
    torch.cuda.synchronize()
    want_d, want_p, want_b = dr.clone(), dp.clone(), db.clone()
    dp.zero_()
    db.zero_()
    g = capture(call)                       # its warm-up call accumulated again
    for r in range(REPLAYS):
        dr.fill_(float("nan"))
        dp.zero_()
        db.zero_()
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        say("dglu replay", r)
        assert torch.equal(dr, want_d), f"replay {r}: D_row differs"
        assert normwise(dp.double().cpu().numpy(), want_p.double().cpu().numpy()) <= 1e-6
        assert normwise(db.double().cpu().numpy(), want_b.double().cpu().numpy()) <= 1e-2
        assert b.gg_device_error(ws) == 0


def test_dsrelu_graph_replays():
    b = lib()
    s = synth.dsrelu_inputs(2, 256, 256, [256, 512], seed=63, device="cuda")
    M = s["padded_offsets"][-1].item()
    dr = torch.empty(M, 256, dtype=torch.bfloat16, device="cuda")
    dp = torch.zeros(M, dtype=torch.float32, device="cuda")
    am = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(b.gg_dsrelu_workspace_size(2), dtype=torch.uint8, device="cuda")

    def call():
        b.gg_dsrelu(s["a"].view(torch.uint8), s["sfa"], s["b_dense"].view(torch.uint8),
                    s["sfb_dense"], None, None, 256, s["c"], s["padded_offsets"], s["alpha"],
                    s["prob"], dr, dp, am, workspace=ws)

    call()
    torch.cuda.synchronize()
    want_d, want_p, want_a = dr.clone(), dp.clone(), am.clone()
    g = capture(call)
    for r in range(REPLAYS):
        dr.fill_(float("nan"))
        dp.zero_()
        am.fill_(-1.0)
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        say("dsrelu replay", r)
        assert torch.equal(dr, want_d), f"replay {r}: D_row differs"
        assert torch.equal(am, want_a), f"replay {r}: amax differs"
        assert normwise(dp.double().cpu().numpy(), want_p.double().cpu().numpy()) <= 1e-6
        assert b.gg_device_error(ws) == 0


def test_wgrad_mx_graph_replays():
    b = lib()
    counts = np.array([256, 512, 0, 256], np.int64)
    inp = synth.wgrad_mx_inputs(256, 512, counts, seed=64, device="cuda")
    E = len(counts)
    out = torch.empty(E, 256, 512, dtype=torch.float32, device="cuda")
    ws = torch.empty(b.gg_wgrad_workspace_size(E), dtype=torch.uint8, device="cuda")

    def call():
        b.gg_wgrad_mx(inp["a"].view(torch.uint8), inp["sfa"], inp["b"].view(torch.uint8),
                      inp["sfb"], inp["offsets"], inp["tokens_sum"], 256, 512, wgrad_dense=out,
                      workspace=ws)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = capture(call)
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        say("wgrad_mx replay", r)
        assert torch.equal(out, want), f"replay {r} differs from the eager call"


def test_dglu_mx_graph_replays():
    b = lib()
    x = synth.dglu_mx_inputs(2, 256, 64, [256, 512], seed=65, discrete=True, device="cuda")
    M = x["padded_offsets"][-1].item()
    bl = [t.view(torch.uint8) for t in x["b_list"]]
    bp = torch.tensor([t.data_ptr() for t in bl], dtype=torch.int64, device="cuda")
    sp = torch.tensor([t.data_ptr() for t in x["sfb_list"]], dtype=torch.int64, device="cuda")
    dr = torch.empty(M, 128, dtype=torch.bfloat16, device="cuda")
    dp = torch.zeros(M, dtype=torch.float32, device="cuda")
    am = torch.empty(2, 2, dtype=torch.float32, device="cuda")
    ws = torch.empty(b.gg_dglu_workspace_size(2, 64, 0), dtype=torch.uint8, device="cuda")

    def call():
        b.gg_dglu_mx(x["a"].view(torch.uint8), x["sfa"], None, None, bp, sp, 64, x["c"],
                     x["padded_offsets"], x["alpha"], x["beta"], x["prob"], dr, dp, amax=am,
                     workspace=ws)

    call()
    torch.cuda.synchronize()
    want_d, want_p, want_a = dr.clone(), dp.clone(), am.clone()
    g = capture(call)
    for r in range(REPLAYS):
        dr.fill_(float("nan"))
        dp.zero_()
        am.fill_(-1.0)
        eager_noise()
        g.replay()
        torch.cuda.synchronize()
        say("dglu_mx replay", r)
        assert torch.equal(dr, want_d), f"replay {r}: D_row differs"
        assert torch.equal(am, want_a), f"replay {r}: amax differs"
        assert normwise(dp.double().cpu().numpy(), want_p.double().cpu().numpy()) <= 1e-6
        assert b.gg_device_error(ws) == 0
