"""GPU parity of gg_wgrad against the oracle (through the C ABI).

Cases span several 256x256 tiles, partial N tiles, ragged token counts
(multiples of 8, not of 64), empty experts, all four operand majors, the
three output dtypes, dense and pointer outputs, accumulate and overwrite;
plus the 256x256 / 4-expert workload in full and the MoE-scale workload
(hidden 4096, intermediate 2048, 64 Zipf experts) on sampled rows in the
launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from moe_grouped_gemm_offset_amd import synth
from tests.parity_util import TOL, assert_close, normwise, say, values

pytestmark = pytest.mark.gpu

MAJ = {"k": 0, "m": 1, "n": 2}


def gg():
    from moe_grouped_gemm_offset_amd import binding
    binding.load_library()
    return binding


def run_gpu(inp, out_dtype, accumulate=False, old=None, discrete=False, ragged=False,
            static=False):
    b = gg()
    E = len(inp["counts"])
    a, bb = inp["a"].cuda(), inp["b"].cuda()
    flags = b.GG_FLAG_STATIC_SCHED if static else 0
    if ragged:
        # tensor_ragged storage of the K-major operands (the others are
        # per-token rows either way)
        flags |= b.GG_FLAG_TENSOR_RAGGED
        if inp["a_major"] == "k":
            a = synth.to_ragged(a, inp["counts"])
        if inp["b_major"] == "k":
            bb = synth.to_ragged(bb, inp["counts"])
    off = inp["offsets"].cuda()
    h, i = inp["hidden"], inp["inter"]
    if discrete:
        outs = [torch.empty(h, i, dtype=out_dtype, device="cuda") for _ in range(E)]
        if accumulate:
            for e in range(E):
                outs[e].copy_(old[e])
        ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device="cuda")
        ws = b.gg_wgrad(a, MAJ[inp["a_major"]], bb, MAJ[inp["b_major"]], off, inp["tokens_sum"], h, i,
                        wgrad_ptrs=ptrs, wgrad_dtype=b._TORCH_DTYPE[out_dtype], accumulate=accumulate,
                        flags=flags)
        torch.cuda.synchronize()
        res = torch.stack(outs)
    else:
        res = old.clone().cuda() if accumulate else torch.full((E, h, i), float("nan"), dtype=out_dtype,
                                                               device="cuda")
        ws = b.gg_wgrad(a, MAJ[inp["a_major"]], bb, MAJ[inp["b_major"]], off, inp["tokens_sum"], h, i,
                        wgrad_dense=res, accumulate=accumulate, flags=flags)
        torch.cuda.synchronize()
    return res.cpu(), b.gg_device_error(ws)


def run_oracle(inp, out_dtype, accumulate=False, old=None, hrows=None):
    od = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16}[out_dtype]
    return orc.wgrad(synth.bits(inp["a"]), 0 if inp["a_major"] == "k" else 1, synth.bits(inp["b"]),
                     0 if inp["b_major"] == "k" else 1, inp["offsets"].numpy(), inp["hidden"],
                     inp["inter"], inp["tokens_sum"], out_dtype=od, accumulate=accumulate,
                     old=None if old is None else synth.bits(old), hrows=hrows), od


def compare(got, inp, out_dtype, accumulate=False, old=None, hrows=None, name=""):
    (exact, _), od = run_oracle(inp, out_dtype, accumulate, old, hrows)
    g = values(got if hrows is None else got[:, hrows, :])
    assert_close(g, exact, od, f"{name} all experts")
    for e, cnt in enumerate(inp["counts"]):
        if cnt == 0 and not accumulate:
            assert np.all(g[e] == 0), f"{name}: empty expert {e} not exactly zero"
        elif cnt == 0 and accumulate:
            want = values(old[e] if hrows is None else old[e][hrows])
            assert np.array_equal(g[e], want), f"{name}: empty expert {e} changed in accumulate mode"
        else:
            err = normwise(g[e], exact[e])
            assert err <= TOL[od], f"{name}: expert {e} normwise error {err:.3e}"


def test_small_workload_exact():
    """hidden 256, intermediate 256, counts [256, 0, 512, 256], fp32 dense,
    overwrite: the full output, expert 1 exactly zero."""
    w = synth.WORKLOADS["wgrad_small"]
    inp = synth.wgrad_inputs(w["hidden"], w["inter"], w["counts"], w["a_major"], w["b_major"],
                             seed=w["seed"])
    say("wgrad_small", w["counts"])
    got, err = run_gpu(inp, torch.float32)
    assert err == 0
    compare(got, inp, torch.float32, name="wgrad_small")


@pytest.mark.parametrize("a_major", ["k", "m"])
@pytest.mark.parametrize("b_major", ["k", "n"])
def test_majors_ragged(a_major, b_major):
    counts = [520, 0, 256, 72, 8, 320]
    inp = synth.wgrad_inputs(512, 384, counts, a_major, b_major, seed=41)
    say("ragged", a_major, b_major, counts)
    got, err = run_gpu(inp, torch.float32)
    assert err == 2  # GG_DEVERR_GRANULE: counts not multiples of 256 (still computed)
    compare(got, inp, torch.float32, name=f"{a_major}{b_major}")


@pytest.mark.parametrize("a_major", ["k", "m"])
@pytest.mark.parametrize("b_major", ["k", "n"])
def test_tensor_ragged(a_major, b_major):
    """GG_FLAG_TENSOR_RAGGED: K-major operands stored as per-expert
    K-contiguous blocks; the result is that of the tensor2d storage."""
    counts = [520, 0, 256, 72, 8, 320]
    inp = synth.wgrad_inputs(512, 384, counts, a_major, b_major, seed=46)
    say("tensor_ragged", a_major, b_major, counts)
    got, err = run_gpu(inp, torch.float32, ragged=True)
    assert err == 2  # GG_DEVERR_GRANULE only
    compare(got, inp, torch.float32, name=f"ragged {a_major}{b_major}")


def test_exact_integers_bit_exact():
    counts = [256, 512, 0, 256]
    inp = synth.wgrad_inputs(256, 320, counts, "m", "n", seed=42, ints=True)
    got, _ = run_gpu(inp, torch.float32)
    (exact, res), _ = run_oracle(inp, torch.float32)
    assert np.array_equal(got.numpy(), res), "integer-valued wgrad must be bit-exact"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("discrete", [False, True])
@pytest.mark.parametrize("accumulate", [False, True])
def test_outputs_and_modes(dtype, discrete, accumulate):
    counts = [256, 0, 768, 512]
    inp = synth.wgrad_inputs(320, 256, counts, "m", "n", seed=43)
    old = synth.wgrad_initial(len(counts), 320, 256, dtype, seed=44) if accumulate else None
    say("modes", dtype, "discrete" if discrete else "dense", "acc" if accumulate else "overwrite")
    got, err = run_gpu(inp, dtype, accumulate, old, discrete)
    assert err == 0
    compare(got, inp, dtype, accumulate, old, name=f"{dtype} {discrete} {accumulate}")


def test_tokens_sum_zero():
    inp = synth.wgrad_inputs(256, 256, [0, 0], "k", "n", seed=45)
    got, err = run_gpu(inp, torch.bfloat16)
    assert err == 0 and torch.all(got == 0)


@pytest.mark.parametrize("a_major", ["k", "m"])
def test_moe_scale_sampled(a_major):
    """The MoE-scale workload, bf16 dense output, on the device; the oracle
    checks sampled hidden rows of every expert."""
    w = synth.WORKLOADS["wgrad_moe"]
    counts = synth.workload_counts("wgrad_moe")
    inp = synth.wgrad_inputs(w["hidden"], w["inter"], counts, a_major, w["b_major"],
                             seed=w["seed"], device="cuda")
    say("wgrad_moe", a_major, "experts", len(counts), "empty", int(np.sum(counts == 0)))
    got, err = run_gpu(inp, torch.bfloat16)
    assert err == 0
    inp_cpu = dict(inp, a=inp["a"].cpu(), b=inp["b"].cpu(), offsets=inp["offsets"].cpu())
    rows = np.array([0, 1, 255, 256, 2047, 2048, 4000, 4095], np.int32)
    compare(got, inp_cpu, torch.bfloat16, hrows=rows, name="wgrad_moe")


def test_work_queues_many_items():
    """More work items than compute units, in a count that is no multiple
    of 8: 100 experts (some empty) on a 2 x 3 tile grid (hidden 512,
    intermediate 768: partial N tiles) give 600 items over the per-XCD
    queues of the persistent kernel.  A second call on the same workspace
    must give the same output (the set-up kernel resets the queues)."""
    rng = np.random.default_rng(47)
    counts = (rng.integers(0, 3, size=100) * 256).astype(np.int64)
    counts[[3, 50, 99]] = 0
    inp = synth.wgrad_inputs(512, 768, counts, "m", "n", seed=47)
    say("work queues", "experts", len(counts), "tokens", int(counts.sum()))
    b = gg()
    a, bb, off = inp["a"].cuda(), inp["b"].cuda(), inp["offsets"].cuda()
    ws = torch.empty(b.gg_wgrad_workspace_size(len(counts)), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        res = torch.full((len(counts), 512, 768), float("nan"), dtype=torch.bfloat16, device="cuda")
        b.gg_wgrad(a, MAJ["m"], bb, MAJ["n"], off, inp["tokens_sum"], 512, 768, wgrad_dense=res,
                   workspace=ws)
        torch.cuda.synchronize()
        assert b.gg_device_error(ws) == 0
        outs.append(res.cpu())
    assert torch.equal(outs[0], outs[1]), "second call on the same workspace differs"
    compare(outs[0], inp, torch.bfloat16, name="work queues")


@pytest.mark.parametrize("a_major", ["k", "m"])
@pytest.mark.parametrize("out", ["bf16_dense", "f32_discrete"])
def test_moe_scale_output_modes(a_major, out):
    """The MoE-scale workload into bf16 dense outputs or discrete per-expert
    fp32 outputs (separate allocations reached through the int64 pointer
    array): accumulate onto seeded N(0,1) values, then overwrite the same
    buffers.  Sampled hidden rows of every expert against the oracle; empty
    experts keep their old values bit for bit when accumulating and are
    exactly zero after the overwrite."""
    w = synth.WORKLOADS["wgrad_moe"]
    counts = synth.workload_counts("wgrad_moe")
    inp = synth.wgrad_inputs(w["hidden"], w["inter"], counts, a_major, w["b_major"],
                             seed=w["seed"], device="cuda")
    E, h, i = len(counts), w["hidden"], w["inter"]
    dt = torch.bfloat16 if out == "bf16_dense" else torch.float32
    init = synth.wgrad_initial(E, h, i, dt, seed=1003, device="cuda")
    say("wgrad_moe", a_major, out, "experts", E, "empty", int(np.sum(counts == 0)))
    b = gg()
    rows = np.array([0, 1, 255, 256, 2047, 2048, 4000, 4095], np.int32)
    inp_cpu = dict(inp, a=inp["a"].cpu(), b=inp["b"].cpu(), offsets=inp["offsets"].cpu())
    old = init.cpu()
    if out == "bf16_dense":
        res = init.clone()
        outs = None
    else:
        outs = [init[e].clone() for e in range(E)]
        ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device="cuda")
    for accumulate in (True, False):
        if outs is None:
            ws = b.gg_wgrad(inp["a"], MAJ[a_major], inp["b"], MAJ["n"], inp["offsets"],
                            inp["tokens_sum"], h, i, wgrad_dense=res, accumulate=accumulate)
        else:
            ws = b.gg_wgrad(inp["a"], MAJ[a_major], inp["b"], MAJ["n"], inp["offsets"],
                            inp["tokens_sum"], h, i, wgrad_ptrs=ptrs,
                            wgrad_dtype=b._TORCH_DTYPE[dt], accumulate=accumulate)
        torch.cuda.synchronize()
        assert b.gg_device_error(ws) == 0
        got = (res if outs is None else torch.stack(outs)).cpu()
        compare(got, inp_cpu, dt, accumulate, old if accumulate else None, hrows=rows,
                name=f"wgrad_moe {out} {'accumulate' if accumulate else 'overwrite'}")


@pytest.mark.parametrize("case", range(8))
def test_random_shapes(case):
    """Seeded random shapes through the persistent scheduler: hidden and
    intermediate multiples of 64 up to 1024 (partial tiles; expert grids of
    3-12 tiles, mostly not a multiple of 8, so the 1-D XCD remap, and one
    of 8 tiles on the 4 x 2 XCD blocks; 63-420 items), 1-40 experts with
    256-multiple counts (some empty), all majors and output dtypes, both
    modes; every element against the oracle.  (A grid of fewer than 8
    items is the 256 x 256, 4-expert workload above.)"""
    rng = np.random.default_rng(900 + case)
    h = int(rng.integers(1, 17)) * 64
    i = int(rng.integers(1, 17)) * 64
    E = int(rng.integers(1, 41))
    counts = (rng.integers(0, 4, size=E) * 256).astype(np.int64)
    if counts.sum() == 0:
        counts[0] = 256
    am, bm = ["k", "m"][case % 2], ["k", "n"][(case // 2) % 2]
    dt = [torch.bfloat16, torch.float16, torch.float32][case % 3]
    accumulate = bool(case % 4 == 3)
    inp = synth.wgrad_inputs(h, i, counts, am, bm, seed=900 + case)
    say("random shape", h, i, "experts", E, "tokens", int(counts.sum()), am, bm, dt, accumulate)
    old = synth.wgrad_initial(E, h, i, dt, seed=950 + case) if accumulate else None
    got, err = run_gpu(inp, dt, accumulate, old)
    assert err == 0
    compare(got, inp, dt, accumulate, old, name=f"random {case}")


@pytest.mark.parametrize("a_major,b_major,dtype,accumulate", [
    ("m", "n", torch.bfloat16, False),     # compile-time bf16 overwrite
    ("k", "n", torch.bfloat16, False),
    ("m", "n", torch.float32, True),       # compile-time fp32 accumulate
    ("k", "k", torch.float16, False),      # run-time format
    ("m", "n", torch.bfloat16, True),
])
def test_static_scheduling(a_major, b_major, dtype, accumulate):
    """GG_FLAG_STATIC_SCHED (the pages' use_dynamic_sched=False): the items
    are walked in a fixed order instead of taken from the work queues.  Each
    tile is computed the same way either way, so the output is bit-identical
    to the dynamic schedule's; the static one is also checked against the
    oracle.  600 items (100 experts, some empty, on a 2 x 3 tile grid) give
    every workgroup several."""
    rng = np.random.default_rng(48)
    counts = (rng.integers(0, 3, size=100) * 256).astype(np.int64)
    counts[[3, 50, 99]] = 0
    inp = synth.wgrad_inputs(512, 768, counts, a_major, b_major, seed=48)
    old = synth.wgrad_initial(len(counts), 512, 768, dtype, seed=49) if accumulate else None
    say("static scheduling", a_major, b_major, dtype, "acc" if accumulate else "overwrite")
    dyn, err_d = run_gpu(inp, dtype, accumulate, old)
    sta, err_s = run_gpu(inp, dtype, accumulate, old, static=True)
    assert err_d == 0 and err_s == 0
    assert torch.equal(dyn.view(torch.int16 if dtype != torch.float32 else torch.int32),
                       sta.view(torch.int16 if dtype != torch.float32 else torch.int32)), \
        "static and dynamic schedules differ"
    compare(sta, inp, dtype, accumulate, old, name="static")


@pytest.mark.parametrize("counts", [[256, 0, 512], [256, 256, 0, 512, 256, 0, 256]])
def test_static_scheduling_small_grid(counts):
    """Fewer items than 8 (a grid of one workgroup per item): each of them
    serves its queue alone, under both schedules."""
    inp = synth.wgrad_inputs(256, 256, counts, "m", "n", seed=50)
    say("static scheduling, small grid", counts)
    dyn, err_d = run_gpu(inp, torch.bfloat16)
    sta, err_s = run_gpu(inp, torch.bfloat16, static=True)
    assert err_d == 0 and err_s == 0
    assert torch.equal(dyn.view(torch.int16), sta.view(torch.int16))
    compare(sta, inp, torch.bfloat16, name="static small grid")


def test_log_reports_launches(capfd, monkeypatch):
    """GG_LOG=1: each launch reports the kernel variant, tile and grid on
    stderr (the library reads GG_LOG at every call)."""
    b = gg()
    inp = synth.wgrad_inputs(256, 256, [256, 0, 512], "m", "n", seed=3)
    out = torch.empty(3, 256, 256, dtype=torch.bfloat16, device="cuda")
    args = (inp["a"].cuda(), 1, inp["b"].cuda(), 2, inp["offsets"].cuda(), inp["tokens_sum"], 256,
            256)
    capfd.readouterr()
    monkeypatch.setenv("GG_LOG", "1")
    b.gg_wgrad(*args, wgrad_dense=out)
    b.gg_wgrad(*args, wgrad_dense=out, flags=b.GG_FLAG_STATIC_SCHED)
    monkeypatch.setenv("GG_LOG", "0")
    b.gg_wgrad(*args, wgrad_dense=out)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("[gg] gg_wgrad")]
    assert len(lines) == 2, err[-2000:]
    assert "wgrad_kernel<A M-major, B N-major, out bf16> (dynamic scheduling)" in lines[0]
    assert "(static scheduling)" in lines[1]
    assert "tile 256x256, 8 waves, grid " in lines[0]
