"""GPU parity of gg_dglu against the oracle (through the C ABI).

Small cases span several 256-row tiles, a partial N tile, an empty group and
rows past valid_m; they cover dSwiGLU and dGeGLU (value and mask filters),
dense / discrete K-major / discrete N-major B, the gate-first order, dbias,
and C/D dtypes.  The two named workloads (dSwiGLU: L 8, K 2048, N 1024,
M 16384; dGeGLU: L 32, K 4096, N 1536, M 32768, discrete B, dbias) run at
full size in the bench's launch configuration: every row of the dSwiGLU
workload, and for dGeGLU sampled rows of every group plus every row and the
dbias of its small groups, all against the oracle.
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


def run_gpu(inp, act, flags=0, d_dtype=torch.bfloat16, dbias=False):
    b = gg()
    dev = lambda x: x.cuda()
    M, N, L = inp["M"], inp["N"], inp["L"]
    a = dev(inp["a"])
    if inp["b_dense"] is not None:
        bd, bp, keep = dev(inp["b_dense"]), None, None
    else:
        keep = [dev(x) for x in inp["b_list"]]
        bd, bp = None, torch.tensor([x.data_ptr() for x in keep], dtype=torch.int64, device="cuda")
    d = torch.full((M, 2 * N), float("nan"), dtype=d_dtype, device="cuda")
    dprob = torch.zeros(M, dtype=torch.float32, device="cuda")
    db = torch.zeros(L, 2 * N, dtype=torch.bfloat16, device="cuda") if dbias else None
    ws = b.gg_dglu(a, bd, bp, 0 if inp["b_major"] == "k" else 2, N, dev(inp["c"]),
                   dev(inp["padded_offsets"]), dev(inp["alpha"]), dev(inp["beta"]), dev(inp["prob"]),
                   d, dprob, db, act=act, flags=flags)
    torch.cuda.synchronize()
    err = b.gg_device_error(ws)
    return d.cpu(), dprob.cpu(), (db.cpu() if dbias else None), err


def run_oracle(inp, act, flags=0, d_dtype=torch.bfloat16, dbias=False, rows=None):
    L, N = inp["L"], inp["N"]
    return orc.dglu(synth.bits(inp["a"]), inp["M"], inp["K"], [synth.bits(x) for x in inp["b_list"]],
                    0 if inp["b_major"] == "k" else 1, N, synth.bits(inp["c"]), ORC_DT[inp["c"].dtype],
                    inp["padded_offsets"].numpy(), inp["alpha"].numpy(), inp["beta"].numpy(),
                    inp["prob"].numpy(), act=act, gate_first=bool(flags & 1), mask_filter=bool(flags & 2),
                    d_dtype=ORC_DT[d_dtype],
                    dbias_in=np.zeros((L, 2 * N), np.uint16) if dbias else None, rows=rows)


def check(inp, act, flags=0, d_dtype=torch.bfloat16, dbias=False, name=""):
    say(name, "act", act, "flags", flags, d_dtype, "dbias" if dbias else "")
    d, dprob, db, err = run_gpu(inp, act, flags, d_dtype, dbias)
    assert err in (0,), f"device error word {err}"
    ref = run_oracle(inp, act, flags, d_dtype, dbias)
    vm = inp["valid_m"]
    odt = ORC_DT[d_dtype]
    assert_close(values(d[:vm]), ref["D"][:vm], odt, f"{name} D_row")
    assert torch.all(torch.isnan(d[vm:])), "rows past valid_m must not be written"
    assert_close(values(dprob[:vm]), ref["dprob"][:vm], orc.F32, f"{name} dprob")
    assert torch.all(dprob[vm:] == 0)
    start = 0
    for g, cnt in enumerate(inp["counts"]):
        if cnt:
            e = normwise(values(d[start:start + cnt]), ref["D"][start:start + cnt])
            assert e <= TOL[odt], f"{name}: group {g} D error {e:.3e}"
        start += cnt
    if dbias:
        assert_close(values(db), ref["dbias"], orc.BF16, f"{name} dbias")
        for g, cnt in enumerate(inp["counts"]):
            if cnt == 0:
                assert torch.all(db[g] == 0), "an empty group's dbias must stay zero"


def small(seed, c_std=2.0, discrete=False, b_major="k", c_dtype=torch.bfloat16):
    counts = [256, 0, 512, 256]
    return synth.dglu_inputs(4, 256, 320, counts, a_std=0.05, b_std=0.05, c_std=c_std,
                             c_dtype=c_dtype, m_extra=64, seed=seed, discrete=discrete,
                             b_major=b_major)


@pytest.mark.parametrize("act", [orc.DSWIGLU, orc.DGEGLU])
@pytest.mark.parametrize("mode", ["dense", "discrete_k", "discrete_n"])
def test_small(act, mode):
    inp = small(51 + act, c_std=4.0 if act == orc.DGEGLU else 2.0, discrete=mode != "dense",
                b_major="n" if mode == "discrete_n" else "k")
    check(inp, act, dbias=True, name=f"small {mode}")


def test_static_sched_flag():
    """GG_FLAG_STATIC_SCHED is accepted and changes nothing: one workgroup
    per tile is already a fixed schedule."""
    inp = small(60, discrete=True, b_major="n")
    base = run_gpu(inp, orc.DGEGLU, 0, dbias=True)
    stat = run_gpu(inp, orc.DGEGLU, gg().GG_FLAG_STATIC_SCHED, dbias=True)
    assert torch.equal(base[0].view(torch.int16), stat[0].view(torch.int16))   # NaN rows unwritten
    # dprob and dbias are summed by atomics, in no fixed order
    assert torch.allclose(base[1], stat[1], rtol=1e-5, atol=1e-6)
    assert torch.allclose(base[2].float(), stat[2].float(), rtol=2 ** -7, atol=0)
    assert base[3] == stat[3] == 0


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_flags(flags):
    inp = small(55, c_std=4.0)
    check(inp, orc.DGEGLU, flags=flags, name="flags")


@pytest.mark.parametrize("c_dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("d_dtype", [torch.float16, torch.float32])
def test_dtypes(c_dtype, d_dtype):
    inp = small(56, c_dtype=c_dtype)
    check(inp, orc.DSWIGLU, d_dtype=d_dtype, name="dtypes")


def _full(name, device="cuda"):
    w = synth.WORKLOADS[name]
    counts = synth.workload_counts(name)
    return synth.dglu_inputs(w["L"], w["K"], w["N"], counts, c_std=w["c_std"], seed=w["seed"],
                             device=device, discrete=w["discrete"]), w


def test_workload_dswiglu_every_row():
    """The dSwiGLU workload at full size (L 8, K 2048, N 1024, M 16384): every
    row of D and dprob against the oracle, whole and per expert."""
    inp, w = _full("dswiglu")
    say("dswiglu counts", inp["counts"].tolist())
    d, dprob, _, err = run_gpu(inp, orc.DSWIGLU)
    assert err == 0
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cpu["b_list"] = [x.cpu() for x in inp["b_list"]]
    ref = run_oracle(cpu, orc.DSWIGLU)
    assert_close(values(d), ref["D"], orc.BF16, "dswiglu D_row (every row)")
    assert_close(values(dprob), ref["dprob"], orc.F32, "dswiglu dprob (every row)")
    start = 0
    for g, c in enumerate(inp["counts"]):
        if c:
            e = normwise(values(d[start:start + c]), ref["D"][start:start + c])
            assert e <= TOL[orc.BF16], f"group {g}: {e:.3e}"
        start += c


def test_workload_dgeglu():
    """The dGeGLU workload at full size (L 32, K 4096, N 1536, M 32768,
    discrete B, dbias): the first, second and last rows of every group, and
    every row of the groups of at most 512 rows (its three 256-row groups
    among them), against the oracle; those groups' dbias (the per-expert row
    reduction of D) against the oracle's, and the empty group's dbias exactly
    zero."""
    inp, w = _full("dgeglu")
    counts = inp["counts"]
    say("dgeglu counts", counts.tolist())
    d, dprob, db, err = run_gpu(inp, orc.DGEGLU, dbias=True)
    assert err == 0
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cpu["b_list"] = [x.cpu() for x in inp["b_list"]]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    whole = [g for g, c in enumerate(counts) if 0 < c <= 512]
    assert sum(1 for g in whole if counts[g] == 256) == 3
    rows = set()
    for g, (s, c) in enumerate(zip(starts, counts)):
        if g in whole:
            rows.update(range(s, s + c))
        elif c:
            rows.update([s, s + 1, s + c - 1])
    rows = np.array(sorted(rows), np.int64)
    ref = run_oracle(cpu, orc.DGEGLU, dbias=True, rows=rows)
    assert_close(values(d[rows]), ref["D"], orc.BF16, "dgeglu D_row (listed rows)")
    assert_close(values(dprob[rows]), ref["dprob"], orc.F32, "dgeglu dprob (listed rows)")
    for g in whole:
        assert_close(values(db[g]), ref["dbias"][g], orc.BF16, f"dgeglu dbias of group {g} ({counts[g]} rows)")
    for g, c in enumerate(counts):
        if c == 0:
            assert torch.all(db[g] == 0), "an empty group's dbias must stay zero"


@pytest.mark.parametrize("case", range(9))
def test_random_shapes(case):
    """Seeded random shapes through the ping-pong main loop: K a multiple of
    64 from 64 (a single load unit, forced in the last case) to 1024, compact N a multiple of 32 up
    to 640 (partial N tiles), 1-6 groups of 256-multiple rows (some empty),
    rows past valid_m, dense or discrete K-/N-major B, both activations,
    with or without dbias; every row against the oracle."""
    rng = np.random.default_rng(800 + case)
    K = int(rng.integers(1, 17)) * 64 if case < 8 else 64
    N = int(rng.integers(1, 21)) * 32
    L = int(rng.integers(1, 7))
    counts = [int(c) * 256 for c in rng.integers(0, 3, size=L)]
    if sum(counts) == 0:
        counts[0] = 256
    discrete = bool(case % 2)
    b_major = "n" if (discrete and case % 4 == 3) else "k"
    act = orc.DGEGLU if case % 3 == 0 else orc.DSWIGLU
    inp = synth.dglu_inputs(L, K, N, counts, a_std=0.05, b_std=0.05, c_std=4.0, m_extra=64 * (case % 2),
                            seed=800 + case, discrete=discrete, b_major=b_major)
    check(inp, act, dbias=bool(case % 3 == 1), name=f"random {case}: K {K} N {N} L {L} {counts} "
          f"{'discrete ' + b_major if discrete else 'dense'}")
