"""GPU parity of gg_wgrad_mx against the oracle (through the C ABI).

Cases span several 256x256 tiles, partial M and N tiles, token counts that
are multiples of 128 but not of 256 (computed, flagged), counts that are
not whole load units (skipped, flagged), empty experts, per-row scale
spreads, the three output dtypes, dense and pointer outputs, accumulate and
overwrite, tensor2d and tensor_ragged storage, exact integers; and the
MoE-scale workload (hidden 4096, intermediate 2048, 64 Zipf experts, 65536
tokens) on sampled rows in the launch configuration the bench times.
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


def run_gpu(inp, out_dtype, accumulate=False, old=None, discrete=False, ragged=False):
    b = gg()
    E = len(inp["counts"])
    a, sfa = inp["a"].cuda().view(torch.uint8), inp["sfa"].cuda()
    bb, sfb = inp["b"].cuda().view(torch.uint8), inp["sfb"].cuda()
    flags = b.GG_FLAG_AB_E5M2 if inp["a"].dtype == torch.float8_e5m2 else 0
    if ragged:
        flags |= b.GG_FLAG_TENSOR_RAGGED
        a, bb = synth.to_ragged(a, inp["counts"]), synth.to_ragged(bb, inp["counts"])
        sfa = synth.to_ragged(sfa, inp["counts"], per=32)
        sfb = synth.to_ragged(sfb, inp["counts"], per=32)
    off = inp["offsets"].cuda()
    h, i, T = inp["hidden"], inp["inter"], inp["tokens_sum"]
    if discrete:
        outs = [torch.empty(h, i, dtype=out_dtype, device="cuda") for _ in range(E)]
        if accumulate:
            for e in range(E):
                outs[e].copy_(old[e])
        ptrs = torch.tensor([o.data_ptr() for o in outs], dtype=torch.int64, device="cuda")
        ws = b.gg_wgrad_mx(a, sfa, bb, sfb, off, T, h, i, wgrad_ptrs=ptrs,
                           wgrad_dtype=b._TORCH_DTYPE[out_dtype], accumulate=accumulate, flags=flags)
        torch.cuda.synchronize()
        res = torch.stack(outs)
    else:
        res = old.clone().cuda() if accumulate else \
            torch.full((E, h, i), float("nan"), dtype=out_dtype, device="cuda")
        ws = b.gg_wgrad_mx(a, sfa, bb, sfb, off, T, h, i, wgrad_dense=res, accumulate=accumulate,
                           flags=flags)
        torch.cuda.synchronize()
    return res.cpu(), b.gg_device_error(ws)


def run_oracle(inp, out_dtype, accumulate=False, old=None, hrows=None):
    od = ORC_DT[out_dtype]
    return orc.wgrad_mx(synth.bits(inp["a"]), synth.bits(inp["sfa"]), synth.bits(inp["b"]),
                        synth.bits(inp["sfb"]), inp["offsets"].numpy(), inp["hidden"],
                        inp["inter"], inp["tokens_sum"], out_dtype=od, accumulate=accumulate,
                        old=None if old is None else synth.bits(old), hrows=hrows,
                        ab_dtype=ORC_DT[inp["a"].dtype]), od


def compare(got, inp, out_dtype, accumulate=False, old=None, hrows=None, name="", skipped=()):
    (exact, _), od = run_oracle(inp, out_dtype, accumulate, old, hrows)
    g = values(got if hrows is None else got[:, hrows, :])
    for e, cnt in enumerate(inp["counts"]):
        if e in skipped:
            assert np.all(g[e] == 0), f"{name}: skipped expert {e} not zero"
            exact[e] = 0.0
        elif cnt == 0 and not accumulate:
            assert np.all(g[e] == 0), f"{name}: empty expert {e} not exactly zero"
        elif cnt == 0 and accumulate:
            want = values(old[e] if hrows is None else old[e][hrows])
            assert np.array_equal(g[e], want), f"{name}: empty expert {e} changed in accumulate mode"
        else:
            err = normwise(g[e], exact[e])
            assert err <= TOL[od], f"{name}: expert {e} normwise error {err:.3e}"
    assert_close(g, exact, od, f"{name} all experts")


def small(seed, counts=(256, 0, 512, 128, 384), hidden=320, inter=384, **kw):
    return synth.wgrad_mx_inputs(hidden, inter, counts, seed=seed, scale_spread=3, **kw)


@pytest.mark.parametrize("ragged", [False, True])
def test_small(ragged):
    inp = small(101)
    say("wgrad_mx small", "ragged" if ragged else "tensor2d", inp["counts"].tolist())
    got, err = run_gpu(inp, torch.float32, ragged=ragged)
    assert err == 2  # GG_DEVERR_GRANULE: counts of 128 and 384 (still computed)
    compare(got, inp, torch.float32, name="small")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("discrete", [False, True])
@pytest.mark.parametrize("accumulate", [False, True])
def test_outputs_and_modes(dtype, discrete, accumulate):
    counts = [256, 0, 768, 512]
    inp = small(102, counts=counts, hidden=256, inter=320)
    old = synth.wgrad_initial(len(counts), 256, 320, dtype, seed=103) if accumulate else None
    say("wgrad_mx modes", dtype, "discrete" if discrete else "dense", "acc" if accumulate else "over")
    got, err = run_gpu(inp, dtype, accumulate, old, discrete)
    assert err == 0
    compare(got, inp, dtype, accumulate, old, name=f"{dtype} {discrete} {accumulate}")


@pytest.mark.parametrize("dtype,discrete,ragged", [(torch.float32, False, False),
                                                   (torch.bfloat16, True, True),
                                                   (torch.float16, False, True)])
def test_e5m2_operands(dtype, discrete, ragged):
    """E5M2 codes for both operands (GG_FLAG_AB_E5M2): the MFMA's format
    fields select E5M2 for A and B."""
    counts = [256, 0, 768, 512]
    inp = small(107, counts=counts, hidden=256, inter=320, ab_dtype=torch.float8_e5m2)
    say("wgrad_mx e5m2", dtype, "discrete" if discrete else "dense", "ragged" if ragged else "")
    got, err = run_gpu(inp, dtype, discrete=discrete, ragged=ragged)
    assert err == 0
    compare(got, inp, dtype, name=f"e5m2 {dtype}")


def test_e5m2_exact_integers_bit_exact():
    """Integers in [-2, 2] are exact in E5M2 too: bit-exact fp32 sums."""
    inp = small(108, counts=(256, 512, 0, 256), hidden=256, inter=256, ints=True,
                ab_dtype=torch.float8_e5m2)
    got, _ = run_gpu(inp, torch.float32)
    (exact, res), _ = run_oracle(inp, torch.float32)
    assert np.array_equal(got.numpy(), res)


def test_exact_integers_bit_exact():
    inp = small(104, counts=(256, 512, 0, 256), hidden=256, inter=256, ints=True)
    got, _ = run_gpu(inp, torch.float32)
    (exact, res), _ = run_oracle(inp, torch.float32)
    assert np.array_equal(got.numpy(), res), "integer-valued wgrad must be bit-exact"


def test_partial_units_are_skipped():
    """A count of 64 is not a whole load unit: that expert and the next (whose
    slice then starts off a unit boundary) are skipped and flagged; the
    others are exact."""
    inp = small(105, counts=(256, 64, 192, 256), hidden=256, inter=256)
    got, err = run_gpu(inp, torch.float32)
    assert err & 8, "GG_DEVERR_SKIPPED"
    compare(got, inp, torch.float32, name="skipped", skipped=(1, 2))


def test_tokens_sum_zero():
    inp = small(106, counts=(0, 0), hidden=256, inter=256)
    got, err = run_gpu(inp, torch.bfloat16)
    assert err == 0 and torch.all(got == 0)


def test_moe_scale_sampled():
    """The MoE-scale workload, bf16 dense output, on the device; the oracle
    checks sampled hidden rows of every expert."""
    w = synth.WORKLOADS["wgrad_mxfp8"]
    counts = synth.workload_counts("wgrad_mxfp8")
    inp = synth.wgrad_mx_inputs(w["hidden"], w["inter"], counts, seed=w["seed"], device="cuda")
    say("wgrad_mxfp8 experts", len(counts), "empty", int(np.sum(counts == 0)))
    got, err = run_gpu(inp, torch.bfloat16)
    assert err == 0
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    rows = np.array([0, 255, 256, 2048, 4095], np.int32)
    compare(got, cpu, torch.bfloat16, hrows=rows, name="wgrad_mxfp8")
