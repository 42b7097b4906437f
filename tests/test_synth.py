"""Input generators: group-size recipes and the MXFP8 encoding (no GPU)."""
import numpy as np
import torch

from moe_grouped_gemm_offset_amd import synth


def test_zipf_groups_profile():
    c = synth.workload_counts("wgrad_moe")
    assert c.sum() == 65536 and np.all(c % 256 == 0) and c.size == 64
    blocks = sorted((c // 256).tolist(), reverse=True)
    assert blocks[0] == 75 and blocks.count(0) == 6
    # same seed, same counts
    assert np.array_equal(c, synth.workload_counts("wgrad_moe"))


def test_multinomial_groups():
    for name, total, L in (("dswiglu", 16384, 8), ("dgeglu", 32768, 32), ("dsrelu_mxfp8", 65536, 16)):
        c = synth.workload_counts(name)
        assert c.size == L and c.sum() == total and np.all(c % 256 == 0)


def test_offsets_are_cumulative_int32():
    off = synth.cumulative([256, 0, 512, 256])
    assert off.dtype == np.int32 and off.tolist() == [256, 256, 768, 1024]


def test_mx_encode_bounds_and_roundtrip():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-8, 9, (64, 1), generator=g).float())
    q, s = synth.mx_encode(x)
    assert q.dtype == torch.float8_e4m3fn and s.dtype == torch.uint8 and s.shape == (64, 8)
    v = q.float().reshape(64, 8, 32) * torch.exp2(s.float() - 127).unsqueeze(2)
    # every block's largest magnitude uses the top binade without saturating
    amax = q.float().abs().reshape(64, 8, 32).amax(2)
    assert torch.all(amax <= 448) and torch.all(amax > 112)
    # relative error of E4M3 (3 fraction bits): at most 2^-4 of the block max
    err = (v.reshape(64, 256) - x).abs().reshape(64, 8, 32).amax(2)
    assert torch.all(err <= x.abs().reshape(64, 8, 32).amax(2) * 2.0 ** -4)
