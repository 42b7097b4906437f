"""Pins of the oracle's number codecs against library routines and the
format definitions (no GPU).

The dGLU page names torch's float8_e4m3fn for FP8 operands and
float8_e8m0fnu for MXFP8 scales ("Support Surface and Constraints / Data
Types"); the output dtypes are bfloat16, float16 and float32.  The decoders
are checked on every code against torch / numpy casts, the encoders against
torch / numpy conversions and against an exact rational rounding.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all(both_nan | (a == b)) and np.array_equal(np.signbit(a) & ~both_nan,
                                                          np.signbit(b) & ~both_nan)


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(orc.decode(codes, orc.BF16), ref)
    assert _same(orc.decode_array(codes, orc.BF16), ref)


def test_f16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    assert _same(orc.decode(codes, orc.F16), ref)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    assert _same(orc.decode_e4m3(codes), ref)


def test_e4m3_spec_points():
    # Points of the OCP 8-bit floating point specification (E4M3).
    with open(os.path.join(GOLDEN, "ocp_e4m3_points.json")) as f:
        pts = json.load(f)["points"]
    for p in pts:
        v = orc.decode_e4m3(np.array([int(p["code"], 16)], np.uint8))[0]
        if p["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == float(Fraction(p["value"])), p


def test_e8m0_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = orc.decode_e8m0(codes)
    for c in range(255):
        assert got[c] == math.ldexp(1.0, c - 127)
    assert math.isnan(got[255])
    if hasattr(torch, "float8_e8m0fnu"):
        ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().double().numpy()
        assert _same(got, ref)


def _rne_fraction(x, p, emin, maxfin):
    """Exact round-to-nearest-even of the rational x into a binary format
    with p significand bits and minimum normal exponent emin."""
    if x == 0:
        return 0.0
    s = -1 if x < 0 else 1
    ax = abs(Fraction(x))
    e = math.floor(math.log2(ax))
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = ax / ulp
    lo = math.floor(q)
    rem = q - lo
    r = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else 0)
    y = r * ulp
    if y > maxfin:
        return s * math.inf
    return s * float(y)


def _random_doubles(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(-1, 1, n)
    exps = rng.integers(-140, 130, n)
    x = np.ldexp(mant, exps)
    return x


def test_bf16_encode_vs_exact_rational():
    xs = list(_random_doubles(3000, 1))
    # ties between neighbouring bf16 values and around the overflow threshold
    for k in range(50):
        base = 1.0 + k / 128.0
        xs += [base + 1 / 256.0, -(base + 1 / 256.0), (base + 1 / 256.0) * 2.0 ** -130]
    maxfin = 255 * 2.0 ** 120
    xs += [maxfin, maxfin * (1 + 2 ** -9), maxfin * (1 + 2 ** -9) * (1 - 2 ** -40), 2.0 ** -133,
           2.0 ** -134, 3 * 2.0 ** -135]
    for x in xs:
        want = _rne_fraction(Fraction(x), 8, -126, Fraction(255) * Fraction(2) ** 120)
        got = orc.decode(np.array([orc.lib().orc_double_to_bf16(x)], np.uint16), orc.BF16)[0]
        assert got == want or (math.isinf(got) and math.isinf(want) and got == want), (x, got, want)


def test_bf16_encode_vs_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_to(x.astype(np.float64), orc.BF16)
    assert np.array_equal(got, ref)


def test_f16_encode_vs_numpy():
    x = np.concatenate([_random_doubles(20000, 3) * 2.0 ** 10,
                        np.ldexp(np.random.default_rng(4).uniform(-1, 1, 5000), -14),
                        [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26]])
    ref = x.astype(np.float16).view(np.uint16)
    got = orc.round_to(x, orc.F16)
    assert np.array_equal(got, ref)


def test_f32_encode_vs_numpy():
    x = _random_doubles(20000, 5) * 2.0 ** 20
    x = np.concatenate([x, [2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -151, 3.4028235677973366e38]])
    ref = x.astype(np.float32)
    got = orc.round_to(x, orc.F32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
