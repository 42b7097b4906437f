"""Pins of the oracle's FP8 output quantization (no GPU).

"Grouped GEMM + dGLU (SM100)", "Block-scaled contract / Equations", step 3:
blocks of 32 values share SFD = norm_const * max|D| * rcp_max and
D_q = D * norm_const / SFD; E8M0 scales hold powers of two, read as the
smallest power of two not below the product, so that |D_q| <= 448 (E4M3).

Pinned by:
* the E4M3 encoder against torch's float8_e4m3fn cast on every code's value,
  the midpoints between codes and their fp32 neighbours, random values and
  subnormals, and against an exact rational round-to-nearest-even;
* per block: 2^e is the smallest power of two at or above
  norm_const * amax / 448 (checked in exact arithmetic away from the
  boundaries), the largest code lies in (224, 448], and every dequantized
  value D_q * 2^e / norm_const is within half an E4M3 step of D;
* an exact case (amax * norm_const = 448 * 2^k gives e = k and code 448);
* the column blocks of D equal the row blocks of D transposed; an all-zero
  block has scale byte 0 and zero codes.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tests.test_oracle_codecs import _rne_fraction

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()


def e4m3_value(codes):
    return E4M3[np.asarray(codes, np.int64)]


def test_encoder_vs_torch():
    v = np.unique(E4M3[np.isfinite(E4M3)])
    mids = (v[1:] + v[:-1]) / 2
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(1e9)).astype(np.float64)
    dn = np.nextafter(mids32, np.float32(-1e9)).astype(np.float64)
    rnd = np.random.default_rng(3).uniform(-448, 448, 20000).astype(np.float32).astype(np.float64)
    sub = np.ldexp(np.random.default_rng(4).uniform(-1, 1, 2000), -8)
    xs = np.concatenate([v, mids, up, dn, rnd, sub])
    got = orc.encode_e4m3(xs)
    ref = torch.from_numpy(xs).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch casts through fp32, so compare where fp32 holds x exactly
    exact = xs.astype(np.float32).astype(np.float64) == xs
    assert exact.sum() > 20000
    bad = np.nonzero((got != ref) & exact)[0]
    assert bad.size == 0, [(xs[i], got[i], ref[i]) for i in bad[:5]]


def test_encoder_vs_exact_rational():
    rng = np.random.default_rng(5)
    xs = list(np.ldexp(rng.uniform(-1, 1, 3000), rng.integers(-12, 9, 3000)))
    xs += [448.0, 464.0, 480.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6 * 1.0625]
    for x in xs:
        ax = min(abs(x), 448.0)
        want = _rne_fraction(Fraction(ax), 4, -6, Fraction(448))
        want = -want if x < 0 else want
        got = e4m3_value(orc.encode_e4m3([x]))[0]
        assert got == want or (got == 0 and want == 0), (x, got, want)


@pytest.mark.parametrize("nc", [1.0, 0.37, 3000.0])
def test_block_scales_and_values(nc):
    rng = np.random.default_rng(6)
    D = rng.normal(size=(64, 96)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    D[5, 32:64] = 0.0                                   # an all-zero row block
    r = orc.quant_fp8(D, nc)
    for (q, sfd, blocks) in ((r["q_row"], r["sfd_row"], "row"), (r["q_col"], r["sfd_col"], "col")):
        if blocks == "row":
            Db, qb, eb = D.reshape(64, 3, 32), q.reshape(64, 3, 32), sfd.astype(np.int64) - 127
        else:
            Db = D.T.reshape(96, 2, 32)
            qb = q.T.reshape(96, 2, 32)
            eb = sfd.astype(np.int64) - 127
        amax = np.abs(Db.astype(np.float32)).max(axis=2).astype(np.float64)
        ratio = nc * amax / 448.0
        nz = amax > 0
        # 2^e is the smallest power of two >= ratio (skip ratios within 1e-6
        # of a power of two, where fp32 rounding decides)
        lg = np.log2(np.where(nz, ratio, 1.0))
        clear = nz & (np.abs(lg - np.round(lg)) > 1e-6)
        assert np.all(eb[clear] == np.ceil(lg[clear]).astype(np.int64))
        assert np.all(eb[~nz] == -127) and np.all(qb[~nz] == 0)
        vals = e4m3_value(qb)
        top = np.abs(vals).max(axis=2)
        assert np.all(top[clear] > 224.0 * (1 - 2.0 ** -4)) and np.all(top <= 448.0)
        deq = vals * np.exp2(eb)[..., None] / nc
        err = np.abs(deq - Db)
        bound = 2.0 ** -4 * np.abs(Db) * (1 + 1e-6) + 2.0 ** -10 * np.exp2(eb)[..., None] / nc
        assert np.all(err <= bound)


def test_exact_power_of_two_case():
    D = np.zeros((32, 32))
    D[3, :] = np.linspace(-1, 1, 32)
    D[3, 7] = 448.0 * 2.0 ** -5          # amax of row 3: 14.0, nc = 1 -> e = -5
    r = orc.quant_fp8(D, 1.0)
    assert r["sfd_row"][3, 0] == 127 - 5
    assert r["q_row"][3, 7] == 0x7E      # 448
    assert r["sfd_row"][0, 0] == 0 and np.all(r["q_row"][0] == 0)


def test_columns_are_rows_of_the_transpose():
    D = np.random.default_rng(7).normal(size=(96, 64)) * 10
    r = orc.quant_fp8(D, 0.5)
    t = orc.quant_fp8(np.ascontiguousarray(D.T), 0.5, with_col=False)
    assert np.array_equal(r["q_col"], t["q_row"].T)
    assert np.array_equal(r["sfd_col"], t["sfd_row"])
