"""Pins of the oracle's FP8 output quantization (no GPU).

"Grouped GEMM + dGLU (SM100)", "Block-scaled contract / Equations", step 3:
blocks of 32 values share SFD = norm_const * max|D| * rcp_max and
D_q = D * norm_const / SFD; E8M0 scales hold powers of two, read as the
smallest power of two not below the product, so that |D_q| <= 448 (E4M3).

Pinned by:
* the E4M3 encoder against torch's float8_e4m3fn cast on every code's value,
  the midpoints between codes and their fp32 neighbours, random values and
  subnormals, and against an exact rational round-to-nearest-even;
* per block, in exact rational arithmetic on the double D: 2^e is the
  smallest power of two at or above norm_const * amax / 448, and every code
  is the round-to-nearest-even E4M3 value of D * norm_const / 2^e; the
  largest code lies in [224, 448], and every dequantized value
  D_q * 2^e / norm_const is within half an E4M3 step of D;
* blocks at and one ulp either side of every power-of-two boundary, and
  values whose double product D * norm_const falls exactly on an E4M3
  rounding midpoint while the exact product does not;
* an exact case (amax * norm_const = 448 * 2^k gives e = k and code 448);
* the column blocks of D equal the row blocks of D transposed; an all-zero
  block has scale byte 0 and zero codes.
"""
import math
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


def _exact_exponent(amax, nc):
    """Smallest integer e with 2^e >= nc * amax / 448, in rational arithmetic
    (-127 for an all-zero block), clamped to the E8M0 range."""
    if amax == 0:
        return -127
    x = Fraction(float(np.float32(nc))) * Fraction(float(amax)) / 448
    e = math.floor(math.log2(x))
    while Fraction(2) ** e < x:
        e += 1
    while Fraction(2) ** (e - 1) >= x:
        e -= 1
    return max(-127, min(127, e))


def _exact_code_value(d, nc, e):
    """The E4M3 value of d * nc / 2^e rounded once, to nearest even, from the
    exact rational (magnitudes above 448 clamped to 448)."""
    x = Fraction(float(d)) * Fraction(float(np.float32(nc))) / Fraction(2) ** e
    ax = min(abs(x), Fraction(448))
    v = _rne_fraction(ax, 4, -6, Fraction(448))
    return -v if x < 0 else v


def _check_blocks_exact(D, nc, r):
    """Every row and column block of orc_quant_fp8's result against the exact
    rational definition: scale exponent and every code."""
    nrows, W = D.shape
    for kind in ("row", "col"):
        if kind == "row":
            Db = D.reshape(nrows, W // 32, 32)
            qb = r["q_row"].reshape(nrows, W // 32, 32)
            eb = r["sfd_row"].astype(np.int64) - 127
        else:
            Db = D.T.reshape(W, nrows // 32, 32)
            qb = r["q_col"].T.reshape(W, nrows // 32, 32)
            eb = r["sfd_col"].astype(np.int64) - 127
        for i in range(Db.shape[0]):
            for j in range(Db.shape[1]):
                blk = Db[i, j]
                e = _exact_exponent(np.abs(blk).max(), nc)
                assert eb[i, j] == e, (kind, i, j, eb[i, j], e)
                got = e4m3_value(qb[i, j])
                want = [_exact_code_value(d, nc, e) for d in blk]
                assert np.array_equal(got, want), (kind, i, j, got, want)


@pytest.mark.parametrize("nc", [1.0, 0.37, 3000.0])
def test_block_scales_and_values(nc):
    rng = np.random.default_rng(6)
    D = rng.normal(size=(64, 96)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    D[5, 32:64] = 0.0                                   # an all-zero row block
    r = orc.quant_fp8(D, nc)
    _check_blocks_exact(D, nc, r)
    for (q, sfd, blocks) in ((r["q_row"], r["sfd_row"], "row"), (r["q_col"], r["sfd_col"], "col")):
        if blocks == "row":
            Db, qb, eb = D.reshape(64, 3, 32), q.reshape(64, 3, 32), sfd.astype(np.int64) - 127
        else:
            Db = D.T.reshape(96, 2, 32)
            qb = q.T.reshape(96, 2, 32)
            eb = sfd.astype(np.int64) - 127
        amax = np.abs(Db).max(axis=2)
        nz = amax > 0
        assert np.all(eb[~nz] == -127) and np.all(qb[~nz] == 0)
        vals = e4m3_value(qb)
        top = np.abs(vals).max(axis=2)
        # the largest code of a block lies in (224, 448]; half an E4M3 step
        # bounds every dequantized value's error
        assert np.all(top[nz] >= 224.0) and np.all(top <= 448.0)
        deq = vals * np.exp2(eb)[..., None] / np.float64(np.float32(nc))
        err = np.abs(deq - Db)
        bound = 2.0 ** -4 * np.abs(Db) * (1 + 1e-12) + 2.0 ** -10 * np.exp2(eb)[..., None] / nc
        assert np.all(err <= bound)


@pytest.mark.parametrize("nc", [1.0, 0.37, 3000.0, 0.1])
def test_power_of_two_boundaries(nc):
    """Blocks whose nc * amax / 448 lies exactly at, or one double ulp either
    side of, a power of two: the scale exponent is the exact one (an fp32
    evaluation of the product rounds the neighbours onto the boundary and
    picks the wrong exponent for the one above it)."""
    ncf = float(np.float32(nc))
    rows = []
    for k in range(-12, 13, 3):
        target = 448.0 * 2.0 ** k / ncf               # nearest double to the boundary amax
        for amax in (np.nextafter(target, 0.0), target, np.nextafter(target, np.inf),
                     np.nextafter(np.nextafter(target, np.inf), np.inf)):
            row = np.linspace(-0.5, 0.5, 32) * amax
            row[7] = amax
            rows.append(row)
    D = np.array(rows, np.float64)
    D = np.concatenate([D, np.zeros(((-len(D)) % 32, 32))])
    r = orc.quant_fp8(D, nc)
    _check_blocks_exact(D, nc, r)
    # at nc = 1 the boundary itself is exact: amax = 448 * 2^k gives e = k and
    # the code 448; one double ulp above gives e = k + 1
    if nc == 1.0:
        for i, k in enumerate(range(-12, 13, 3)):
            assert r["sfd_row"][4 * i + 1, 0] == 127 + k and r["q_row"][4 * i + 1, 7] == 0x7E
            assert r["sfd_row"][4 * i + 2, 0] == 127 + k + 1
            assert r["sfd_row"][4 * i, 0] == 127 + k


def test_code_rounding_uses_the_exact_product():
    """Values whose double product d * nc rounds onto an E4M3 rounding
    midpoint while the exact product lies beside it: the code follows the
    exact product (rounding the double product would tie to even instead)."""
    rng = np.random.default_rng(8)
    mids = [232.0, 248.0, 208.0, 176.0, 13.5, 0.5 + 2 ** -5]   # midpoints between E4M3 values
    found = []
    for _ in range(200000):
        nc = float(np.float32(rng.uniform(0.3, 3.0)))
        m = mids[len(found) % len(mids)]
        d = m / nc
        for dd in (np.nextafter(d, 0.0), d, np.nextafter(d, np.inf)):
            if dd * nc == m and Fraction(float(dd)) * Fraction(nc) != Fraction(m):
                found.append((dd, nc))
                break
        if len(found) >= 12:
            break
    assert len(found) >= 12
    for d, nc in found:
        D = np.zeros((32, 32))
        D[0, 0] = d
        D[0, 1] = 448.0 / nc                      # amax with e = 0 (448 / nc * nc = 448)
        e = _exact_exponent(np.abs(D[0]).max(), nc)
        r = orc.quant_fp8(D, nc, with_col=False)
        assert r["sfd_row"][0, 0] == 127 + e
        got = e4m3_value(r["q_row"][0, :1])[0]
        assert got == _exact_code_value(d, nc, e), (d, nc, e, got)


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
