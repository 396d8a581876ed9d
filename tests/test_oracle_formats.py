"""Pins of the oracle's number formats and its two-level quantizer.

Everything here is checked against something other than the oracle itself:
the E2M1 value list the memory-wall blog prints (section 2), PyTorch's
float8_e4m3fn conversions, and a brute-force nearest-value search in exact
rational arithmetic (``fractions.Fraction``).
"""
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# ----------------------------------------------------------------- fixtures


def _page_grid(golden_dir):
    with open(os.path.join(golden_dir, "e2m1_grid.txt")) as f:
        line = [ln for ln in f if not ln.startswith("#") and ln.strip()][0]
    return [float(t) for t in line.split()]


def _torch_e4m3_values():
    b = torch.arange(256, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


E4M3_T = _torch_e4m3_values()
E4M3_FR = [Fraction(float(E4M3_T[b])) for b in range(0x7F)]  # finite non-negative bytes 0..126


def _magnitudes(golden_dir):
    g = sorted({abs(v) for v in _page_grid(golden_dir)})
    assert len(g) == 8
    return [Fraction(v) for v in g]


def bf_scale_byte(amax: Fraction, g: Fraction) -> int:
    """Nearest E4M3 value (torch's table) to amax/(6g); ties to the even byte."""
    r = amax / (6 * g)
    return min(range(0x7F), key=lambda b: (abs(r - E4M3_FR[b]), b & 1))


def bf_code(x: float, bs: Fraction, g: Fraction, mags) -> int:
    """Nearest page-list magnitude to |x|/(bs*g); ties to the even code; sign bit kept."""
    sign = 8 if math.copysign(1.0, x) < 0 else 0
    if bs == 0:
        return sign
    y = abs(Fraction(x)) / (bs * g)
    return sign | min(range(8), key=lambda c: (abs(y - mags[c]), c & 1))


def bf_quantize_row(row, g, mags):
    gf = Fraction(float(np.float32(g)))
    codes = np.zeros(64, np.uint8)
    scales = np.zeros(8, np.uint8)
    for b in range(8):
        blk = [float(v) for v in row[16 * b:16 * b + 16]]
        amax = max(abs(Fraction(v)) for v in blk)
        sb = bf_scale_byte(amax, gf)
        scales[b] = sb
        bs = E4M3_FR[sb]
        for i, v in enumerate(blk):
            d = 16 * b + i
            codes[d // 2] |= bf_code(v, bs, gf, mags) << (4 * (d & 1))
    return codes, scales


# ------------------------------------------------------------------- E2M1


def test_e2m1_codes_are_the_page_grid(golden_dir):
    grid = _page_grid(golden_dir)
    vals = [oracle.e2m1_value(c) for c in range(16)]
    # the 16 codes give exactly the 16 listed values, signed zeros included
    key = lambda v: (v, math.copysign(1.0, v))
    assert sorted(map(key, vals)) == sorted(map(key, grid))
    # codes 0..7 are the magnitudes in increasing order; code | 8 is the negative
    mags = sorted({abs(v) for v in grid})
    for c in range(8):
        assert vals[c] == mags[c] and math.copysign(1.0, vals[c]) > 0
        assert vals[c | 8] == -mags[c] and math.copysign(1.0, vals[c | 8]) < 0


def test_e2m1_grid_round_trips_exactly(golden_dir):
    """Every grid value survives quantize -> dequantize with amax 6, g 1 (scale 1)."""
    grid = _page_grid(golden_dir)
    row = np.array((grid * 8)[:128], np.float32)
    row[0] = 6.0  # every block holds a 6 or -6, so amax = 6 and the block scale is exactly 1
    for b in range(8):
        assert max(abs(v) for v in row[16 * b:16 * b + 16]) == 6.0
    codes, scales = oracle.quantize_rows(row, 1.0)
    assert (scales == 0x38).all()  # E4M3 byte of 1.0
    back = oracle.dequantize_rows(codes, scales, 1.0)[0]
    assert np.array_equal(back, row.astype(np.float64))
    assert np.array_equal(np.signbit(back), np.signbit(row))


@pytest.mark.parametrize("y,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
                                    (0.2500001, 1), (0.7499999, 1), (4.9999999, 6), (5.0000001, 7), (7.0, 7),
                                    (1e300, 7), (0.0, 0)])
def test_e2m1_ties_to_even_and_saturation(y, code):
    assert oracle.e2m1_encode(y) == code


# ------------------------------------------------------------------- E4M3


def test_e4m3_decode_matches_torch():
    for b in range(256):
        v, t = oracle.e4m3_value(b), E4M3_T[b]
        if math.isnan(t):
            assert math.isnan(v)
        else:
            assert v == t and math.copysign(1.0, v) == math.copysign(1.0, t)


def test_e4m3_encode_matches_torch_on_float32():
    rng = np.random.default_rng(7)
    # every bf16 bit pattern in [0, 448] plus random float32 values and exact midpoints
    pats = (np.arange(0, 0x43E1, dtype=np.uint32) << 16).view(np.float32)
    rnd = rng.uniform(0, 448, 20000).astype(np.float32)
    small = (rng.uniform(0, 1, 20000) * 2.0 ** -6).astype(np.float32)
    finite = E4M3_T[:0x7F]
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)
    xs = np.concatenate([pats, rnd, small, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    xs = xs[(xs >= 0) & (xs <= 448)]
    ref = torch.from_numpy(xs.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("r,byte", [(448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (1e300, 0x7E),
                                    (2.0 ** -10, 0x00), (2.0 ** -10 * 1.0000001, 0x01), (3 * 2.0 ** -10, 0x02),
                                    (0.0, 0x00)])
def test_e4m3_saturation_and_subnormal_ties(r, byte):
    assert oracle.e4m3_encode(r) == byte


# ------------------------------------------------------- two-level quantizer


def _random_rows(rng, n):
    rows = []
    for i in range(n):
        kind = i % 6
        if kind == 0:
            r = rng.normal(0, 0.02, 128)
        elif kind == 1:
            r = rng.normal(0, 0.02, 128)
            r[rng.integers(0, 128, 3)] = rng.choice([-6.0, 6.0], 3)
        elif kind == 2:
            r = rng.normal(0, 1, 128) * np.exp(rng.uniform(-20, 20, 128))
        elif kind == 3:
            r = rng.normal(0, 0.02, 128)
            r[16:32] = 0.0
            r[40] = -0.0
        elif kind == 4:
            r = rng.standard_cauchy(128)
        else:
            r = rng.uniform(-1, 1, 128) * 1e-6
        rows.append(r.astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("g", [1.0, 6.0 / 2688.0, 1.0 / 448.0, 0.37, 1e-4, 3.0e3])
def test_quantizer_matches_exact_rational_brute_force(golden_dir, g):
    mags = _magnitudes(golden_dir)
    rng = np.random.default_rng(abs(hash(g)) % 2 ** 32)
    rows = _random_rows(rng, 24)
    codes, scales = oracle.quantize_rows(rows, g)
    for r in range(rows.shape[0]):
        bc, bsb = bf_quantize_row(rows[r], g, mags)
        assert np.array_equal(scales[r], bsb), (r, scales[r], bsb)
        assert np.array_equal(codes[r], bc), r


def test_quantizer_exact_ties(golden_dir):
    """Values placed exactly on code midpoints and block amax exactly on scale midpoints."""
    mags = _magnitudes(golden_dir)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    finite = [float(v) for v in E4M3_T[:0x7F]]
    rows = []
    # code ties: bs = 1 (amax 6, g 1); the block holds every midpoint of both signs
    r = np.zeros(128, np.float32)
    for b in range(8):
        blk = [6.0] + mids + [-m for m in mids] + [-0.0]
        r[16 * b:16 * b + 16] = blk[:16]
    rows.append((r, 1.0))
    # code ties at a non-power-of-two scale: g = 0.5, amax = 6*g*1.5 -> bs = 1.5
    r = np.zeros(128, np.float32)
    for b in range(8):
        blk = [4.5] + [m * 1.5 * 0.5 for m in mids] + [-m * 1.5 * 0.5 for m in mids] + [0.0]
        r[16 * b:16 * b + 16] = blk[:16]
    rows.append((r, 0.5))
    # scale ties: amax/(6g) exactly on E4M3 midpoints (g = 0.5, amax = 3*midpoint is exact in float32)
    g = 0.5
    sel = [0, 1, 7, 8, 30, 63, 64, 100, 124]
    r = np.zeros(128, np.float32)
    for b, k in enumerate(sel[:8]):
        m = (Fraction(finite[k]) + Fraction(finite[k + 1])) / 2
        amax = float(m * 3)
        assert Fraction(float(np.float32(amax))) == m * 3
        r[16 * b] = amax
        r[16 * b + 1:16 * b + 16] = np.linspace(-amax, amax, 15)
    rows.append((r, g))
    for r, g in rows:
        codes, scales = oracle.quantize_rows(r, g)
        bc, bsb = bf_quantize_row(r, g, mags)
        assert np.array_equal(scales[0], bsb)
        assert np.array_equal(codes[0], bc)


def test_zero_and_underflow_blocks():
    r = np.zeros(128, np.float32)
    r[16:32] = -0.0
    r[32:48] = 1e-30  # amax/(6g) far below 2^-10 -> scale 0
    r[48:64] = -1e-30
    codes, scales = oracle.quantize_rows(r, 1.0)
    assert (scales[0, :4] == 0).all()
    nib = np.stack([codes[0] & 15, codes[0] >> 4], 1).reshape(-1)
    assert (nib[:16] == 0).all() and (nib[16:32] == 8).all()
    assert (nib[32:48] == 0).all() and (nib[48:64] == 8).all()
