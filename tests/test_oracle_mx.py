"""Pins for the oracle's MXFP4 comparison format (CPU only).

MXFP4 is the format NVFP4 is measured against: nmedialink.com "NVIDIA NVFP4:
LLM memory doubled, inference 3x", accuracy section and Fig. 6 (NVFP4 KV
caches score above MXFP4 ones, credited to the finer blocks and the E4M3
scales), and cloud.tencent.com.cn "NVFP4: breaking the memory wall of GPU
inference", E2M1 encoding and two-level scaling section (32 values share one
MXFP4 scale, 16 one NVFP4 scale; the smaller block loses about 30% less
precision).  The scale rule itself is the OCP MX v1.0 definition (a power of
two, E8M0, chosen from the block maximum's exponent), which the pages do not
spell out.

Pins: the E8M0 byte values, the scale exponent from amax (hand-worked values
and the invariant amax / X in [4, 8)), exact round trips of values on the
scaled E2M1 grid, every tie, saturation, the worst-case error bound, the
plane layout at hand-computed byte positions, decode attention against numpy
attention over dequantized rows, and the pages' direction of the NVFP4 vs
MXFP4 accuracy comparison.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_values():
    for b in (0, 1, 100, 126, 127, 128, 200, 254):
        assert oracle.e8m0_value(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(oracle.e8m0_value(255))


@pytest.mark.parametrize("amax,byte", [
    (6.0, 127), (4.0, 127), (7.999, 127), (8.0, 128), (3.999, 126), (2.0, 126), (1.0, 125),
    (0.02, 127 + (-6 - 2)),          # 0.02 = 1.28 * 2^-6
    (2.0 ** -125, 0), (2.0 ** -124, 1), (2.0 ** -140, 0),
    (1.5 * 2.0 ** 127, 252), (0.0, 0),
])
def test_scale_byte_hand_values(amax, byte):
    assert oracle.e8m0_scale_for(amax) == byte


def test_scale_puts_amax_in_4_to_8():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((400, 128)) * np.exp(rng.uniform(-20, 20, (400, 1)))).astype(np.float32)
    _, s = oracle.mx_quantize_rows(x)
    amax = np.abs(x.astype(np.float64)).reshape(400, 4, 32).max(axis=2)
    X = np.ldexp(1.0, s.astype(np.int64) - 127)
    r = amax / X
    assert ((r >= 4.0) & (r < 8.0)).all()


@pytest.mark.parametrize("j", [-100, -8, 0, 3, 60])
def test_grid_values_round_trip(j):
    # a block holding every signed E2M1 value times 2^j (amax 6 * 2^j -> X = 2^j)
    vals = np.array(GRID + [-v for v in GRID], np.float64)
    row = np.tile(vals, 8)[:128] * 2.0 ** j
    x = row.astype(np.float32)[None, :]
    c, s = oracle.mx_quantize_rows(x)
    assert (s == 127 + j).all()
    assert np.array_equal(oracle.mx_dequantize_rows(c, s)[0], row)


def test_ties_go_to_even_codes():
    # X = 1 (one 6.0 per block); midpoints between neighbouring E2M1 values
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = np.zeros(128, np.float32)
    for b in range(4):
        row[32 * b] = 6.0
        row[32 * b + 1: 32 * b + 8] = mids
        row[32 * b + 8: 32 * b + 15] = -np.array(mids)
    c, s = oracle.mx_quantize_rows(row[None, :])
    d = oracle.mx_dequantize_rows(c, s)[0]
    for b in range(4):
        assert list(d[32 * b + 1: 32 * b + 8]) == want
        assert list(d[32 * b + 8: 32 * b + 15]) == [-w for w in want]


def test_saturates_at_six_times_scale():
    row = np.zeros(128, np.float32)
    row[0], row[1], row[2] = 7.9, -7.9, 6.5       # amax 7.9 -> X = 1
    c, s = oracle.mx_quantize_rows(row[None, :])
    d = oracle.mx_dequantize_rows(c, s)[0]
    assert s[0, 0] == 127 and list(d[:3]) == [6.0, -6.0, 6.0]
    assert (c[0, 0] & 0xF) == 0x7 and (c[0, 0] >> 4) == 0xF


def test_error_bound_and_signs():
    # nearest-grid bound: |x - x_hat| <= half the local step (X/4 below 2X,
    # X/2 up to 4X, X up to 6X), clamped values above 6X go to 6X
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((300, 128)) * rng.uniform(0.01, 100, (300, 1))).astype(np.float32)
    x[::7, ::5] *= 40.0
    c, s = oracle.mx_quantize_rows(x)
    d = oracle.mx_dequantize_rows(c, s)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    ax = np.abs(x.astype(np.float64))
    half = np.where(ax <= 2 * X, X / 4, np.where(ax <= 4 * X, X / 2, X))
    inside = ax <= 6 * X
    assert (np.abs(d - x)[inside] <= half[inside]).all()
    assert (np.abs(d)[~inside] == 6 * X[~inside]).all()
    assert (np.sign(d)[d != 0] == np.sign(x)[d != 0]).all()


def test_plane_layout_positions():
    H, P = 2, 4
    planes = oracle.MxPlanes(P, H)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, H, 128)).astype(np.float32)
    v = rng.standard_normal((1, H, 128)).astype(np.float32)
    slot = 2 * 16 + 5                                   # page 2, offset 5
    kc, ks, vc, vs = oracle.mx_quantize_append(planes, k, v, [slot])
    for h in range(H):
        tile = 2 * H + h
        for b in range(4):
            assert planes.k_scales[tile * 64 + 5 * 4 + b] == ks[h, b]
            assert planes.v_scales[tile * 64 + b * 16 + 5] == vs[h, b]
        # K codes: token-major rows of 64 bytes; V codes: token-quad interleave
        assert np.array_equal(planes.k_codes[tile * 1024 + 5 * 64: tile * 1024 + 6 * 64], kc[h])
        for d in range(0, 128, 2):
            at = tile * 1024 + (5 // 4) * 256 + (d // 8) * 16 + (5 % 4) * 4 + (d % 8) // 2
            assert planes.v_codes[at] == vc[h, d // 2]
    assert planes.k_scales.sum() == ks.sum() and planes.v_scales.sum() == vs.sum()
    gc, gs = oracle.mx_gather_rows(planes.v_codes, planes.v_scales, [slot], H, True)
    assert np.array_equal(gc, vc) and np.array_equal(gs, vs)


def _numpy_attention(q, k, v, sm_scale):
    s = sm_scale * (k @ q)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ v


def test_decode_attention_matches_numpy_over_dequantized_rows():
    H, Hq, lens = 2, 8, [37, 16, 0, 70]
    bt, pool = synth.page_tables(lens, seed=21)
    planes = oracle.MxPlanes(pool, H)
    rng = np.random.default_rng(8)
    rows = {}
    for b, n in enumerate(lens):
        if n == 0:
            continue
        k = (rng.standard_normal((n, H, 128)) * np.exp(rng.uniform(-3, 3, (n, H, 1)))).astype(np.float32)
        v = rng.standard_normal((n, H, 128)).astype(np.float32)
        kc, ks, vc, vs = oracle.mx_quantize_append(planes, k, v, synth.slots_for(bt[b], 0, n))
        rows[b] = (oracle.mx_dequantize_rows(kc, ks).reshape(n, H, 128),
                   oracle.mx_dequantize_rows(vc, vs).reshape(n, H, 128))
    q = rng.standard_normal((len(lens), Hq, 128)).astype(np.float32)
    sm = np.float32(0.088)
    out = oracle.mx_decode_attention(planes, q, bt, np.array(lens, np.int32), sm).reshape(len(lens), Hq, 128)
    for b, n in enumerate(lens):
        for j in range(Hq):
            if n == 0:
                assert (out[b, j] == 0).all()
                continue
            K, V = rows[b]
            ref = _numpy_attention(q[b, j].astype(np.float64), K[:, j // 4], V[:, j // 4], float(sm))
            np.testing.assert_allclose(out[b, j], ref, rtol=1e-12, atol=1e-14)


def _kv(dist, frac, n=2048, H=8, which=0):
    return synth.kv_values(n, H, dist, frac, which, torch.float32, "cpu", 31).numpy()


@pytest.mark.parametrize("dist,frac", [("sparse6", 0.005), ("chan50", 0.0)])
def test_nvfp4_is_more_accurate_than_mxfp4(dist, frac):
    # direction of the pages' comparison: per-value error of the cached K/V and
    # error of the attention output that reads them
    for which in (0, 1):
        x = _kv(dist, frac, which=which).reshape(-1, 128)
        g = synth.global_scale(float(np.abs(x).max()))
        nv = oracle.dequantize_rows(*oracle.quantize_rows(x, g), g)
        mx = oracle.mx_dequantize_rows(*oracle.mx_quantize_rows(x))
        e_nv = np.sqrt(np.mean((nv - x) ** 2))
        e_mx = np.sqrt(np.mean((mx - x) ** 2))
        assert e_nv < e_mx, (which, e_nv, e_mx)


def test_smaller_blocks_lose_less():
    # [TC]: 16-value blocks beat 32-value blocks (the page's figure is ~30%
    # less error on its data); with the [MW] section-2 quantizer on Gaussian
    # values the 16-value block must at least be better
    x = np.random.default_rng(20261106).normal(0.0, 0.02, 1 << 16)
    e16 = np.sqrt(np.mean((oracle.unrounded_block_dequant(x, 16) - x) ** 2))
    e32 = np.sqrt(np.mean((oracle.unrounded_block_dequant(x, 32) - x) ** 2))
    assert e16 < e32
