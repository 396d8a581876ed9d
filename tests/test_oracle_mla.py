"""Pins of the oracle's Sparse-MLA latent cache (readings M1-M4 of the oracle):
NVFP4 latent rows of 576 values and sparse decode attention over listed slots.

* Quantizer: every byte against an exact rational brute force of the block rule
  (torch's E4M3 table, the page's E2M1 list, Fraction arithmetic), and the
  byte positions of single values.
* Decode: against a numpy float64 softmax attention over rows dequantized by
  the (separately pinned) GQA row dequantizer; closed forms -- one entry,
  every entry the same slot, a zero query, no valid entry, the rotary part
  alone deciding the weights; invariance under permutation and under added
  out-of-range entries; duplicates counted twice.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_formats import E4M3_FR, _magnitudes, bf_code, bf_scale_byte

D, DV = oracle.MLA_D, oracle.MLA_DV


def _rows(rng, n):
    x = rng.normal(0, 0.02, (n, D))
    out = rng.random((n, D)) < 0.01
    x[out] = rng.choice([-6.0, 6.0], out.sum())
    x[0, 100:132] = 0.0          # zero blocks
    if n > 2:
        x[1, 7] = -0.0
        x[2, 512:] *= 40.0       # a loud rotary part
    return x.astype(np.float32)


def _bf_row(row, g, mags):
    gf = Fraction(float(np.float32(g)))
    codes = np.zeros(D // 2, np.uint8)
    scales = np.zeros(D // 16, np.uint8)
    for b in range(D // 16):
        blk = [float(v) for v in row[16 * b:16 * b + 16]]
        sb = bf_scale_byte(max(abs(Fraction(v)) for v in blk), gf)
        scales[b] = sb
        for i, v in enumerate(blk):
            d = 16 * b + i
            codes[d // 2] |= bf_code(v, E4M3_FR[sb], gf, mags) << (4 * (d & 1))
    return codes, scales


@pytest.mark.parametrize("g", [1.0, 6.0 / 2688.0, 0.37])
def test_mla_quantizer_matches_exact_rational_brute_force(golden_dir, g):
    mags = _magnitudes(golden_dir)
    x = _rows(np.random.default_rng(5), 6)
    codes, scales = oracle.mla_quantize_rows(x, g)
    assert codes.shape == (6, 288) and scales.shape == (6, 36)
    for r in range(x.shape[0]):
        bc, bs = _bf_row(x[r], g, mags)
        assert np.array_equal(scales[r], bs), r
        assert np.array_equal(codes[r], bc), r


def test_mla_layout_byte_positions():
    """A single nonzero value at dim d lands in code byte d/2 (nibble d%2) and scale byte d/16."""
    for d in (0, 1, 15, 16, 511, 512, 575):
        x = np.zeros((1, D), np.float32)
        x[0, d] = 3.0
        codes, scales = oracle.mla_quantize_rows(x, 1.0)
        # amax 3 -> scale E4M3(0.5) = byte 0x30; 3 / 0.5 = 6 -> magnitude code 7
        assert np.flatnonzero(scales[0]).tolist() == [d // 16] and scales[0, d // 16] == 0x30
        assert np.flatnonzero(codes[0]).tolist() == [d // 2]
        assert codes[0, d // 2] == (7 << (4 * (d & 1)))


def _cache(rng, n_slots, g, fill=None):
    x = _rows(rng, n_slots) if fill is None else fill
    planes = oracle.MlaPlanes(n_slots)
    oracle.mla_quantize_append(planes, x, np.arange(n_slots), g)
    return planes


def _np_decode(planes, g, q, idx, sm):
    rows = oracle.mla_dequantize_rows(planes.codes, planes.scales, g)
    T, Hq, _ = q.shape
    out = np.zeros((T, Hq, DV))
    for t in range(T):
        sel = [int(s) for s in idx[t] if 0 <= s < planes.num_slots]
        if not sel:
            continue
        k = rows[sel]                                  # [n, 576]
        s = float(np.float32(sm)) * (q[t].astype(np.float64) @ k.T)   # [Hq, n]
        w = np.exp(s - s.max(1, keepdims=True))
        out[t] = (w / w.sum(1, keepdims=True)) @ k[:, :DV]
    return out


def test_mla_decode_matches_numpy_softmax_attention():
    rng = np.random.default_rng(11)
    n_slots, g, sm = 300, 6.0 / 2688.0, 1 / math.sqrt(D)
    planes = _cache(rng, n_slots, g)
    T, Hq, topk = 5, 16, 40
    q = (rng.normal(0, 1, (T, Hq, D)) * 3).astype(np.float32)
    idx = rng.integers(0, n_slots, (T, topk)).astype(np.int32)
    idx[0, :5] = -1                    # skipped
    idx[1, 3] = n_slots                # past the cache: skipped
    idx[2, :10] = idx[2, 0]            # a listed duplicate is one more term of the softmax
    idx[3, :] = -7                     # nothing valid: zeros
    got = oracle.mla_sparse_decode(planes, g, q, idx, sm)
    ref = _np_decode(planes, g, q, idx, sm)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    assert not got[3].any()


def test_mla_decode_closed_forms():
    rng = np.random.default_rng(12)
    n_slots, g, sm = 64, 0.01, 0.05
    planes = _cache(rng, n_slots, g)
    rows = oracle.mla_dequantize_rows(planes.codes, planes.scales, g)
    q = rng.normal(0, 1, (1, 4, D)).astype(np.float32)
    # one valid entry: its latent values
    one = np.array([[-1, 9, -1, n_slots + 3]], np.int32)
    out = oracle.mla_sparse_decode(planes, g, q, one, sm)
    assert np.array_equal(out[0], np.broadcast_to(rows[9, :DV], (4, DV)))
    # every entry the same slot
    same = np.full((1, 7), 21, np.int32)
    out = oracle.mla_sparse_decode(planes, g, q, same, sm)
    assert np.abs(out[0] - rows[21, :DV]).max() <= 1e-15
    # a zero query weighs every entry equally (a duplicate twice)
    lst = np.array([[3, 5, 5, 40]], np.int32)
    out = oracle.mla_sparse_decode(planes, g, np.zeros((1, 4, D), np.float32), lst, sm)
    mean = (rows[3, :DV] + 2 * rows[5, :DV] + rows[40, :DV]) / 4
    assert np.abs(out[0] - mean).max() <= 1e-15
    # permuted list, and out-of-range entries added: the same output
    lst = rng.permutation(n_slots)[:20].astype(np.int32)[None]
    base = oracle.mla_sparse_decode(planes, g, q, lst, sm)
    perm = oracle.mla_sparse_decode(planes, g, q, lst[:, ::-1].copy(), sm)
    padded = oracle.mla_sparse_decode(planes, g, q, np.concatenate([lst, [[-1, -2, n_slots]]], 1).astype(np.int32),
                                      sm)
    assert np.abs(base - perm).max() <= 1e-14 and np.abs(base - padded).max() <= 1e-15


def test_mla_scores_use_the_rotary_part_and_output_only_the_latent():
    """A query that is zero on the 512 latent dims weighs entries by their 64
    rotary values alone (two entries: a logistic weight), and the 64 rotary
    values never reach the output."""
    rng = np.random.default_rng(13)
    x = _rows(rng, 2)
    planes = _cache(rng, 2, 1.0, fill=x)
    rows = oracle.mla_dequantize_rows(planes.codes, planes.scales, 1.0)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, DV:] = rng.normal(0, 1, D - DV)
    sm = 0.3
    out = oracle.mla_sparse_decode(planes, 1.0, q, np.array([[0, 1]], np.int32), sm)
    s = [float(np.float32(sm)) * float(q[0, 0, DV:].astype(np.float64) @ rows[j, DV:]) for j in (0, 1)]
    w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    ref = w0 * rows[0, :DV] + (1 - w0) * rows[1, :DV]
    assert np.abs(out[0, 0] - ref).max() <= 1e-14
    # changing the cached rows' rotary values under a latent-only query leaves the output unchanged
    q2 = rng.normal(0, 1, (1, 1, D)).astype(np.float32)
    q2[0, 0, DV:] = 0.0
    x2 = x.copy()
    x2[:, DV:] = rng.normal(0, 1, (2, D - DV))
    planes2 = _cache(rng, 2, 1.0, fill=x2)
    a = oracle.mla_sparse_decode(planes, 1.0, q2, np.array([[0, 1]], np.int32), sm)
    b = oracle.mla_sparse_decode(planes2, 1.0, q2, np.array([[0, 1]], np.int32), sm)
    assert np.array_equal(a, b)
