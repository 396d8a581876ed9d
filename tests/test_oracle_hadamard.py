"""Pins for the oracle's Hadamard rotation of K (and Q), CPU only.

cloud.tencent.com.cn "NVFP4: breaking the memory wall of GPU inference",
E2M1 encoding and two-level scaling section, quantization tricks: a Hadamard
transform applied before quantization is orthogonal and spreads a local
outlier over the whole vector (its example turns [0.1, 0.1, 0.1, 5.0] into
roughly equal entries; the printed numbers are illustrative).  The oracle
multiplies K rows by the 128-point Sylvester matrix times 2^-4 and queries by
the same matrix times 2^-3, so scores are unchanged.

Pins: the matrix against scipy's Hadamard construction and its own recursive
block structure, exact preservation of dot products on integer vectors, the
page's outlier example on the 4-point matrix, the mechanism (block maxima
evened out), and the direction of the page's claim where it holds: MXFP4 (one
power-of-two scale per 32 values) loses less on K with outlier channels, and
so do the scores.  NVFP4's 16-value E4M3 blocks already confine such outliers
to their own blocks; there the rotation spreads them into every block and the
error grows (not asserted; measured by the same oracle functions).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.linalg
import torch

import oracle
from synthetic import synth


def _matrix():
    return oracle.hadamard_rows(np.eye(128), 1.0)  # row i of the result is H e_i = column i = row i (symmetric)


def test_matrix_is_sylvester_hadamard():
    H = _matrix()
    assert np.array_equal(H, scipy.linalg.hadamard(128).astype(np.float64))
    assert np.array_equal(H @ H.T, 128 * np.eye(128))
    n = 128
    while n > 1:  # H_2m = [[H_m, H_m], [H_m, -H_m]]
        m = n // 2
        B = H[:n, :n]
        assert np.array_equal(B[:m, :m], B[:m, m:]) and np.array_equal(B[:m, :m], B[m:, :m])
        assert np.array_equal(B[m:, m:], -B[:m, :m])
        n = m
    assert H[0, 0] == 1.0


def test_scores_preserved_exactly():
    rng = np.random.default_rng(2)
    q = rng.integers(-100, 101, (50, 128)).astype(np.float64)
    k = rng.integers(-100, 101, (50, 128)).astype(np.float64)
    qr = oracle.hadamard_rows(q, oracle.Q_ROT_SCALE)
    kr = oracle.hadamard_rows(k, oracle.K_ROT_SCALE)
    assert np.array_equal((qr * kr).sum(1), (q * k).sum(1))
    assert np.array_equal(qr @ kr.T, q @ k.T)


def test_page_outlier_example_spreads():
    # the page's 4-value vector through the 4-point Sylvester matrix (the top
    # left 4x4 block), normalised by 1/2: the 5.0 is no longer in one place
    H4 = _matrix()[:4, :4]
    x = np.array([0.1, 0.1, 0.1, 5.0])
    y = H4 @ x / 2.0
    assert np.isclose(np.linalg.norm(y), np.linalg.norm(x))
    assert np.abs(y).max() < 0.6 * 5.0 and np.abs(y).min() > 2.3
    # and on a 128-value row: one outlier's energy is spread evenly
    x = np.full(128, 0.1)
    x[3] = 5.0
    y = oracle.hadamard_rows(x, 1 / math.sqrt(128))
    assert np.isclose(np.linalg.norm(y), np.linalg.norm(x))
    assert np.abs(y).max() < 1.6 and np.abs(np.abs(y[1:]) - 5.0 / math.sqrt(128)).max() < 0.1 * 127 / math.sqrt(128)


def _mx_roundtrip(x):
    return oracle.mx_dequantize_rows(*oracle.mx_quantize_rows(x))


def _chan50_k(n=2048, H=8, seed=7):
    return synth.kv_values(n, H, "chan50", 0.0, 0, torch.float32, "cpu", seed).numpy().reshape(-1, 128)


def test_rotation_evens_out_block_maxima():
    # the mechanism: two x50 channels make two of a row's eight 16-value
    # blocks far larger than the rest; after rotation every block sees them
    k = _chan50_k()
    kr = oracle.rotate_k(k).astype(np.float64)
    spread = lambda x: np.median(np.abs(x).reshape(-1, 8, 16).max(2).max(1) / np.abs(x).reshape(-1, 8, 16).max(2).min(1))
    assert spread(k) > 10.0 and spread(kr) < 2.0


def test_rotation_lowers_mxfp4_k_and_score_error_on_outlier_channels():
    # the page's claim, on the format with coarse blocks and power-of-two
    # scales: K rows and the scores q.k read back from MXFP4 lose less with the
    # rotation
    k = _chan50_k()
    back = oracle.hadamard_rows(_mx_roundtrip(oracle.rotate_k(k)), 1.0 / (128 * oracle.K_ROT_SCALE))  # H^T H = 128 I
    plain = _mx_roundtrip(k)
    e = lambda a: np.sqrt(np.mean((a - k) ** 2))
    assert e(back) < 0.8 * e(plain), (e(back), e(plain))
    q = synth.queries(64, 1, torch.float32, "cpu", 3).numpy().reshape(-1, 128).astype(np.float64)
    s_ref = q @ k.T.astype(np.float64)
    s_plain = q @ plain.T
    s_rot = oracle.rotate_q(q) @ _mx_roundtrip(oracle.rotate_k(k)).T  # the scores the rotated cache gives
    err = lambda s: np.sqrt(np.mean((s - s_ref) ** 2))
    assert err(s_rot) < 0.8 * err(s_plain), (err(s_rot), err(s_plain))
