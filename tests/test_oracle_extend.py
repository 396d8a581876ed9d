"""Pins of the oracle's FP8 rows of a new chunk and its extend attention.

The FP8 rows are checked by round trips of every E4M3 byte, exact midpoints
(ties to the even byte), saturation, signed zeros, PyTorch's float8_e4m3fn
conversion on exactly representable quotients, and skipped rows.  The extend
attention is checked against closed forms: one visible key, identical keys (the
mean of exactly the visible value rows, which fixes the causal limit), a zero
query, two keys (a sigmoid), invariance to keys after the causal limit, the
sequence and grouped-head mapping, how the two scales enter, and the decode
oracle on an exact FP8 image of an NVFP4 cache.
"""
import math

import numpy as np
import pytest
import torch

import oracle

E4M3 = np.array([oracle.e4m3_value(b) for b in range(0x7F)])  # non-negative finite bytes 0x00..0x7E


def _quant(x, scale):
    x = np.asarray(x, np.float32)
    if x.ndim == 1:
        x = x.reshape(-1, 1, 1) * np.ones((1, 1, 128), np.float32)
    T, H, _ = x.shape
    ws = np.zeros((T, H, 128), np.uint8)
    oracle.fp8_quantize_rows(x, np.arange(T), scale, ws)
    return ws


@pytest.mark.parametrize("scale", [0.125, 3.0])
def test_fp8_rows_round_trip_every_byte(scale):
    vals = (E4M3 * scale).astype(np.float32)
    assert np.all(vals.astype(np.float64) == E4M3 * scale)  # exact: <= 4 + 2 significant bits
    ws = _quant(vals, scale)
    assert np.array_equal(ws[:, 0, 0], np.arange(0x7F))
    ws = _quant(-vals, scale)
    assert np.array_equal(ws[:, 0, 0], np.arange(0x7F) | 0x80)


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_fp8_rows_midpoints_go_to_even(scale):
    mids = (E4M3[:-1] + E4M3[1:]) / 2
    x = (mids * scale).astype(np.float32)
    assert np.all(x.astype(np.float64) == mids * scale)
    ws = _quant(x, scale)[:, 0, 0]
    lo = np.arange(0x7E)
    assert np.array_equal(ws, np.where(lo % 2 == 0, lo, lo + 1))
    # a hair above / below a midpoint goes up / down
    up = _quant(np.nextafter(x, np.float32(np.inf)), scale)[:, 0, 0]
    dn = _quant(np.nextafter(x, np.float32(0)), scale)[:, 0, 0]
    assert np.array_equal(up, lo + 1) and np.array_equal(dn[1:], lo[1:])


def test_fp8_rows_saturation_zeros_and_torch():
    s = 0.5
    ws = _quant([448 * s, 464 * s, 1e30, -1e30, 0.0, -0.0, 2.0 ** -11, -2.0 ** -11], s)[:, 0, 0]
    assert list(ws) == [0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x00, 0x80]
    # PyTorch's float8_e4m3fn conversion (round to nearest even) on quotients exact in float32
    rng = np.random.default_rng(3)
    x = rng.normal(0, 40, (257, 2, 128)).astype(np.float32)
    x = np.clip(x, -440, 440)
    ws = np.zeros_like(x, dtype=np.uint8)
    oracle.fp8_quantize_rows(x, np.arange(257), 1.0, ws)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ws, ref)


def test_fp8_rows_layout_and_skips():
    rng = np.random.default_rng(4)
    T, H, cap = 9, 3, 20
    x = rng.normal(0, 1, (T, H, 128)).astype(np.float32)
    rows = np.array([5, -1, 0, 19, -7, 2, 11, 13, 7], np.int32)
    ws = np.full((cap, H, 128), 0x5A, np.uint8)
    oracle.fp8_quantize_rows(x, rows, 0.25, ws)
    for t, r in enumerate(rows):
        if r >= 0:
            assert np.array_equal(ws[r], _quant(x[t:t + 1], 0.25)[0])
    untouched = sorted(set(range(cap)) - {int(r) for r in rows if r >= 0})
    assert np.all(ws[untouched] == 0x5A)


# ---------------------------------------------------------------- attention
def _dec(ws):
    """E4M3 value of every byte of a workspace (float64)."""
    sgn = np.where(ws & 0x80, -1.0, 1.0)
    return sgn * E4M3[np.minimum(ws & 0x7F, 0x7E)]


def _layout(rng, prefixes, chunks, H, gap=3):
    """Per-sequence workspace rows [prefix | chunk] with gaps between sequences."""
    offs, at = [], 0
    for p, c in zip(prefixes, chunks):
        offs.append(at)
        at += p + c + gap
    qo = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return np.array(offs, np.int32), qo, at


def test_single_visible_key_gives_its_value():
    rng = np.random.default_rng(5)
    H, Hq = 2, 4
    kb = rng.integers(0, 0x7F, (6, H, 128)).astype(np.uint8) | (rng.integers(0, 2, (6, H, 128)) << 7).astype(np.uint8)
    vb = rng.integers(0, 0x7F, (6, H, 128)).astype(np.uint8)
    q = rng.normal(0, 1, (1, Hq, 128)).astype(np.float32)
    # prefill (empty prefix), first token: only key 0 is visible
    out = oracle.extend_attention(kb, vb, 0.5, 0.25, q, [0, 1], [2], [0], 0.1).reshape(Hq, 128)
    for qh in range(Hq):
        assert np.array_equal(out[qh], _dec(vb[2, qh // 2]) * 0.25)


def test_identical_keys_average_exactly_the_visible_rows():
    rng = np.random.default_rng(6)
    H, Hq = 2, 6
    prefixes, chunks = [5, 0, 17], [4, 6, 3]
    offs, qo, cap = _layout(rng, prefixes, chunks, H)
    kb = np.zeros((cap, H, 128), np.uint8)
    kb[:] = rng.integers(0, 0x7F, (1, H, 128)).astype(np.uint8)  # every key row the same (per head)
    vb = rng.integers(0, 0x7F, (cap, H, 128)).astype(np.uint8)
    q = rng.normal(0, 1, (int(qo[-1]), Hq, 128)).astype(np.float32)
    out = oracle.extend_attention(kb, vb, 1.0, 1.0, q, qo, offs, prefixes, 0.3).reshape(-1, Hq, 128)
    G = Hq // H
    for i, (p, c) in enumerate(zip(prefixes, chunks)):
        for j in range(c):
            for qh in range(Hq):
                rows = _dec(vb[offs[i]: offs[i] + p + j + 1, qh // G])
                np.testing.assert_allclose(out[qo[i] + j, qh], rows.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_zero_query_is_uniform():
    rng = np.random.default_rng(7)
    H, Hq = 1, 2
    kb = rng.integers(0, 0x7F, (30, H, 128)).astype(np.uint8)
    vb = rng.integers(0, 0x7F, (30, H, 128)).astype(np.uint8)
    q = np.zeros((3, Hq, 128), np.float32)
    out = oracle.extend_attention(kb, vb, 1.0, 2.0, q, [0, 3], [4], [10], 1.0).reshape(3, Hq, 128)
    for j in range(3):
        np.testing.assert_allclose(out[j, 0], 2.0 * _dec(vb[4:4 + 11 + j, 0]).mean(axis=0), rtol=1e-13)


def test_two_keys_is_a_sigmoid():
    rng = np.random.default_rng(8)
    kb = rng.integers(0, 0x60, (2, 1, 128)).astype(np.uint8)
    vb = rng.integers(0, 0x7F, (2, 1, 128)).astype(np.uint8)
    q = rng.normal(0, 1, (1, 1, 128)).astype(np.float32)
    sm, ks, vs = float(np.float32(0.07)), 0.5, 4.0  # the scales are float32 arguments
    out = oracle.extend_attention(kb, vb, ks, vs, q, [0, 1], [0], [1], sm)[0]
    s = [sm * float(np.dot(q[0, 0].astype(np.float64), _dec(kb[t, 0]) * ks)) for t in range(2)]
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    ref = vs * (p0 * _dec(vb[0, 0]) + (1 - p0) * _dec(vb[1, 0]))
    np.testing.assert_allclose(out, ref, rtol=1e-12)


def test_keys_after_the_causal_limit_do_not_matter():
    rng = np.random.default_rng(9)
    H, Hq = 2, 4
    prefixes, chunks = [7, 12], [5, 8]
    offs, qo, cap = _layout(rng, prefixes, chunks, H, gap=0)
    kb = rng.integers(0, 0x7F, (cap, H, 128)).astype(np.uint8)
    vb = rng.integers(0, 0x7F, (cap, H, 128)).astype(np.uint8)
    q = rng.normal(0, 1, (int(qo[-1]), Hq, 128)).astype(np.float32)
    base = oracle.extend_attention(kb, vb, 1.0, 1.0, q, qo, offs, prefixes, 0.2).reshape(-1, Hq, 128)
    for i, (p, c) in enumerate(zip(prefixes, chunks)):
        for j in range(c):
            k2, v2 = kb.copy(), vb.copy()
            lim = offs[i] + p + j  # last visible row
            k2[lim + 1:] ^= 0x11
            v2[lim + 1:] ^= 0x22
            o2 = oracle.extend_attention(k2, v2, 1.0, 1.0, q, qo, offs, prefixes, 0.2).reshape(-1, Hq, 128)
            assert np.array_equal(o2[qo[i] + j], base[qo[i] + j])
            v3 = vb.copy()
            v3[lim] ^= 0x22  # the last visible key does matter
            o3 = oracle.extend_attention(kb, v3, 1.0, 1.0, q, qo, offs, prefixes, 0.2).reshape(-1, Hq, 128)
            assert not np.array_equal(o3[qo[i] + j], base[qo[i] + j])


def test_sequences_and_grouped_heads_read_their_own_rows():
    rng = np.random.default_rng(10)
    H, Hq = 3, 6
    prefixes, chunks = [4, 9], [3, 2]
    offs, qo, cap = _layout(rng, prefixes, chunks, H)
    kb = rng.integers(0, 0x7F, (cap, H, 128)).astype(np.uint8)
    vb = np.zeros((cap, H, 128), np.uint8)
    for i in range(2):
        for h in range(H):
            vb[offs[i]: offs[i] + prefixes[i] + chunks[i], h] = 0x30 + 8 * i + h  # a constant per (sequence, head)
    q = rng.normal(0, 1, (int(qo[-1]), Hq, 128)).astype(np.float32)
    out = oracle.extend_attention(kb, vb, 1.0, 1.0, q, qo, offs, prefixes, 0.5).reshape(-1, Hq, 128)
    for i in range(2):
        for j in range(chunks[i]):
            for qh in range(Hq):
                np.testing.assert_allclose(out[qo[i] + j, qh], E4M3[0x30 + 8 * i + qh // 2], rtol=1e-14)


def test_scales_enter_as_logit_and_output_factors():
    rng = np.random.default_rng(11)
    kb = rng.integers(0, 0x7F, (20, 2, 128)).astype(np.uint8)
    vb = rng.integers(0, 0x7F, (20, 2, 128)).astype(np.uint8)
    q = rng.normal(0, 1, (4, 2, 128)).astype(np.float32)
    a = oracle.extend_attention(kb, vb, 2.0, 1.0, q, [0, 4], [1], [9], 0.25)
    b = oracle.extend_attention(kb, vb, 1.0, 1.0, q, [0, 4], [1], [9], 0.5)
    c = oracle.extend_attention(kb, vb, 1.0, 3.0, q, [0, 4], [1], [9], 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(c, 3.0 * b, rtol=1e-13)


def test_one_token_chunk_matches_decode_on_an_exact_fp8_image():
    """Power-of-two block scales, global scale and workspace scale make every
    dequantized NVFP4 value exactly representable in E4M3, so the FP8
    workspace is an exact image of the cache and extend == decode."""
    rng = np.random.default_rng(12)
    T, H, Hq = 45, 2, 4
    x = rng.normal(0, 1, (2, T, H, 128))
    planes = oracle.Planes(8, H)
    pages = rng.permutation(8)[:3].astype(np.int32)
    slots = (pages[np.arange(T) // 16] * 16 + np.arange(T) % 16).astype(np.int32)
    # codes and power-of-two scale bytes (mantissa 0) written straight into the planes
    codes = rng.integers(0, 256, (2, T * H, 64)).astype(np.uint8)
    scales = (rng.integers(4, 11, (2, T * H, 8)) << 3).astype(np.uint8)
    oracle.scatter_rows(codes[0], scales[0], slots, H, False, planes.k_codes, planes.k_scales)
    oracle.scatter_rows(codes[1], scales[1], slots, H, True, planes.v_codes, planes.v_scales)
    g, ws_scale = 0.5, 0.25
    bt = pages.reshape(1, -1)
    wk = oracle.fp8_workspace(planes, False, g, bt, [T], [0], ws_scale, T)
    wv = oracle.fp8_workspace(planes, True, g, bt, [T], [0], ws_scale, T)
    kh = oracle.dequantize_rows(codes[0], scales[0], g).reshape(T, H, 128)
    assert np.array_equal(_dec(wk) * ws_scale, kh)  # the image is exact
    q = rng.normal(0, 1, (1, Hq, 128)).astype(np.float32)
    dec = oracle.decode_attention(planes, g, g, q, bt, np.array([T], np.int32), 0.125)
    ext = oracle.extend_attention(wk, wv, ws_scale, ws_scale, q, [0, 1], [0], [T - 1], 0.125)
    np.testing.assert_allclose(ext, dec, rtol=1e-12, atol=1e-15)
