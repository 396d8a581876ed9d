"""Pins of the oracle's paged layout, decode attention and FP8 workspace.

Checked against closed forms (one token, identical keys, zero query), against
PyTorch's float64 softmax attention on the logically ordered dequantized cache
(brute force on tiny inputs), and against PyTorch's float8_e4m3fn conversion
and an exact rational search for the workspace bytes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _cache(rng, T, H, num_pages=None, g_k=1.0, g_v=1.0, outliers=0.005):
    """Random K/V (float32 [T, H, 128]) appended at random slots of a page pool."""
    k = rng.normal(0, 0.02, (T, H, 128)).astype(np.float32)
    v = rng.normal(0, 0.02, (T, H, 128)).astype(np.float32)
    for x in (k, v):
        m = rng.random(x.shape) < outliers
        x[m] = rng.choice([-6.0, 6.0], m.sum())
    n_pages = num_pages or (T + 15) // 16 + 3
    pages = rng.permutation(n_pages)[: (T + 15) // 16].astype(np.int32)
    slots = (pages[np.arange(T) // 16] * 16 + np.arange(T) % 16).astype(np.int32)
    planes = oracle.Planes(n_pages, H)
    kc, ks, vc, vs = oracle.quantize_append(planes, k, v, slots, g_k, g_v)
    k_hat = oracle.dequantize_rows(kc, ks, g_k).reshape(T, H, 128)
    v_hat = oracle.dequantize_rows(vc, vs, g_v).reshape(T, H, 128)
    return planes, pages, slots, k_hat, v_hat


def test_layout_round_trip():
    rng = np.random.default_rng(1)
    T, H = 77, 3
    planes, pages, slots, _, _ = _cache(rng, T, H)
    k = rng.normal(0, 1, (T, H, 128)).astype(np.float32)
    kc, ks = oracle.quantize_rows(k, 0.01)
    for is_v in (False, True):
        cp = np.zeros_like(planes.k_codes)
        sp = np.zeros_like(planes.k_scales)
        oracle.scatter_rows(kc, ks, slots, H, is_v, cp, sp)
        c2, s2 = oracle.gather_rows(cp, sp, slots, H, is_v)
        assert np.array_equal(c2, kc) and np.array_equal(s2, ks)
        # every written byte belongs to exactly the written tiles: 72 bytes per (token, head)
        assert np.count_nonzero(sp) <= T * H * 8


def test_layout_tile_positions():
    """Spot-check the documented byte positions inside a (page, head) tile."""
    H = 2
    planes = oracle.Planes(4, H)
    row = np.zeros((1, H, 128), np.float32)
    row[0, 1, 37] = -6.0  # head 1, dim 37 (block 2, octet 4), amax 6, g 1 -> code 0xF, scale 1.0
    slot = np.array([3 * 16 + 9], np.int32)  # page 3, offset 9
    oracle.quantize_append(planes, row, row, slot, 1.0, 1.0)
    tile = (3 * H + 1)
    assert planes.k_codes[tile * 1024 + 9 * 64 + 37 // 2] == 0xF0  # odd dim -> high nibble
    assert planes.k_scales[tile * 128 + 9 * 8 + 2] == 0x38
    # V: one byte holds one dimension of slots 2k (low nibble) and 2k+1 (high)
    v_at = tile * 1024 + (9 // 4) * 256 + (37 // 8) * 16 + ((9 // 2) % 2) * 8 + (37 % 2) * 4 + (37 % 8) // 2
    assert planes.v_codes[v_at] == 0xF0  # odd slot -> high nibble
    assert planes.v_scales[tile * 128 + 2 * 16 + 9] == 0x38
    assert np.count_nonzero(planes.k_codes) == 1 and np.count_nonzero(planes.v_codes) == 1
    # the even neighbour (offset 8) at an even dimension lands in the low nibble of its own byte
    row2 = np.zeros((1, H, 128), np.float32)
    row2[0, 0, 100] = 6.0  # head 0, dim 100: code 0x7
    oracle.quantize_append(planes, row2, row2, np.array([3 * 16 + 8], np.int32), 1.0, 1.0)
    t0 = 3 * H
    assert planes.k_codes[t0 * 1024 + 8 * 64 + 50] == 0x07
    v2 = t0 * 1024 + (8 // 4) * 256 + (100 // 8) * 16 + ((8 // 2) % 2) * 8 + 0 * 4 + (100 % 8) // 2
    assert planes.v_codes[v2] == 0x07
    assert np.count_nonzero(planes.v_codes) == 2


def _sdpa_ref(q, k_hat, v_hat, sm_scale):
    """float64 attention of q [Hq,128] over logically ordered k_hat/v_hat [T,Hkv,128]."""
    Hq, Hkv = q.shape[0], k_hat.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, 128))
    for j in range(Hq):
        h = j // G
        kk = torch.from_numpy(k_hat[:, h, :])
        vv = torch.from_numpy(v_hat[:, h, :])
        qq = torch.from_numpy(q[j].astype(np.float64))
        p = torch.softmax((kk @ qq) * sm_scale, dim=0)
        out[j] = (p @ vv).numpy()
    return out


@pytest.mark.parametrize("T,Hkv,G", [(1, 1, 4), (15, 2, 2), (16, 1, 8), (17, 2, 3), (100, 2, 4)])
def test_decode_attention_matches_torch_softmax(T, Hkv, G):
    rng = np.random.default_rng(T * 100 + Hkv * 10 + G)
    planes, pages, slots, k_hat, v_hat = _cache(rng, T, Hkv, g_k=0.02, g_v=0.5)
    Hq = Hkv * G
    q = (rng.normal(0, 1, (1, Hq, 128)) * 3).astype(np.float32)
    bt = np.full((1, (T + 15) // 16 + 2), -1, np.int32)
    bt[0, : pages.size] = pages
    sm = 1 / math.sqrt(128)
    got = oracle.decode_attention(planes, 0.02, 0.5, q, bt, np.array([T], np.int32), sm)
    ref = _sdpa_ref(q[0], k_hat, v_hat, np.float32(sm))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_decode_attention_closed_forms():
    rng = np.random.default_rng(5)
    T, Hkv, G = 40, 2, 2
    planes, pages, slots, k_hat, v_hat = _cache(rng, T, Hkv)
    bt = pages[None, :].copy()
    q = rng.normal(0, 1, (1, Hkv * G, 128)).astype(np.float32)
    sm = 0.125
    # one token: the output is that token's dequantized V
    o1 = oracle.decode_attention(planes, 1.0, 1.0, q, bt, np.array([1], np.int32), sm)
    for j in range(Hkv * G):
        assert np.array_equal(o1[j], v_hat[0, j // G])
    # zero query: uniform weights, output = mean of V
    o0 = oracle.decode_attention(planes, 1.0, 1.0, np.zeros_like(q), bt, np.array([T], np.int32), sm)
    for j in range(Hkv * G):
        assert np.allclose(o0[j], v_hat[:, j // G].mean(0), rtol=1e-13, atol=1e-16)
    # empty sequence: zeros
    oe = oracle.decode_attention(planes, 1.0, 1.0, q, bt, np.array([0], np.int32), sm)
    assert not oe.any()


def test_decode_attention_identical_keys():
    rng = np.random.default_rng(9)
    T, H = 33, 1
    k = np.tile(rng.normal(0, 0.5, (1, H, 128)).astype(np.float32), (T, 1, 1))
    v = rng.normal(0, 0.5, (T, H, 128)).astype(np.float32)
    planes = oracle.Planes(4, H)
    slots = np.arange(T, dtype=np.int32)
    _, _, vc, vs = oracle.quantize_append(planes, k, v, slots, 1.0, 1.0)
    v_hat = oracle.dequantize_rows(vc, vs, 1.0).reshape(T, 128)
    q = rng.normal(0, 1, (1, 3, 128)).astype(np.float32)
    o = oracle.decode_attention(planes, 1.0, 1.0, q, np.arange(3, dtype=np.int32)[None], np.array([T], np.int32), 0.3)
    for j in range(3):
        assert np.allclose(o[j], v_hat.mean(0), rtol=1e-13, atol=1e-16)


def test_decode_attention_row_selection_and_batch():
    rng = np.random.default_rng(11)
    B, Hkv, G = 3, 2, 2
    lens = [5, 0, 37]
    planes = oracle.Planes(16, Hkv)
    bt = np.zeros((B, 4), np.int32)
    perm = rng.permutation(16).astype(np.int32)
    k_hats, v_hats = [], []
    for b in range(B):
        bt[b] = perm[4 * b: 4 * b + 4]
        T = lens[b]
        k = rng.normal(0, 0.1, (T, Hkv, 128)).astype(np.float32)
        v = rng.normal(0, 0.1, (T, Hkv, 128)).astype(np.float32)
        slots = (bt[b][np.arange(T) // 16] * 16 + np.arange(T) % 16).astype(np.int32)
        kc, ks, vc, vs = oracle.quantize_append(planes, k, v, slots, 0.05, 0.05)
        k_hats.append(oracle.dequantize_rows(kc, ks, 0.05).reshape(T, Hkv, 128))
        v_hats.append(oracle.dequantize_rows(vc, vs, 0.05).reshape(T, Hkv, 128))
    q = rng.normal(0, 1, (B, Hkv * G, 128)).astype(np.float32)
    rows = np.array([0, 3, 5, 8, 11], np.int64)
    got = oracle.decode_attention(planes, 0.05, 0.05, q, bt, np.array(lens, np.int32), 0.2, rows)
    for i, r in enumerate(rows):
        b, j = divmod(int(r), Hkv * G)
        if lens[b] == 0:
            assert not got[i].any()
            continue
        ref = _sdpa_ref(q[b, j:j + 1].repeat(Hkv * G, 0), k_hats[b], v_hats[b], np.float32(0.2))[j]
        assert np.allclose(got[i], ref, rtol=1e-12, atol=1e-15)


def _torch_e4m3_fr():
    b = torch.arange(0x7F, dtype=torch.uint8)
    return [Fraction(float(x)) for x in b.view(torch.float8_e4m3fn).to(torch.float64)]


def test_fp8_workspace_matches_exact_rational():
    rng = np.random.default_rng(3)
    T, H = 40, 2
    g = 0.01
    planes, pages, slots, k_hat, v_hat = _cache(rng, T, H, g_k=g, g_v=g)
    bt = np.stack([pages, pages])
    prefix = np.array([T, 13], np.int32)
    offs = np.array([0, T, T + 13], np.int32)
    ws_scale = 6 * g  # calibration amax/448 with amax = 448*6*g
    e4 = _torch_e4m3_fr()
    for is_v, xh in ((False, k_hat), (True, v_hat)):
        ws = oracle.fp8_workspace(planes, is_v, g, bt, prefix, offs, ws_scale, T + 13)
        assert np.array_equal(ws[T:], ws[:13])  # second sequence is the first 13 tokens again
        wsf = Fraction(float(np.float32(ws_scale)))
        for t in range(0, T, 3):
            for h in range(H):
                for d in range(0, 128, 5):
                    x = xh[t, h, d]
                    y = abs(Fraction(float(x))) / wsf
                    byte = min(range(0x7F), key=lambda c: (abs(y - e4[c]), c & 1))
                    if math.copysign(1.0, x) < 0:
                        byte |= 0x80
                    assert ws[t, h, d] == byte, (t, h, d, x)
        # and torch agrees wherever x_hat / ws_scale is exact in float32
        q = xh / np.float64(np.float32(ws_scale))
        q32 = q.astype(np.float32)
        ok = (q32.astype(np.float64) == q) & (np.abs(q) <= 448)
        ref = torch.from_numpy(q32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ws[:T][ok], ref[ok])
