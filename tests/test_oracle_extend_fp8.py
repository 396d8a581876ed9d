"""Pins of the oracle's extend attention in FP8 arithmetic (reading R11).

Checked against an independent statement built on PyTorch's float8_e4m3fn
casts (library rounding to nearest even for Q and the weights, library decoding
of the workspace bytes); against the exact extend oracle where every rounding
is exact (integer base-2 logits, Q already on the E4M3 grid); by exact
invariance to a power-of-two scale of Q; by identical keys (the mean of exactly
the visible value rows); and the comparison bound's own properties.
"""
import math

import numpy as np
import pytest
import torch

import oracle

LOG2E = 1.4426950408889634


def _workspace(rng, T, H):
    """Random finite E4M3 bytes (no NaN 0x7F / 0xFF), either sign."""
    b = rng.integers(0, 0x7F, (T, H, 128)).astype(np.uint8)
    return b | (rng.integers(0, 2, (T, H, 128)).astype(np.uint8) << 7)


def _torch_reference(ws_k, ws_v, ks, vs, q, qo, offs, pl, sm, rows):
    """The same attention from the definition, with torch doing every E4M3 cast and decode."""
    dec = lambda b: torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    K, V = dec(ws_k), dec(ws_v)
    Tq, Hq, _ = q.shape
    G = Hq // ws_k.shape[1]
    c = float(np.float32(sm * ks * LOG2E))
    out = np.zeros((len(rows), 128))
    for n, rr in enumerate(rows):
        qrow, qh = divmod(int(rr), Hq)
        i = int(np.searchsorted(qo, qrow, side="right") - 1)
        j = qrow - qo[i]
        keys = np.arange(pl[i] + j + 1) + offs[i]
        qv = (q[qrow, qh] * np.float32(c)).astype(np.float64)  # float32 products
        amax = np.abs(qv).max()
        E = 0
        if amax > 0:
            E = math.ceil(math.log2(amax / 448.0)) - 2
            while amax > 448.0 * 2.0 ** E:
                E += 1
        q8 = torch.from_numpy((qv * 2.0 ** -E).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        x = (K[keys, qh // G] @ q8) * 2.0 ** E
        M = math.ceil(x.max())
        y = np.exp2(x - M + (8.0 if abs(M) < 2.0 ** 27 else 0.0)).astype(np.float32)
        w = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        out[n] = vs * (w @ V[keys, qh // G]) / w.sum()
    return out


@pytest.mark.parametrize("sm", [0.088, -0.3, 1e12])
def test_fp8_extend_matches_torch_casts(sm):
    rng = np.random.default_rng({0.088: 5, -0.3: 6}.get(sm, 7))
    H, Hq = 2, 4
    prefixes, chunks = [7, 0, 20], [3, 5, 2]
    offs = np.array([0, 12, 20], np.int32)
    cap = 45
    ws_k, ws_v = _workspace(rng, cap, H), _workspace(rng, cap, H)
    qo = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = (rng.normal(0, 1, (int(qo[-1]), Hq, 128)) * np.exp(rng.normal(0, 2, (int(qo[-1]), Hq, 1)))).astype(np.float32)
    q[0, 0, :5] = [0.0, -0.0, 1e-30, -1e-30, 0.0]  # zeros and values far below the row's E4M3 grid
    q[1, 1] = 0.0                                   # a zero row
    ks, vs = 0.02, 0.5
    rows = np.arange(int(qo[-1]) * Hq, dtype=np.int64)
    got, tol = oracle.extend_attention_fp8(ws_k, ws_v, ks, vs, q, qo, offs, np.array(prefixes, np.int32), sm, rows)
    want = _torch_reference(ws_k, ws_v, ks, vs, q, qo, offs, prefixes, sm, rows)
    scale = np.abs(want).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - want) <= 1e-12 * scale + 1e-300)
    assert np.all(np.isfinite(tol)) and np.all(tol >= 0)


def test_fp8_extend_equals_exact_oracle_when_every_rounding_is_exact():
    """Q on the E4M3 grid with max 448 (E = 0), logit scale exactly 1, one-hot unit
    keys picking integer query entries: base-2 logits are integers within 14 of
    the maximum, so every weight 2^(x - M + 8) is an E4M3 value and the FP8
    statement is the exact softmax."""
    H, Hq = 1, 2
    prefixes, chunks = [10], [4]
    cap = 14
    ks = 0.5
    sm = 1.0 / (ks * LOG2E)
    assert np.float32(sm * ks * LOG2E) == 1.0
    ws_k = np.zeros((cap, H, 128), np.uint8)
    pick = [3, 7, 1, 12, 9, 2, 11, 5, 8, 4, 6, 10, 13, 0]  # dims; q[d] = d + 1 (integers on the grid)
    for t, d in enumerate(pick):
        ws_k[t, 0, d] = 0x38  # E4M3 1.0
    rng = np.random.default_rng(9)
    ws_v = _workspace(rng, cap, H)
    q = np.zeros((4, Hq, 128), np.float32)
    q[:, :, :14] = np.arange(1, 15, dtype=np.float32)
    q[:, :, 100] = 448.0  # fixes E = 0; never picked by a key
    q[:, 1, :14] *= -1    # second head: logits negated (still integers)
    offs = np.array([0], np.int32)
    qo = np.array([0, 4], np.int32)
    pl = np.array(prefixes, np.int32)
    got, tol = oracle.extend_attention_fp8(ws_k, ws_v, ks, 0.25, q, qo, offs, pl, sm)
    exact = oracle.extend_attention(ws_k, ws_v, ks, 0.25, q, qo, offs, pl, sm)
    # the exact oracle takes sm_scale as float32 (2^-24 relative), which moves its
    # natural-log logits off the integers by up to 14 * 2^-24: weights by 14 ln2 2^-24
    assert np.allclose(got, exact, rtol=0, atol=2e-6 * np.abs(exact).max())
    # no weight near a rounding midpoint: only the accumulation terms (and small weights) remain
    assert np.all(tol <= 0.02 * np.abs(exact).max(axis=1))


def test_fp8_extend_power_of_two_scale_of_q_changes_nothing():
    rng = np.random.default_rng(11)
    H, Hq = 2, 8
    ws_k, ws_v = _workspace(rng, 60, H), _workspace(rng, 60, H)
    qo = np.array([0, 9], np.int32)
    q = rng.normal(0, 0.3, (9, Hq, 128)).astype(np.float32)
    args = (np.array([0], np.int32), np.array([51], np.int32), 0.088)
    base, _ = oracle.extend_attention_fp8(ws_k, ws_v, 0.01, 0.02, q, qo, *args)
    for k in (-20, 3, 40):
        got, _ = oracle.extend_attention_fp8(ws_k, ws_v, 0.01, 0.02, q * np.float32(2.0 ** k), qo, args[0], args[1],
                                             args[2] * 2.0 ** -k)
        assert np.array_equal(got, base)


def test_fp8_extend_identical_keys_give_the_mean_of_visible_values():
    rng = np.random.default_rng(12)
    H, Hq = 1, 2
    prefixes, chunks = [5, 2], [3, 4]
    offs = np.array([0, 9], np.int32)
    ws_k = np.tile(_workspace(rng, 1, H), (20, 1, 1))
    ws_v = _workspace(rng, 20, H)
    qo = np.array([0, 3, 7], np.int32)
    q = rng.normal(0, 1, (7, Hq, 128)).astype(np.float32)
    got, _ = oracle.extend_attention_fp8(ws_k, ws_v, 0.1, 2.0, q, qo, offs, np.array(prefixes, np.int32), 0.088)
    V = np.array([oracle.e4m3_value(b & 0x7F) * (-1 if b & 0x80 else 1) for b in ws_v.reshape(-1)]).reshape(ws_v.shape)
    for qrow in range(7):
        i = 0 if qrow < 3 else 1
        n = prefixes[i] + (qrow - qo[i]) + 1
        want = 2.0 * V[offs[i]:offs[i] + n, 0].mean(axis=0)
        for qh in range(Hq):
            assert np.allclose(got[qrow * Hq + qh], want, rtol=1e-13, atol=1e-13)


def test_fp8_extend_bound_grows_near_midpoints():
    """Two keys: logit 0 (weight 2^8) and x = -a*b for E4M3 values a (in Q) and b
    (in K), logit scale exactly 1.  The pair is chosen so that 2^(x + 8) lies
    0.3-2% from an E4M3 midpoint: with nothing else in the row a kernel's
    float32 logit cannot cross it, so the bound is only the accumulation terms.
    Adding two cancelling products of 64 leaves x unchanged but lets the FP8
    matrix cores' accumulation move it by up to 2^-11 * 64: now the weight may
    round either way, and the bound takes that step."""
    H, Hq, ks = 1, 1, 0.5
    sm = 1.0 / (ks * LOG2E)
    assert np.float32(sm * ks * LOG2E) == 1.0
    vals = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    pick = None
    for ia in range(0x30, 0x48):        # a, b in [0.5, 4): x in (-16, -0.25]
        for ib in range(0x30, 0x48):
            y = 2.0 ** (8.0 - vals[ia] * vals[ib])
            if y < 0.25:
                continue
            rel = np.min(np.abs(mids - y)) / y
            if 0.003 <= rel <= 0.02:
                pick = (ia, ib, y)
                break
        if pick:
            break
    assert pick is not None
    ia, ib, y = pick
    w1 = vals[np.argmin(np.abs(vals - y))]
    ws_k = np.zeros((2, H, 128), np.uint8)
    ws_k[0, 0, 0] = 0x38        # key 0 meets q[0] = 0: logit 0
    ws_k[1, 0, 1] = 0x80 | ib   # key 1: -b against q[1] = a
    ws_v = np.zeros((2, H, 128), np.uint8)
    ws_v[0, 0, :] = 0x38
    ws_v[1, 0, :] = 0xB8
    q = np.zeros((1, Hq, 128), np.float32)
    q[0, 0, 1] = vals[ia]
    q[0, 0, 127] = 448.0        # E = 0
    qo, offs, pl = np.array([0, 1], np.int32), np.array([0], np.int32), np.array([1], np.int32)
    out_a, t_a = oracle.extend_attention_fp8(ws_k, ws_v, ks, 1.0, q, qo, offs, pl, sm)
    assert out_a[0, 0] == pytest.approx((256 - w1) / (256 + w1), abs=1e-15)
    q[0, 0, 2] = q[0, 0, 3] = 64.0
    ws_k[1, 0, 2], ws_k[1, 0, 3] = 0x38, 0xB8   # +64 and -64: x unchanged
    out_b, t_b = oracle.extend_attention_fp8(ws_k, ws_v, ks, 1.0, q, qo, offs, pl, sm)
    assert out_b[0, 0] == out_a[0, 0]
    assert t_a[0] < 0.01 and t_b[0] > 4 * t_a[0]
