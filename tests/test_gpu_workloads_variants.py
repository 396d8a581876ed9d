"""Full-size parity, on sampled units, of the decode paths the benchmark times
beside plain NVFP4 decode, at the 70B-class shape (batch 32, 64 q / 8 kv
heads, 8192-token contexts, 16-token pages in random order): MXFP4,
Hadamard-rotated K, two query tokens per sequence, and the decode step that
appends its own new token.  Each layer is filled as the benchmark fills it
(same seeds, chunks and launch configuration); the oracle recomputes sampled
(sequence, kv head) units from the raw rows -- their cache bytes bit for bit
and their query heads' attention to 1e-3."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import ATTN_TOL, row_rel_err

pytestmark = pytest.mark.gpu

WL = "gqa70b_b32_8k"
SAMPLES = [(0, 0), (19, 5), (31, 7)]
SM = 1 / math.sqrt(128)
SMF = float(np.float32(SM))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _fill(fill_len, pool_len, mx=False, hadamard=False):
    """Fill layer 0 of the workload; return (workload, filled layer, raw rows of the sampled units)."""
    from synthetic.workloads import build_layer

    wl = synth.WORKLOADS[WL]
    lens = [fill_len] * wl.batch
    seq_start = np.concatenate([[0], np.cumsum(lens)])
    raw = {u: ([], []) for u in SAMPLES}

    def keep(c0, n, k, v, seq, pos):
        for (b, h) in SAMPLES:
            lo, hi = max(c0, seq_start[b]), min(c0 + n, seq_start[b + 1])
            if lo < hi:
                raw[(b, h)][0].append(k[lo - c0:hi - c0, h].float().cpu().numpy())
                raw[(b, h)][1].append(v[lo - c0:hi - c0, h].float().cpu().numpy())

    fl = build_layer(wl, lens, [pool_len] * wl.batch, 0, "cuda", on_chunk=keep, mx=mx, hadamard=hadamard)
    return wl, fl, {u: (np.concatenate(a), np.concatenate(b)) for u, (a, b) in raw.items()}


def _planes1(kc, ks, vc, vs, n):
    """A one-head NVFP4 cache holding rows 0..n-1 in order."""
    pages = (n + 15) // 16
    planes = oracle.Planes(pages, 1)
    local = np.arange(n, dtype=np.int32)
    oracle.scatter_rows(kc, ks, local, 1, False, planes.k_codes, planes.k_scales)
    oracle.scatter_rows(vc, vs, local, 1, True, planes.v_codes, planes.v_scales)
    return planes, np.arange(pages, dtype=np.int32)[None]


def _host_planes(layer):
    return tuple(getattr(layer, n).cpu().numpy() for n in ("k_codes", "k_scales", "v_codes", "v_scales"))


def _check_bytes(hp, fl, b, h, n, okc, oks, ovc, ovs, H):
    slots = synth.slots_for(fl.block_table[b], 0, n)
    sel = np.arange(n) * H + h
    gkc, gks = oracle.gather_rows(hp[0], hp[1], slots, H, False)
    gvc, gvs = oracle.gather_rows(hp[2], hp[3], slots, H, True)
    assert np.array_equal(gkc[sel], okc) and np.array_equal(gks[sel], oks), f"K bytes differ at unit {(b, h)}"
    assert np.array_equal(gvc[sel], ovc) and np.array_equal(gvs[sel], ovs), f"V bytes differ at unit {(b, h)}"


def test_mxfp4_full_size():
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: full-size MXFP4 {WL}, samples {SAMPLES}")
    wl, fl, raw = _fill(8192, 8192, mx=True)
    B, Hq, H, G, ctx = wl.batch, wl.q_heads, wl.kv_heads, wl.group, wl.ctx
    q = synth.queries(B, Hq, wl.in_dtype, "cuda", 4, 0)
    sl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    out = nk.mx_paged_decode_attn(fl.layer, q, fl.block_table_dev, sl, ctx, SM)
    torch.cuda.synchronize()
    out_h, q_h = out.cpu().numpy(), q.float().cpu().numpy()
    kc_g, ks_g = fl.layer.k_codes.cpu().numpy(), fl.layer.k_scales.cpu().numpy()
    vc_g, vs_g = fl.layer.v_codes.cpu().numpy(), fl.layer.v_scales.cpu().numpy()
    for (b, h) in SAMPLES:
        k_rows, v_rows = raw[(b, h)]
        n = k_rows.shape[0]
        slots = synth.slots_for(fl.block_table[b], 0, n)
        sel = np.arange(n) * H + h
        for rows, cp, sp, is_v in ((k_rows, kc_g, ks_g, False), (v_rows, vc_g, vs_g, True)):
            oc, os_ = oracle.mx_quantize_rows(rows)
            gc, gs = oracle.mx_gather_rows(cp, sp, slots, H, is_v)
            assert np.array_equal(gc[sel], oc) and np.array_equal(gs[sel], os_), f"MXFP4 bytes differ at {(b, h)}"
        planes = oracle.MxPlanes((n + 15) // 16, 1)
        oracle.mx_quantize_append(planes, k_rows[:, None], v_rows[:, None], np.arange(n, dtype=np.int32))
        ref = oracle.mx_decode_attention(planes, q_h[b:b + 1, h * G:(h + 1) * G].copy(),
                                         np.arange((n + 15) // 16, dtype=np.int32)[None], np.array([n], np.int32), SMF)
        err = row_rel_err(out_h[b, h * G:(h + 1) * G], ref)
        _say(f"  unit {(b, h)}: {n} tokens, bytes bit-exact, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL


def test_hadamard_k_full_size():
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: full-size Hadamard-rotated NVFP4 {WL}, samples {SAMPLES}")
    wl, fl, raw = _fill(8192, 8192, hadamard=True)
    B, Hq, H, G, ctx = wl.batch, wl.q_heads, wl.kv_heads, wl.group, wl.ctx
    g_k, g_v = fl.layer.k_global, fl.layer.v_global
    q = synth.queries(B, Hq, wl.in_dtype, "cuda", 4, 0)
    sl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    out = nk.paged_decode_attn(fl.layer, q, fl.block_table_dev, sl, ctx, SM, hadamard=True)
    torch.cuda.synchronize()
    out_h, hp = out.cpu().numpy(), _host_planes(fl.layer)
    q_rot = oracle.rotate_q(q.float().cpu().numpy()).astype(np.float32)
    for (b, h) in SAMPLES:
        k_rows, v_rows = raw[(b, h)]
        n = k_rows.shape[0]
        okc, oks = oracle.quantize_rows(oracle.rotate_k(k_rows), g_k)
        ovc, ovs = oracle.quantize_rows(v_rows, g_v)
        _check_bytes(hp, fl, b, h, n, okc, oks, ovc, ovs, H)
        planes, bt1 = _planes1(okc, oks, ovc, ovs, n)
        ref = oracle.decode_attention(planes, g_k, g_v, q_rot[b:b + 1, h * G:(h + 1) * G].copy(), bt1,
                                      np.array([n], np.int32), SMF)
        err = row_rel_err(out_h[b, h * G:(h + 1) * G], ref)
        _say(f"  unit {(b, h)}: {n} tokens, rotated bytes bit-exact, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL


def test_multi_token_full_size():
    """Two query tokens per sequence: token i of 2 sees the first ctx - 1 + i keys."""
    import nvfp4_quantized_paged_kv_amd as nk

    T = 2
    _say(f"case: full-size two-token decode {WL}, samples {SAMPLES}")
    wl, fl, raw = _fill(8192, 8192)
    B, Hq, H, G, ctx = wl.batch, wl.q_heads, wl.kv_heads, wl.group, wl.ctx
    g_k, g_v = fl.layer.k_global, fl.layer.v_global
    q = synth.queries(B * T, Hq, wl.in_dtype, "cuda", 5, 0).reshape(B, T, Hq, 128)
    sl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    out = nk.paged_decode_attn_multi(fl.layer, q, fl.block_table_dev, sl, ctx, SM)
    torch.cuda.synchronize()
    out_h, q_h, hp = out.cpu().numpy(), q.float().cpu().numpy(), _host_planes(fl.layer)
    for (b, h) in SAMPLES:
        k_rows, v_rows = raw[(b, h)]
        n = k_rows.shape[0]
        okc, oks = oracle.quantize_rows(k_rows, g_k)
        ovc, ovs = oracle.quantize_rows(v_rows, g_v)
        _check_bytes(hp, fl, b, h, n, okc, oks, ovc, ovs, H)
        planes, bt1 = _planes1(okc, oks, ovc, ovs, n)
        ref = oracle.decode_attention(planes, g_k, g_v, q_h[b, :, h * G:(h + 1) * G].copy(), np.repeat(bt1, T, 0),
                                      np.array([n - (T - 1 - i) for i in range(T)], np.int32), SMF)
        err = row_rel_err(out_h[b, :, h * G:(h + 1) * G], ref)
        _say(f"  unit {(b, h)}: {n} tokens, {T} query tokens, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL


def test_decode_step_full_size():
    """The step at full size: each sequence's new token (position ctx - 1) is
    quantized into its page (the append kernel, then the decode: 8K-token units
    take two launches), then the decode attends over ctx keys."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: full-size decode step {WL}, samples {SAMPLES}")
    wl, fl, raw = _fill(8192 - 1, 8192)
    B, Hq, H, G, ctx = wl.batch, wl.q_heads, wl.kv_heads, wl.group, wl.ctx
    g_k, g_v = fl.layer.k_global, fl.layer.v_global
    kn = synth.kv_values(B, H, wl.dist, wl.outlier_frac, 0, wl.in_dtype, "cuda", 3, 0)
    vn = synth.kv_values(B, H, wl.dist, wl.outlier_frac, 1, wl.in_dtype, "cuda", 3, 0)
    q = synth.queries(B, Hq, wl.in_dtype, "cuda", 4, 0)
    sl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    out = nk.paged_decode_step(fl.layer, kn.reshape(B, 1, H, 128), vn.reshape(B, 1, H, 128), q.reshape(B, 1, Hq, 128),
                               fl.block_table_dev, sl, ctx, SM)
    torch.cuda.synchronize()
    out_h, q_h = out.cpu().numpy().reshape(B, Hq, 128), q.float().cpu().numpy()
    kn_h, vn_h, hp = kn.float().cpu().numpy(), vn.float().cpu().numpy(), _host_planes(fl.layer)
    for (b, h) in SAMPLES:
        k_rows = np.concatenate([raw[(b, h)][0], kn_h[b:b + 1, h]])
        v_rows = np.concatenate([raw[(b, h)][1], vn_h[b:b + 1, h]])
        n = k_rows.shape[0]
        assert n == ctx
        okc, oks = oracle.quantize_rows(k_rows, g_k)
        ovc, ovs = oracle.quantize_rows(v_rows, g_v)
        _check_bytes(hp, fl, b, h, n, okc, oks, ovc, ovs, H)
        planes, bt1 = _planes1(okc, oks, ovc, ovs, n)
        ref = oracle.decode_attention(planes, g_k, g_v, q_h[b:b + 1, h * G:(h + 1) * G].copy(), bt1,
                                      np.array([n], np.int32), SMF)
        err = row_rel_err(out_h[b, h * G:(h + 1) * G], ref)
        _say(f"  unit {(b, h)}: {n} tokens incl. the new one, bytes bit-exact, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL
