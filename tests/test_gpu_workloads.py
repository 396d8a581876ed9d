"""Full-size parity on sampled outputs: each workload's cache is filled exactly
as the bench fills it (same seeds, chunks and launch configuration), decode
runs over the whole batch, and the oracle recomputes sampled (sequence,
kv head) units from the raw inputs: their codes and scale bytes bit for bit,
and their query heads' attention outputs to 1e-3."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import ATTN_TOL, row_rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_units(wl, lens, fl, samples, raw, q, out, g_k, g_v):
    """raw[(b, h)] = (k_rows, v_rows) float32 [len_b, 128] in position order."""
    Hq, H, G = wl.q_heads, wl.kv_heads, wl.group
    kc_gpu, ks_gpu = fl.layer.k_codes.cpu().numpy(), fl.layer.k_scales.cpu().numpy()
    vc_gpu, vs_gpu = fl.layer.v_codes.cpu().numpy(), fl.layer.v_scales.cpu().numpy()
    sm = float(np.float32(1 / math.sqrt(128)))
    for (b, h) in samples:
        n = lens[b]
        k_rows, v_rows = raw[(b, h)]
        assert k_rows.shape == (n, 128)
        # codes and scales: oracle quantizes the raw rows; compare with the GPU planes' bytes
        okc, oks = oracle.quantize_rows(k_rows, g_k)
        ovc, ovs = oracle.quantize_rows(v_rows, g_v)
        slots = synth.slots_for(fl.block_table[b], 0, n)
        gkc, gks = oracle.gather_rows(kc_gpu, ks_gpu, slots, H, False)
        gvc, gvs = oracle.gather_rows(vc_gpu, vs_gpu, slots, H, True)
        sel = np.arange(n) * H + h
        assert np.array_equal(gkc[sel], okc) and np.array_equal(gks[sel], oks), f"K bytes differ at unit {(b, h)}"
        assert np.array_equal(gvc[sel], ovc) and np.array_equal(gvs[sel], ovs), f"V bytes differ at unit {(b, h)}"
        # attention of the unit's query heads, from the oracle's own single-head cache
        pages = (n + 15) // 16
        planes = oracle.Planes(pages, 1)
        local = np.arange(n, dtype=np.int32)
        oracle.scatter_rows(okc, oks, local, 1, False, planes.k_codes, planes.k_scales)
        oracle.scatter_rows(ovc, ovs, local, 1, True, planes.v_codes, planes.v_scales)
        qg = q[b:b + 1, h * G:(h + 1) * G, :].copy()
        ref = oracle.decode_attention(planes, g_k, g_v, qg, np.arange(pages, dtype=np.int32)[None],
                                      np.array([n], np.int32), sm)
        got = out[b, h * G:(h + 1) * G, :]
        err = row_rel_err(got, ref)
        _say(f"  unit {(b, h)}: {n} tokens, codes bit-exact, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL, (b, h, err.max())


def _run(name, samples, layer_idx=0):
    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic.workloads import build_layer

    wl = synth.WORKLOADS[name]
    lens = [wl.ctx] * wl.batch
    seq_start = np.concatenate([[0], np.cumsum(lens)])
    raw = {u: ([], []) for u in samples}

    def keep(c0, n, k, v, seq, pos):
        for (b, h) in samples:
            lo, hi = max(c0, seq_start[b]), min(c0 + n, seq_start[b + 1])
            if lo < hi:
                raw[(b, h)][0].append(k[lo - c0:hi - c0, h].float().cpu().numpy())
                raw[(b, h)][1].append(v[lo - c0:hi - c0, h].float().cpu().numpy())

    _say(f"case: full-size {name}, samples {samples}")
    fl = build_layer(wl, lens, lens, layer_idx, "cuda", on_chunk=keep)
    raw = {u: (np.concatenate(a), np.concatenate(b)) for u, (a, b) in raw.items()}
    q = synth.queries(wl.batch, wl.q_heads, wl.in_dtype, "cuda", 4, layer_idx)
    sl = torch.full((wl.batch,), wl.ctx, dtype=torch.int32, device="cuda")
    out = nk.paged_decode_attn(fl.layer, q, fl.block_table_dev, sl, wl.ctx, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    _check_units(wl, lens, fl, samples, raw, q.float().cpu().numpy(), out.cpu().numpy(), fl.layer.k_global,
                 fl.layer.v_global)


def test_gqa70b_b32_8k_full_size():
    _run("gqa70b_b32_8k", [(0, 0), (17, 3), (31, 7)])


def test_long_b8_128k_full_size():
    """Four of the 64 units, the first and the last among them; with 64 units
    over 256 workgroups every unit's pages are shared by several workgroups,
    so each checked output went through the in-kernel merge."""
    _run("long_b8_128k", [(0, 0), (3, 4), (5, 6), (7, 7)])


def test_agentic_b1_2m_full_size():
    """All 8 kv heads of the 2,000,000-token sequence: every code and scale byte
    of the layer and all 96 query heads' outputs."""
    _run("agentic_b1_2m", [(0, h) for h in range(8)])


def test_mixed_64_full_size():
    """Ragged 64-sequence step: append 16/2048 tokens, FP8 workspace of 8 prefixes, decode of 56."""
    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic.workloads import build_mixed_step

    wl = synth.WORKLOADS["mixed_64"]
    lens = list(wl.lens)
    ext, dec = synth.mixed_roles(len(lens))
    H, G = wl.kv_heads, wl.group
    # sampled units: two decoding sequences (short and long) and one extended sequence
    dec_s = [int(dec[np.argmin(np.asarray(lens)[dec])]), int(dec[np.argmax(np.asarray(lens)[dec])])]
    ext_s = int(ext[0])
    samples = [(dec_s[0], 1), (dec_s[1], 6), (ext_s, 3)]
    seq_start = np.concatenate([[0], np.cumsum(lens)])
    raw = {u: ([], []) for u in samples}

    def keep(c0, n, k, v, seq, pos):
        for (b, h) in samples:
            lo, hi = max(c0, seq_start[b]), min(c0 + n, seq_start[b + 1])
            if lo < hi:
                raw[(b, h)][0].append(k[lo - c0:hi - c0, h].float().cpu().numpy())
                raw[(b, h)][1].append(v[lo - c0:hi - c0, h].float().cpu().numpy())

    _say(f"case: full-size mixed_64, samples {samples}")
    st = build_mixed_step(wl, 0, "cuda", on_chunk=keep)
    layer = st.filled.layer
    g_k, g_v = layer.k_global, layer.v_global
    raw = {u: (np.concatenate(a), np.concatenate(b)) for u, (a, b) in raw.items()}

    # the step, in the bench's order and launch configuration
    cap = int(st.ext_offsets[-1].item())
    ws_k = torch.zeros((cap, H, 128), dtype=torch.uint8, device="cuda")
    ws_v = torch.zeros_like(ws_k)
    nk.quantize_append(layer, st.new_k, st.new_v, st.new_slots)
    nk.dequant_to_fp8_workspace(layer, st.ext_table, st.ext_prefix, st.ext_offsets, st.max_prefix, 6 * g_k, 6 * g_v,
                                ws_k, ws_v)
    out = nk.paged_decode_attn(layer, st.dec_q, st.dec_table, st.dec_lens, st.max_dec_len, 1 / math.sqrt(128))
    torch.cuda.synchronize()

    # every new token's bytes
    nkf, nvf = st.new_k.float().cpu().numpy(), st.new_v.float().cpu().numpy()
    planes_new = oracle.Planes(layer.num_pages, H)
    oracle.quantize_append(planes_new, nkf, nvf, st.new_slots.cpu().numpy(), g_k, g_v)
    slots_new = st.new_slots.cpu().numpy()
    for name, is_v in (("k", False), ("v", True)):
        gc = getattr(layer, name + "_codes").cpu().numpy()
        gs = getattr(layer, name + "_scales").cpu().numpy()
        a = oracle.gather_rows(gc, gs, slots_new, H, is_v)
        b = oracle.gather_rows(getattr(planes_new, name + "_codes"), getattr(planes_new, name + "_scales"),
                               slots_new, H, is_v)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"new-token {name} bytes differ"
    _say(f"  {slots_new.size} new tokens: codes bit-exact")

    kc_gpu, ks_gpu = layer.k_codes.cpu().numpy(), layer.k_scales.cpu().numpy()
    vc_gpu, vs_gpu = layer.v_codes.cpu().numpy(), layer.v_scales.cpu().numpy()
    q_all = st.dec_q.float().cpu().numpy()
    out_h = out.cpu().numpy()
    wsk_h, wsv_h = ws_k.cpu().numpy(), ws_v.cpu().numpy()
    sm = float(np.float32(1 / math.sqrt(128)))
    for (b, h) in samples:
        n = lens[b]
        k_rows, v_rows = raw[(b, h)]
        okc, oks = oracle.quantize_rows(k_rows, g_k)
        ovc, ovs = oracle.quantize_rows(v_rows, g_v)
        slots = synth.slots_for(st.filled.block_table[b], 0, n)
        sel = np.arange(n) * H + h
        gkc, gks = oracle.gather_rows(kc_gpu, ks_gpu, slots, H, False)
        gvc, gvs = oracle.gather_rows(vc_gpu, vs_gpu, slots, H, True)
        assert np.array_equal(gkc[sel], okc) and np.array_equal(gks[sel], oks)
        assert np.array_equal(gvc[sel], ovc) and np.array_equal(gvs[sel], ovs)
        if b in ext:
            i = int(np.flatnonzero(ext == b)[0])
            off = int(st.ext_offsets[i].item())
            pages = (n + 15) // 16
            planes = oracle.Planes(pages, 1)
            local = np.arange(n, dtype=np.int32)
            oracle.scatter_rows(okc, oks, local, 1, False, planes.k_codes, planes.k_scales)
            oracle.scatter_rows(ovc, ovs, local, 1, True, planes.v_codes, planes.v_scales)
            bt1 = np.arange(pages, dtype=np.int32)[None]
            ref_k = oracle.fp8_workspace(planes, False, g_k, bt1, np.array([n], np.int32), np.array([0, n], np.int32),
                                         6 * g_k, n)
            ref_v = oracle.fp8_workspace(planes, True, g_v, bt1, np.array([n], np.int32), np.array([0, n], np.int32),
                                         6 * g_v, n)
            assert np.array_equal(wsk_h[off:off + n, h], ref_k[:, 0]) and np.array_equal(wsv_h[off:off + n, h],
                                                                                          ref_v[:, 0])
            _say(f"  extend unit {(b, h)}: {n}-token prefix, workspace bytes bit-exact")
        else:
            # decode over the prefix plus this sequence's 16 new tokens
            mine = np.flatnonzero(st.new_seq == b)
            k_all = np.concatenate([k_rows, nkf[mine, h]])
            v_all = np.concatenate([v_rows, nvf[mine, h]])
            m = k_all.shape[0]
            ckc, cks = oracle.quantize_rows(k_all, g_k)
            cvc, cvs = oracle.quantize_rows(v_all, g_v)
            pages = (m + 15) // 16
            planes = oracle.Planes(pages, 1)
            local = np.arange(m, dtype=np.int32)
            oracle.scatter_rows(ckc, cks, local, 1, False, planes.k_codes, planes.k_scales)
            oracle.scatter_rows(cvc, cvs, local, 1, True, planes.v_codes, planes.v_scales)
            i = int(np.flatnonzero(dec == b)[0])
            qg = q_all[i:i + 1, h * G:(h + 1) * G].copy()
            ref = oracle.decode_attention(planes, g_k, g_v, qg, np.arange(pages, dtype=np.int32)[None],
                                          np.array([m], np.int32), sm)
            err = row_rel_err(out_h[i, h * G:(h + 1) * G], ref)
            _say(f"  decode unit {(b, h)}: {m} tokens, attention max row rel err {err.max():.2e}")
            assert err.max() <= ATTN_TOL
