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
from nvfp4_quantized_paged_kv_amd import synth
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
    from nvfp4_quantized_paged_kv_amd.workloads import build_layer

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
    _run("long_b8_128k", [(5, 6)])


def test_agentic_b1_2m_full_size():
    _run("agentic_b1_2m", [(0, 2)])
