"""GPU parity of the MXFP4 comparison format through the C ABI: quantize-append
bytes bit-exact against the oracle, decode attention within 1e-3 of the
oracle's float64 attention (row-normalised), at small ragged sizes and on
sampled units of the full 70B-class decode batch (32 sequences x 8192 tokens,
64 query / 8 kv heads) as the bench runs it."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import ATTN_TOL, host_f32, row_rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _wide(n, H, which, seed):
    """Gaussian values with a random power of two (2^-40 .. 2^40) per 32-value
    block, so block scales span most of the E8M0 range the data can reach."""
    g = torch.Generator().manual_seed(seed * 2 + which)
    x = torch.randn((n, H, 128), generator=g)
    e = torch.randint(-40, 41, (n, H, 4), generator=g).repeat_interleave(32, dim=2).float()
    return x * torch.exp2(e)


def _kv(n, H, dtype, dist, seed, b, which):
    if dist == "wide":
        return _wide(n, H, which, seed * 1000 + b).to(dtype)
    frac = 0.005 if dist == "sparse6" else 0.0
    return synth.kv_values(n, H, dist, frac, which, dtype, "cpu", seed, b)


def _build(lens, H, dtype, dist, seed, extra_pages=3):
    import nvfp4_quantized_paged_kv_amd as nk

    bt, pool = synth.page_tables(lens, sum((n + 15) // 16 for n in lens) + extra_pages, seed=seed)
    ks, vs, slots = [], [], []
    for b, n in enumerate(lens):
        if n:
            ks.append(_kv(n, H, dtype, dist, seed, b, 0))
            vs.append(_kv(n, H, dtype, dist, seed, b, 1))
            slots.append(synth.slots_for(bt[b], 0, n))
    k, v = torch.cat(ks), torch.cat(vs)
    sl = np.concatenate(slots)
    planes = oracle.MxPlanes(pool, H)
    oracle.mx_quantize_append(planes, host_f32(k), host_f32(v), sl)
    layer = nk.MxKVCacheLayer.allocate(pool, H)
    nk.mx_quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    return layer, planes, bt


def _planes_diff(layer, planes):
    bad = []
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        g, o = getattr(layer, name).cpu().numpy(), getattr(planes, name)
        if not np.array_equal(g, o):
            i = np.flatnonzero(g != o)
            bad.append((name, int(i.size), int(i[0]), int(g[i[0]]), int(o[i[0]])))
    return bad


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dist", ["sparse6", "chan50", "wide"])
def test_mx_append_bit_exact(dtype, dist):
    lens = [1, 15, 16, 17, 100, 257]
    _say(f"case: mx append {dtype} {dist} lens {lens}")
    layer, planes, _ = _build(lens, 4, dtype, dist, seed=41)
    assert _planes_diff(layer, planes) == []


def test_mx_append_ties_saturation_and_signed_zero():
    import nvfp4_quantized_paged_kv_amd as nk

    # one token, 2 heads: blocks with amax 6 holding every midpoint, values
    # above 6X, negative zeros and an all-zero block
    row = np.zeros((1, 2, 128), np.float32)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    row[0, 0, 0] = 6.0
    row[0, 0, 1:8] = mids
    row[0, 0, 8:15] = -np.array(mids)
    row[0, 0, 32] = 7.9
    row[0, 0, 33] = -7.5
    row[0, 0, 34] = -0.0
    row[0, 1, 64:96] = -0.0          # a block of negative zeros
    row[0, 1, 0] = 2.0 ** -130        # subnormal amax: scale byte 0
    row[0, 1, 1] = -(2.0 ** -131)
    planes = oracle.MxPlanes(2, 2)
    oracle.mx_quantize_append(planes, row, row, [5])
    layer = nk.MxKVCacheLayer.allocate(2, 2)
    x = torch.from_numpy(row).cuda()
    nk.mx_quantize_append(layer, x, x, torch.tensor([5], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert _planes_diff(layer, planes) == []


def test_mx_append_skips_bad_slots():
    import nvfp4_quantized_paged_kv_amd as nk

    H, pool = 2, 4
    k = torch.randn((5, H, 128), generator=torch.Generator().manual_seed(3))
    v = torch.randn((5, H, 128), generator=torch.Generator().manual_seed(4))
    slots = np.array([0, -1, 17, pool * 16, 63], np.int32)
    planes = oracle.MxPlanes(pool, H)
    ok = np.where((slots >= 0) & (slots < pool * 16), slots, -1).astype(np.int32)
    oracle.mx_quantize_append(planes, k.numpy(), v.numpy(), ok)
    layer = nk.MxKVCacheLayer.allocate(pool, H)
    nk.mx_quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert _planes_diff(layer, planes) == []


def _decode_both(layer, planes, bt, lens, Hq, q_dtype, seed, max_seq_len=None, q_scale=1.0):
    import nvfp4_quantized_paged_kv_amd as nk

    B = len(lens)
    q = (synth.queries(B, Hq, torch.float32, "cpu", seed, 1) * q_scale).to(q_dtype)
    msl = max(max(lens), 1) if max_seq_len is None else max_seq_len
    need = (msl + 15) // 16
    if bt.shape[1] < need:
        bt = np.concatenate([bt, np.zeros((B, need - bt.shape[1]), np.int32)], 1)
    sm = 1 / math.sqrt(128)
    out = nk.mx_paged_decode_attn(layer, q.cuda().contiguous(), torch.from_numpy(np.ascontiguousarray(bt)).cuda(),
                                  torch.tensor(lens, dtype=torch.int32, device="cuda"), msl, sm)
    torch.cuda.synchronize()
    ref = oracle.mx_decode_attention(planes, host_f32(q), bt, np.array(lens, np.int32), float(np.float32(sm)))
    return out.cpu().numpy().reshape(B * Hq, 128), ref


@pytest.mark.parametrize("lens,H,G,q_dtype,dist", [
    ([256, 77], 2, 4, torch.bfloat16, "sparse6"),
    ([1, 15, 16, 17, 33, 0, 300], 2, 8, torch.float32, "sparse6"),
    ([513, 40, 1000], 1, 16, torch.bfloat16, "chan50"),
    ([700, 5, 129], 4, 1, torch.float32, "chan50"),
    ([200, 64, 31], 2, 12, torch.bfloat16, "wide"),
    ([90, 300], 2, 8, torch.float32, "wide"),
])
def test_mx_decode_matches_oracle(lens, H, G, q_dtype, dist):
    _say(f"case: mx decode lens {lens} H {H} G {G} q {q_dtype} {dist}")
    layer, planes, bt = _build(lens, H, torch.bfloat16, dist, seed=53)
    # wide: K blocks reach 2^42, so Q is scaled by 2^-40 to keep the logits
    # where an fp32 softmax resolves them (the block scales still span 2^+-40)
    got, ref = _decode_both(layer, planes, bt, lens, H * G, q_dtype, seed=7,
                            q_scale=2.0 ** -40 if dist == "wide" else 1.0)
    err = row_rel_err(got, ref)
    _say(f"  max row rel err {err.max():.2e}")
    assert err.max() <= ATTN_TOL
    for b, n in enumerate(lens):
        if n == 0:
            assert (got.reshape(len(lens), H * G, 128)[b] == 0).all()


def test_mx_decode_huge_logits_stay_finite():
    # logits near 1e13 (wide K, unscaled Q): the softmax weights must neither
    # overflow nor all vanish; the output is a convex combination of V rows
    lens = [200, 64, 31]
    _say(f"case: mx decode huge logits lens {lens}")
    layer, planes, bt = _build(lens, 2, torch.bfloat16, "wide", seed=53)
    got, ref = _decode_both(layer, planes, bt, lens, 24, torch.bfloat16, seed=7)
    assert np.isfinite(got).all()
    vmax = np.abs(oracle.mx_dequantize_rows(*oracle.mx_gather_rows(
        planes.v_codes, planes.v_scales, np.arange(planes.num_pages * 16, dtype=np.int32), 2, True))).max()
    assert np.abs(got).max() <= vmax * (1 + 1e-3)
    err = row_rel_err(got, ref)
    _say(f"  finite; max row rel err vs oracle {err.max():.2e}")
    assert err.max() <= ATTN_TOL  # the softmax is one-hot here and the scores are far apart


def test_mx_decode_long_split_and_larger_bound():
    # a sequence long enough to be split across workgroups, and a launch bound
    # above every length (pages past the end are never read)
    lens = [20000, 3, 4100]
    _say(f"case: mx decode split lens {lens}")
    layer, planes, bt = _build(lens, 2, torch.bfloat16, "sparse6", seed=61)
    got, ref = _decode_both(layer, planes, bt, lens, 16, torch.bfloat16, seed=9, max_seq_len=24000)
    err = row_rel_err(got, ref)
    _say(f"  max row rel err {err.max():.2e}")
    assert err.max() <= ATTN_TOL


def test_mx_full_size_sampled():
    """The bench's MXFP4 decode: the 70B-class batch filled as the bench fills it."""
    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic.workloads import build_layer

    wl = synth.WORKLOADS["gqa70b_b32_8k"]
    lens = [wl.ctx] * wl.batch
    samples = [(0, 0), (13, 5), (31, 7)]
    seq_start = np.concatenate([[0], np.cumsum(lens)])
    raw = {u: ([], []) for u in samples}

    def keep(c0, n, k, v, seq, pos):
        for (b, h) in samples:
            lo, hi = max(c0, seq_start[b]), min(c0 + n, seq_start[b + 1])
            if lo < hi:
                raw[(b, h)][0].append(k[lo - c0:hi - c0, h].float().cpu().numpy())
                raw[(b, h)][1].append(v[lo - c0:hi - c0, h].float().cpu().numpy())

    _say(f"case: mx full-size {wl.name}, samples {samples}")
    fl = build_layer(wl, lens, lens, 0, "cuda", on_chunk=keep, mx=True)
    q = synth.queries(wl.batch, wl.q_heads, wl.in_dtype, "cuda", 4, 0)
    sl = torch.full((wl.batch,), wl.ctx, dtype=torch.int32, device="cuda")
    out = nk.mx_paged_decode_attn(fl.layer, q, fl.block_table_dev, sl, wl.ctx, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    out, q = out.cpu().numpy(), host_f32(q)
    H, G = wl.kv_heads, wl.group
    kc, ks = fl.layer.k_codes.cpu().numpy(), fl.layer.k_scales.cpu().numpy()
    vc, vs = fl.layer.v_codes.cpu().numpy(), fl.layer.v_scales.cpu().numpy()
    for (b, h) in samples:
        n = lens[b]
        k_rows, v_rows = np.concatenate(raw[(b, h)][0]), np.concatenate(raw[(b, h)][1])
        okc, oks = oracle.mx_quantize_rows(k_rows)
        ovc, ovs = oracle.mx_quantize_rows(v_rows)
        slots = synth.slots_for(fl.block_table[b], 0, n)
        gkc, gks = oracle.mx_gather_rows(kc, ks, slots, H, False)
        gvc, gvs = oracle.mx_gather_rows(vc, vs, slots, H, True)
        sel = np.arange(n) * H + h
        assert np.array_equal(gkc[sel], okc) and np.array_equal(gks[sel], oks), f"K bytes differ at {(b, h)}"
        assert np.array_equal(gvc[sel], ovc) and np.array_equal(gvs[sel], ovs), f"V bytes differ at {(b, h)}"
        pages = (n + 15) // 16
        planes = oracle.MxPlanes(pages, 1)  # the unit alone, from the raw rows
        oracle.mx_quantize_append(planes, k_rows[:, None, :], v_rows[:, None, :], np.arange(n, dtype=np.int32))
        ref = oracle.mx_decode_attention(planes, q[b:b + 1, h * G:(h + 1) * G], np.arange(pages, dtype=np.int32)[None],
                                         np.array([n], np.int32), float(np.float32(1 / math.sqrt(128))))
        err = row_rel_err(out[b, h * G:(h + 1) * G], ref)
        _say(f"  unit {(b, h)}: bytes bit-exact, attention max row rel err {err.max():.2e}")
        assert err.max() <= ATTN_TOL
