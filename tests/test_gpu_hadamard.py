"""GPU parity of the Hadamard-rotated K path through the C ABI (both cache
formats): rotated quantize-append bytes bit-exact against the oracle (which
rotates by the matrix definition, then quantizes), and decode over the rotated
cache -- Q rotated in the kernel -- within 1e-3 of the oracle's float64
attention with the oracle's rotated Q."""
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


def _kv(n, H, dtype, dist, seed, b, which):
    x = synth.kv_values(n, H, dist, 0.005 if dist == "sparse6" else 0.0, which, torch.float32, "cpu", seed, b)
    if dtype == torch.float32:
        # float32 rows are rotated exactly (float64 sums) when their values span
        # at most 22 binades; keep magnitudes at or above 2^-12
        x = torch.where(x.abs() < 2.0 ** -12, torch.copysign(torch.full_like(x, 2.0 ** -12), x), x)
    return x.to(dtype)


def _build(lens, H, dtype, dist, seed, mx, extra_pages=3):
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
    k_rot = oracle.rotate_k(host_f32(k))  # float32 nearest to H k / 16
    if mx:
        planes = oracle.MxPlanes(pool, H)
        oracle.mx_quantize_append(planes, k_rot, host_f32(v), sl)
        layer = nk.MxKVCacheLayer.allocate(pool, H)
        nk.mx_quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(sl).cuda(), hadamard=True)
        g = (1.0, 1.0)
    else:
        g = (synth.global_scale(float(np.abs(k_rot).max())), synth.global_scale(float(v.float().abs().max())))
        planes = oracle.Planes(pool, H)
        oracle.quantize_append(planes, k_rot, host_f32(v), sl, *g)
        layer = nk.KVCacheLayer.allocate(pool, H, *g)
        nk.quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(sl).cuda(), hadamard=True)
    torch.cuda.synchronize()
    return layer, planes, bt, g


def _planes_diff(layer, planes):
    bad = []
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        g, o = getattr(layer, name).cpu().numpy(), getattr(planes, name)
        if not np.array_equal(g, o):
            i = np.flatnonzero(g != o)
            bad.append((name, int(i.size), int(i[0]), int(g[i[0]]), int(o[i[0]])))
    return bad


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dist", ["sparse6", "chan50"])
def test_rotated_append_bit_exact(mx, dtype, dist):
    lens = [1, 15, 16, 17, 100, 257]
    _say(f"case: rotated append mx={mx} {dtype} {dist} lens {lens}")
    layer, planes, _, _ = _build(lens, 4, dtype, dist, seed=71, mx=mx)
    assert _planes_diff(layer, planes) == []


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("lens,H,G,q_dtype,dist", [
    ([256, 77], 2, 4, torch.bfloat16, "chan50"),
    ([1, 15, 16, 17, 33, 0, 300], 2, 8, torch.float32, "sparse6"),
    ([513, 40, 1000], 1, 16, torch.bfloat16, "chan50"),
    ([700, 5, 129], 4, 1, torch.float32, "chan50"),
])
def test_rotated_decode_matches_oracle(mx, lens, H, G, q_dtype, dist):
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: rotated decode mx={mx} lens {lens} H {H} G {G} q {q_dtype} {dist}")
    layer, planes, bt, g = _build(lens, H, torch.bfloat16, dist, seed=73, mx=mx)
    B, Hq = len(lens), H * G
    q = synth.queries(B, Hq, q_dtype, "cpu", 11, 1)
    msl = max(lens)
    sm = 1 / math.sqrt(128)
    args = (q.cuda().contiguous(), torch.from_numpy(np.ascontiguousarray(bt)).cuda(),
            torch.tensor(lens, dtype=torch.int32, device="cuda"), msl, sm)
    out = (nk.mx_paged_decode_attn if mx else nk.paged_decode_attn)(layer, *args, hadamard=True)
    torch.cuda.synchronize()
    q_rot = oracle.rotate_q(host_f32(q)).astype(np.float32)
    smf = float(np.float32(sm))
    lens_np = np.array(lens, np.int32)
    ref = (oracle.mx_decode_attention(planes, q_rot, bt, lens_np, smf) if mx
           else oracle.decode_attention(planes, g[0], g[1], q_rot, bt, lens_np, smf))
    got = out.cpu().numpy().reshape(B * Hq, 128)
    err = row_rel_err(got, ref)
    _say(f"  max row rel err {err.max():.2e}")
    assert err.max() <= ATTN_TOL
    for b, n in enumerate(lens):
        if n == 0:
            assert (got.reshape(B, Hq, 128)[b] == 0).all()


def test_rotated_and_plain_caches_agree():
    """Both caches approximate the same attention: with K stored rotated and Q
    rotated alike, the output stays close to the unrotated cache's output."""
    import nvfp4_quantized_paged_kv_amd as nk

    lens, H, G = [400, 130], 2, 8
    bt, pool = synth.page_tables(lens, sum((n + 15) // 16 for n in lens), seed=5)
    k = torch.cat([_kv(n, H, torch.bfloat16, "sparse6", 5, b, 0) for b, n in enumerate(lens)]).cuda()
    v = torch.cat([_kv(n, H, torch.bfloat16, "sparse6", 5, b, 1) for b, n in enumerate(lens)]).cuda()
    sl = torch.from_numpy(np.concatenate([synth.slots_for(bt[b], 0, n) for b, n in enumerate(lens)])).cuda()
    q = synth.queries(len(lens), H * G, torch.bfloat16, "cuda", 5, 1)
    args = (q, torch.from_numpy(bt).cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens),
            1 / math.sqrt(128))
    outs = []
    for rot in (False, True):
        L = nk.MxKVCacheLayer.allocate(pool, H)
        nk.mx_quantize_append(L, k, v, sl, hadamard=rot)
        outs.append(nk.mx_paged_decode_attn(L, *args, hadamard=rot).cpu().numpy())
    diff = row_rel_err(outs[1], outs[0]).max()
    _say(f"  rotated vs plain MXFP4 cache: max row rel diff {diff:.2e}")
    assert diff < 0.1
