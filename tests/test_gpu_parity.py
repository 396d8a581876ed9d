"""GPU parity: the HIP library (called through its C ABI) against the CPU
oracle on the same seeded inputs.  Codes and scale bytes must match bit for
bit; decode attention must agree to 1e-3 row-normalised max relative error."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import ATTN_TOL, build_cache, decode_both, host_f32, planes_equal, row_rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_paged_kv_amd as nk  # noqa: F401  (fails loudly if the library is missing)
    yield


# ------------------------------------------------------------ quantize-append


def test_append_tiny_fp32_bitexact():
    _say("case: append tiny fp32 H=1 T=256 g=1")
    c = build_cache([256], 1, torch.float32, "sparse6", 0.005, True, seed=1)
    assert planes_equal(c.layer, c.planes) == []


@pytest.mark.parametrize("H,dist,frac", [(8, "chan50", 0.0), (8, "sparse6", 0.002), (3, "sparse6", 0.05)])
def test_append_bf16_ragged_bitexact(H, dist, frac):
    _say(f"case: append bf16 ragged H={H} {dist}")
    c = build_cache([1, 15, 16, 17, 100, 333], H, torch.bfloat16, dist, frac, False, seed=2 + H)
    assert planes_equal(c.layer, c.planes) == []


def test_append_strided_and_skipped_slots():
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: append strided input, negative and out-of-range slots")
    H, T = 4, 50
    big_k = synth.kv_values(T, H + 2, "sparse6", 0.01, 0, torch.bfloat16, "cpu", 77, 0)
    big_v = synth.kv_values(T, H + 2, "sparse6", 0.01, 1, torch.bfloat16, "cpu", 77, 0)
    k, v = big_k[:, :H, :], big_v[:, :H, :]
    k_dev, v_dev = big_k.cuda()[:, :H, :], big_v.cuda()[:, :H, :]  # token stride (H+2)*128 elements
    assert k_dev.stride(0) == (H + 2) * 128
    pool = 8
    rng = np.random.default_rng(3)
    slots = rng.permutation(pool * 16)[:T].astype(np.int32)
    slots[::7] = -1
    slots[3] = pool * 16 + 5  # beyond the pool: must be skipped
    planes = oracle.Planes(pool, H)
    ok = slots.copy()
    ok[ok >= pool * 16] = -1
    oracle.quantize_append(planes, host_f32(k), host_f32(v), ok, 0.01, 0.02)
    layer = nk.KVCacheLayer.allocate(pool, H, 0.01, 0.02)
    nk.quantize_append(layer, k_dev, v_dev, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert planes_equal(layer, planes) == []


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_append_v_slot_pairs(dt):
    """V bytes are shared by slot pairs (2k, 2k+1).  Slot runs that start at an
    even slot (neighbouring lanes pair), at an odd slot (a lane quantizes the
    token on its other side too), in descending order, split pairs written by
    far-apart tokens, lone slots and pairs with a skipped member, over planes
    holding random bytes; then a second call fills the partners of the first
    call's lone slots.  Every plane must match the oracle's bytes."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: append V slot pairs {dt}")
    H, pool = 3, 16
    even_run = list(range(16 * 2, 16 * 2 + 20))           # 20 slots from an even slot
    odd_run = list(range(16 * 4 + 3, 16 * 4 + 3 + 21))     # 21 slots from an odd slot
    down_run = list(range(16 * 7 + 9, 16 * 7 - 1, -1))     # 10 slots descending from an odd slot
    lone = [16 * 9 + 4, 16 * 9 + 7, 16 * 10 + 0, 16 * 10 + 13]
    split = [16 * 11 + 6]
    skipped_pair = [16 * 12 + 2, -1]
    slots1 = even_run + odd_run + split + down_run + lone + skipped_pair + [16 * 11 + 7] + [16 * 13 + 1]
    slots2 = [x ^ 1 for x in lone] + [16 * 12 + 3, 16 * 13 + 0, 16 * 14 + 5, 16 * 14 + 6]
    rng = np.random.default_rng(21)
    init = {n: rng.integers(0, 256, (pool * H * (1024 if "codes" in n else 128),), dtype=np.uint8)
            for n in ("k_codes", "k_scales", "v_codes", "v_scales")}
    planes = oracle.Planes(pool, H)
    layer = nk.KVCacheLayer.allocate(pool, H, 0.01, 0.02)
    for n, a in init.items():
        getattr(planes, n)[:] = a
        getattr(layer, n).copy_(torch.from_numpy(a).reshape(getattr(layer, n).shape))
    for call, slots in enumerate((slots1, slots2)):
        T = len(slots)
        k = synth.kv_values(T, H, "sparse6", 0.01, 0, dt, "cpu", 91 + call, 0)
        v = synth.kv_values(T, H, "sparse6", 0.01, 1, dt, "cpu", 91 + call, 0)
        sl = np.array(slots, np.int32)
        oracle.quantize_append(planes, host_f32(k), host_f32(v), sl, 0.01, 0.02)
        nk.quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(sl).cuda())
        torch.cuda.synchronize()
        assert planes_equal(layer, planes) == [], f"call {call}"


def _tie_rows():
    """Rows whose values sit exactly on E2M1 midpoints / whose amax sits on E4M3 midpoints."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    r = np.zeros(128, np.float32)
    for b in range(8):
        r[16 * b:16 * b + 16] = ([6.0] + mids + [-m for m in mids] + [-0.0])[:16]
    rows.append((r, 1.0))
    r = np.zeros(128, np.float32)
    for b in range(8):
        r[16 * b:16 * b + 16] = ([4.5] + [m * 0.75 for m in mids] + [-m * 0.75 for m in mids] + [0.0])[:16]
    rows.append((r, 0.5))
    e4 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    r = np.zeros(128, np.float32)
    for b, k in enumerate([0, 1, 7, 8, 30, 63, 100, 124]):
        amax = np.float32((e4[k] + e4[k + 1]) / 2 * 3)  # g = 0.5 -> amax/(6g) = midpoint exactly
        r[16 * b] = amax
        r[16 * b + 1:16 * b + 16] = np.linspace(-amax, amax, 15)
    rows.append((r, 0.5))
    r = np.zeros(128, np.float32)
    r[16:32] = 1e-30
    r[32:48] = -1e-30
    r[48:64] = 3e38
    r[64:80] = np.float32(1.5e-45)  # float32 subnormals
    rows.append((r, 1.0))
    # a 12-bit global scale that is not a power of two (1/(6g) is inexact):
    # E4M3 ties of amax/(6g), then E2M1 ties of x/(bs*g) at known scale bytes
    # (every product below has at most 19 significant bits: exact in float32)
    g = 1.234375
    r = np.zeros(128, np.float32)
    for b, k in enumerate([0, 2, 9, 33, 64, 90, 111, 125]):
        amax = np.float32((e4[k] + e4[k + 1]) / 2 * 6 * g)
        r[16 * b] = amax
        r[16 * b + 1:16 * b + 16] = np.linspace(-amax, amax, 15)
    rows.append((r, g))
    r = np.zeros(128, np.float32)
    for b, k in enumerate([8, 16, 40, 56, 72, 88, 104, 118]):
        bs0 = e4[k]  # amax = 6 * bs0 * g gives scale byte k exactly
        r[16 * b:16 * b + 16] = np.array([6 * bs0 * g] + [m * bs0 * g for m in mids] + [-m * bs0 * g for m in mids]
                                         + [0.0], np.float64)[:16].astype(np.float32)
    rows.append((r, g))
    return rows


def test_append_exact_ties_fp32():
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: append exact ties")
    for r, g in _tie_rows():
        k = np.stack([r, -r])[:, None, :]
        planes = oracle.Planes(1, 1)
        slots = np.array([0, 5], np.int32)
        oracle.quantize_append(planes, k, k, slots, g, g)
        layer = nk.KVCacheLayer.allocate(1, 1, g, g)
        kt = torch.from_numpy(k).cuda()
        nk.quantize_append(layer, kt, kt, torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        assert planes_equal(layer, planes) == [], g


def test_append_random_scales_fuzz():
    """Many global scales and magnitudes: every code and scale byte bit-exact."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: append fuzz over scales")
    rng = np.random.default_rng(11)
    for it in range(12):
        g = float(np.float32(np.exp(rng.uniform(-60, 60))))
        T, H = 64, 2
        x = (rng.standard_cauchy((T, H, 128)) * g * np.exp(rng.uniform(-8, 8, (T, H, 1)))).astype(np.float32)
        x = np.clip(x, -3e38, 3e38).astype(np.float32)
        slots = np.arange(T, dtype=np.int32)
        planes = oracle.Planes(4, H)
        oracle.quantize_append(planes, x, -x, slots, g, g)
        layer = nk.KVCacheLayer.allocate(4, H, g, g)
        xt = torch.from_numpy(x).cuda()
        nk.quantize_append(layer, xt, -xt, torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        assert planes_equal(layer, planes) == [], (it, g)


# ---------------------------------------------------------- decode attention


def test_decode_tiny_workload():
    """1 layer, batch 1, 4 q heads / 1 kv head, 256 tokens, fp32, g = 1."""
    _say("case: decode tiny")
    c = build_cache([256], 1, torch.float32, "sparse6", 0.005, True, seed=1)
    assert planes_equal(c.layer, c.planes) == []
    got, ref = decode_both(c, 4, torch.float32, seed=1)
    err = row_rel_err(got, ref)
    assert err.max() <= ATTN_TOL, err


@pytest.mark.parametrize("lens,H,G,qdt", [
    ([1], 1, 1, torch.bfloat16),
    ([15, 16, 17], 2, 4, torch.bfloat16),
    ([0, 33, 64, 65], 2, 8, torch.bfloat16),
    ([1000, 7, 513], 8, 8, torch.bfloat16),
    ([300, 2049], 8, 12, torch.bfloat16),
    ([200], 2, 16, torch.float32),
    ([4097], 1, 3, torch.float32),
])
def test_decode_matches_oracle(lens, H, G, qdt):
    _say(f"case: decode lens={lens} H={H} G={G} q={qdt}")
    c = build_cache(lens, H, torch.bfloat16, "chan50" if H == 8 else "sparse6", 0.003, False, seed=sum(lens) + G)
    got, ref = decode_both(c, H * G, qdt, seed=G)
    err = row_rel_err(got, ref)
    assert err.max() <= ATTN_TOL, (err.max(), np.argmax(err))


@pytest.mark.parametrize("q_scale", [30.0, 300.0])
def test_decode_peaked_softmax(q_scale):
    """Large queries: a peaked softmax (exercises the running-max rescale)."""
    _say(f"case: decode peaked q_scale={q_scale}")
    c = build_cache([777, 129], 2, torch.bfloat16, "sparse6", 0.01, False, seed=5)
    got, ref = decode_both(c, 2 * 8, torch.bfloat16, seed=9, q_scale=q_scale)
    err = row_rel_err(got, ref)
    assert err.max() <= ATTN_TOL, err.max()


def test_decode_max_batch():
    """The largest batch one launch takes (4096 sequences: every slot of the
    prologue's prefix scan), ragged lengths 0..40 including empty sequences."""
    _say("case: decode max batch 4096")
    rng = np.random.default_rng(97)
    lens = [int(x) for x in rng.integers(0, 41, 4096)]
    lens[0], lens[-1], lens[2048] = 0, 40, 1
    c = build_cache(lens, 1, torch.bfloat16, "sparse6", 0.005, False, seed=97)
    got, ref = decode_both(c, 2, torch.bfloat16, seed=13)
    err = row_rel_err(got, ref)
    _say(f"  max row rel err {err.max():.2e}")
    assert err.max() <= ATTN_TOL, (err.max(), int(np.argmax(err)))
    assert (got.reshape(4096, 2, 128)[np.array(lens) == 0] == 0).all()


def test_decode_huge_logits_stay_finite():
    """Queries scaled by 1e13 (logits far above 2^32): the softmax weights come
    from the rounded logit, so none overflows; the output stays finite and
    matches the oracle."""
    _say("case: decode huge logits")
    c = build_cache([300, 47, 129], 2, torch.bfloat16, "sparse6", 0.005, False, seed=83)
    got, ref = decode_both(c, 2 * 8, torch.bfloat16, seed=11, q_scale=1e13)
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    _say(f"  finite; max row rel err vs oracle {err.max():.2e}")
    assert err.max() <= ATTN_TOL, err.max()


def _cancelling_kv(lens, H, seed):
    """Per sequence: K = -1 and random V, except tokens 0 and 1: K = 1 (token
    1: 0.75 in dim 127), V = +1 and -1.  With g = 1 every K block has the scale
    0.171875, so K dequantizes to +-1.03125 and dim 127 of token 1 to 0.6875."""
    gen = torch.Generator().manual_seed(seed)
    kv = []
    for n in lens:
        k = -torch.ones((n, H, 128))
        v = torch.randn((n, H, 128), generator=gen)
        k[0] = 1.0
        k[1] = 1.0
        k[1, :, 127] = 0.75
        v[0] = 1.0
        v[1] = -1.0
        kv.append((k, v))
    return kv


def test_decode_cancelling_rows():
    """Rows whose output nearly cancels: with Q = 1.75 (0.25 in dim 127) the
    logits of tokens 0 and 1 are about 20.4 and 0.0076 apart, every other token
    sits about 40.8 lower, and V is +1 and -1 there, so each output is about
    0.4% of a V value.  P in f16 alone (2^-12 relative) could leave up to 3% of
    the row's largest value; the f16 hi + lo pair keeps it within 1e-3.  All
    products and sums of the logits are exact in the MFMA."""
    _say("case: decode cancelling rows")
    lens, H, Hq = [100, 37, 300], 2, 16
    c = build_cache(lens, H, torch.bfloat16, None, 0.0, True, seed=89, kv=_cancelling_kv(lens, H, 89))
    q = torch.full((len(lens), Hq, 128), 1.75)
    q[:, :, 127] = 0.25
    got, ref = decode_both(c, Hq, torch.bfloat16, seed=0, q=q)
    assert np.abs(ref).max(axis=1).max() < 0.01  # every row cancels to below 1% of a V value
    err = row_rel_err(got, ref)
    _say(f"  max row rel err vs oracle {err.max():.2e}")
    assert err.max() <= ATTN_TOL, err.max()


def test_decode_split_count_invariance():
    """A larger max_seq_len changes the split geometry; both results stay within the parity bound.

    The softmax weights are taken relative to a running maximum that depends
    on how tokens are grouped into splits, and enter the PV product as an f16
    hi + lo pair, so two split geometries differ at the level of that
    rounding, not bit for bit."""
    _say("case: decode split invariance")
    c = build_cache([1500, 900], 2, torch.bfloat16, "sparse6", 0.005, False, seed=21)
    a, ref = decode_both(c, 16, torch.bfloat16, seed=3)
    b, _ = decode_both(c, 16, torch.bfloat16, seed=3, max_seq_len=64 * 1024)
    assert row_rel_err(a, ref).max() <= ATTN_TOL
    assert row_rel_err(b, ref).max() <= ATTN_TOL
    assert row_rel_err(a, b).max() <= ATTN_TOL


def test_decode_workspace_reuse_and_counters():
    """Sequences shared by many workgroups: repeated calls on one workspace give the
    same result and leave every arrival counter at zero."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: decode workspace reuse (shared sequences)")
    c = build_cache([20000, 3, 16000], 2, torch.bfloat16, "sparse6", 0.003, False, seed=41)
    B, Hq = 3, 2 * 8
    q = synth.queries(B, Hq, torch.bfloat16, "cpu", 41, 1).cuda()
    bt = torch.from_numpy(c.bt).cuda()
    sl = torch.tensor(c.lens, dtype=torch.int32, device="cuda")
    ws = nk.decode_workspace(B, Hq, 2, 20000)
    outs = []
    for _ in range(3):
        outs.append(nk.paged_decode_attn(c.layer, q, bt, sl, 20000, 1 / math.sqrt(128), workspace=ws).clone())
    torch.cuda.synchronize()
    n_units = B * 2
    assert not ws[: 4 * n_units].any(), "arrival counters not reset"
    ref = oracle.decode_attention(c.planes, c.g_k, c.g_v, host_f32(q), c.bt, np.array(c.lens, np.int32),
                                  float(np.float32(1 / math.sqrt(128))))
    for o in outs:
        assert row_rel_err(o.cpu().numpy().reshape(-1, 128), ref).max() <= ATTN_TOL
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("seed", [7, 8])
def test_decode_ragged_many_units(seed):
    """A ragged batch whose work shares start and end everywhere: empty and
    one-token sequences between long ones, lengths on and off page boundaries,
    units much shorter than a share (many per workgroup) and units split over
    several workgroups; the output is checked row by row against the oracle."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 33, 250, 511, 1024, 3000, 9000], size=40)]
    lens[0], lens[-1] = 0, 1
    H, G = 4, 6
    _say(f"case: decode ragged many units seed={seed} lens={lens}")
    c = build_cache(lens, H, torch.bfloat16, "sparse6", 0.003, False, seed=seed)
    got, ref = decode_both(c, H * G, torch.bfloat16, seed=seed)
    err = row_rel_err(got, ref)
    assert err.max() <= ATTN_TOL, (err.max(), np.argmax(err))
    # empty sequences give zeros
    for b, n in enumerate(lens):
        if n == 0:
            assert not got.reshape(len(lens), H * G, 128)[b].any()


# ------------------------------------------------------- FP8 workspace dequant


@pytest.mark.parametrize("g_one", [True, False])
def test_dequant_ws_bitexact(g_one):
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: fp8 workspace g_one={g_one}")
    lens = [100, 37, 0, 256]
    H = 4
    c = build_cache(lens, H, torch.bfloat16, "sparse6", 0.01, g_one, seed=31)
    prefix = np.array([100, 20, 0, 256], np.int32)
    offs = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32)
    total = int(offs[-1])
    ks = 6 * c.g_k if not g_one else 6.0 / 448
    vs = 6 * c.g_v if not g_one else 6.0 / 448
    ref_k = oracle.fp8_workspace(c.planes, False, c.g_k, c.bt, prefix, offs, ks, total)
    ref_v = oracle.fp8_workspace(c.planes, True, c.g_v, c.bt, prefix, offs, vs, total)
    ws_k = torch.zeros((total + 5, H, 128), dtype=torch.uint8, device="cuda")
    ws_v = torch.zeros_like(ws_k)
    nk.dequant_to_fp8_workspace(c.layer, torch.from_numpy(c.bt).cuda(), torch.from_numpy(prefix).cuda(),
                                torch.from_numpy(offs).cuda(), int(prefix.max()), ks, vs, ws_k, ws_v)
    torch.cuda.synchronize()
    assert np.array_equal(ws_k[:total].cpu().numpy(), ref_k)
    assert np.array_equal(ws_v[:total].cpu().numpy(), ref_v)
    assert not ws_k[total:].any() and not ws_v[total:].any()


# ------------------------------------------------------- multi-token decode
def _multi_both(c, T, Hq, qdt, seed, max_seq_len=None):
    """Decode of T new tokens per sequence against the oracle: query token i of
    sequence b is a plain decode over its first lens[b] - (T-1-i) tokens."""
    import nvfp4_quantized_paged_kv_amd as nk

    B = len(c.lens)
    q = synth.queries(B * T, Hq, qdt, "cpu", seed, 2).reshape(B, T, Hq, 128)
    msl = max(max(c.lens), 1) if max_seq_len is None else max_seq_len
    bt = c.bt
    need = (msl + 15) // 16
    if bt.shape[1] < need:
        bt = np.concatenate([bt, np.zeros((B, need - bt.shape[1]), np.int32)], 1)
    out = nk.paged_decode_attn_multi(c.layer, q.cuda().contiguous(), torch.from_numpy(np.ascontiguousarray(bt)).cuda(),
                                     torch.tensor(c.lens, dtype=torch.int32, device="cuda"), msl, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    vlens = np.array([max(c.lens[b] - (T - 1 - i), 0) for b in range(B) for i in range(T)], np.int32)
    vbt = np.repeat(c.bt, T, axis=0)
    ref = oracle.decode_attention(c.planes, c.g_k, c.g_v, host_f32(q).reshape(B * T, Hq, 128), vbt, vlens,
                                  float(np.float32(1 / math.sqrt(128))))
    return out.cpu().numpy().reshape(B * T * Hq, 128), ref


@pytest.mark.parametrize("lens,H,G,T,qdt", [
    ([40, 17, 300], 2, 8, 2, torch.bfloat16),      # 16 query rows: the full MFMA tile
    ([1, 2, 3, 64, 65], 2, 4, 4, torch.bfloat16),   # tokens without keys, page boundaries
    ([100], 1, 1, 16, torch.float32),               # 16 tokens of one head
    ([257, 31], 3, 3, 5, torch.bfloat16),           # odd group: 15 rows
    ([9000, 20, 6000], 2, 8, 2, torch.bfloat16),    # units shared by several workgroups (partials)
])
def test_decode_multi_matches_oracle(lens, H, G, T, qdt):
    _say(f"case: multi-token decode lens={lens} H={H} G={G} T={T} q={qdt}")
    c = build_cache(lens, H, torch.bfloat16, "sparse6", 0.003, False, seed=sum(lens) + 17 * T)
    got, ref = _multi_both(c, T, H * G, qdt, seed=T)
    err = row_rel_err(got, ref)
    assert err.max() <= ATTN_TOL, (err.max(), int(np.argmax(err)))


def test_decode_multi_one_token_is_plain_decode():
    """T = 1 through the multi-token entry point gives the plain decode's result bit for bit."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: multi-token decode T=1 vs plain decode")
    c = build_cache([700, 33, 1500], 2, torch.bfloat16, "sparse6", 0.003, False, seed=91)
    q = synth.queries(3, 16, torch.bfloat16, "cpu", 91, 1).cuda()
    bt = torch.from_numpy(c.bt).cuda()
    sl = torch.tensor(c.lens, dtype=torch.int32, device="cuda")
    a = nk.paged_decode_attn(c.layer, q, bt, sl, 1500, 0.088)
    b = nk.paged_decode_attn_multi(c.layer, q.reshape(3, 1, 16, 128).contiguous(), bt, sl, 1500, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(a, b.reshape(3, 16, 128))


# ------------------------------------------------- decode step with its append
@pytest.mark.parametrize("lens,H,G,T,qdt", [
    ([33, 16, 17, 1000], 2, 8, 1, torch.bfloat16),   # the new token opens a page / ends one / mid-page
    ([17, 40, 2], 2, 8, 2, torch.bfloat16),          # two new tokens straddling pages 0 and 1
    ([1000, 50, 900], 2, 4, 4, torch.float32),       # one launch, units split over several workgroups, float32
    ([1, 3, 5], 1, 2, 4, torch.bfloat16),            # sequences shorter than the new tokens
])
def test_decode_step_equals_append_then_decode(lens, H, G, T, qdt):
    _step_case(lens, H, G, T, qdt, max(lens))


@pytest.mark.parametrize("lens,H,G,T,msl", [([33, 16, 17, 1000], 2, 8, 1, 270000), ([17, 40, 2], 2, 8, 2, 1025),
                                             ([1, 3, 5], 1, 2, 4, 4096), ([12000, 50, 9000], 2, 4, 4, 12000)])
def test_decode_step_two_launch_schedule(lens, H, G, T, msl):
    """max_seq_len above 1024 tokens: the step appends with the append kernel, then decodes."""
    _step_case(lens, H, G, T, torch.bfloat16 if msl != 12000 else torch.float32, msl)


def _step_case(lens, H, G, T, qdt, msl):
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: decode step lens={lens} H={H} G={G} T={T} q={qdt} max_seq_len={msl}")
    B, Hq = len(lens), H * G
    c = build_cache(lens, H, torch.bfloat16, "sparse6", 0.003, False, seed=sum(lens) + 5 * T)
    kn = synth.kv_values(B * T, H, "sparse6", 0.003, 0, qdt, "cpu", 77, T).reshape(B, T, H, 128)
    vn = synth.kv_values(B * T, H, "sparse6", 0.003, 1, qdt, "cpu", 77, T).reshape(B, T, H, 128)
    q = synth.queries(B * T, Hq, qdt, "cpu", 78, T).reshape(B, T, Hq, 128)
    bt_h = c.bt
    if bt_h.shape[1] * 16 < msl:  # room for max_seq_len (entries past the sequences are never read)
        bt_h = np.concatenate([bt_h, np.zeros((B, (msl + 15) // 16 - bt_h.shape[1]), np.int32)], 1)
    bt = torch.from_numpy(np.ascontiguousarray(bt_h)).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    # the new tokens' slots (positions len - T + i >= 0)
    pos = [(b, i, lens[b] - T + i) for b in range(B) for i in range(T)]
    slots = np.array([c.bt[b, p // 16] * 16 + p % 16 if p >= 0 else -1 for (b, i, p) in pos], np.int32)
    # reference path on a copy of the cache: append, then multi-token decode
    ref_layer = nk.KVCacheLayer(*(t.clone() for t in (c.layer.k_codes, c.layer.k_scales, c.layer.v_codes,
                                                        c.layer.v_scales)), c.layer.num_pages, H, c.g_k, c.g_v)
    nk.quantize_append(ref_layer, kn.reshape(B * T, H, 128).cuda(), vn.reshape(B * T, H, 128).cuda(),
                       torch.from_numpy(slots).cuda())
    ref_out = nk.paged_decode_attn_multi(ref_layer, q.cuda(), bt, sl, msl, 1 / math.sqrt(128))
    out = nk.paged_decode_step(c.layer, kn.cuda(), vn.cuda(), q.cuda(), bt, sl, msl, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(c.layer, name), getattr(ref_layer, name)), name
    assert torch.equal(out, ref_out)
    # and against the oracle: the appended bytes, then attention of every (sequence, token) row
    oracle.quantize_append(c.planes, host_f32(kn).reshape(B * T, H, 128), host_f32(vn).reshape(B * T, H, 128), slots,
                           c.g_k, c.g_v)
    assert planes_equal(c.layer, c.planes) == []
    vlens = np.array([max(lens[b] - (T - 1 - i), 0) for b in range(B) for i in range(T)], np.int32)
    ref = oracle.decode_attention(c.planes, c.g_k, c.g_v, host_f32(q).reshape(B * T, Hq, 128),
                                  np.repeat(c.bt, T, axis=0), vlens, float(np.float32(1 / math.sqrt(128))))
    err = row_rel_err(out.cpu().numpy().reshape(-1, 128), ref)
    assert err.max() <= ATTN_TOL, err.max()
