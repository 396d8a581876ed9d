"""GPU parity of the extend path: FP8 rows of new tokens (bit-exact against the
oracle) and causal extend / prefill attention over FP8 workspace rows (within
the 1e-3 row-normalised bound of the decode attention), through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import ATTN_TOL, build_cache, host_f32, row_rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_paged_kv_amd as nk  # noqa: F401  (fails loudly if the library is missing)
    yield


def _kv_values(rng, T, H, chan50=True):
    """K/V-like float32 values: N(0, 0.02), K with 2 channels x50 (the 70B-class recipe)."""
    k = rng.normal(0, 0.02, (T, H, 128)).astype(np.float32)
    v = rng.normal(0, 0.02, (T, H, 128)).astype(np.float32)
    if chan50:
        k[:, :, [5, 77]] *= 50
    return k, v


# ------------------------------------------------------------------- FP8 rows
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fp8_rows_bitexact(dtype):
    import nvfp4_quantized_paged_kv_amd as nk

    _say(f"case: fp8 rows dtype={dtype}")
    rng = np.random.default_rng(51)
    T, H, cap = 333, 4, 400
    k, v = _kv_values(rng, T, H)
    # exact E4M3 midpoints (times the scale) in a few rows: ties go to the even byte
    ks, vs = float(np.abs(k).max() / 448), float(np.abs(v).max() / 448)
    e4 = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (e4[:-1] + e4[1:]) / 2
    k[:4].reshape(-1)[: 4 * H * 128] = np.resize(mids * 1.0, 4 * H * 128).astype(np.float32)
    if dtype == torch.float32:
        ks = 1.0  # the midpoints above are exact quotients only for a unit scale
    kt = torch.from_numpy(k).to(dtype)
    vt = torch.from_numpy(v).to(dtype)
    if dtype == torch.float32:  # token-strided input: rows of a wider buffer
        def strided(x):
            wide = torch.zeros((T, H * 128 + 64), dtype=dtype)
            wide[:, : H * 128] = x.reshape(T, -1)
            return wide.cuda()[:, : H * 128].reshape(T, H, 128)
        kd, vd = strided(kt), strided(vt)
        assert kd.stride(0) == H * 128 + 64
    else:
        kd, vd = kt.cuda(), vt.cuda()
    rows = rng.permutation(cap)[:T].astype(np.int32)
    rows[::17] = -1                   # skipped
    rows[5] = cap + 3                 # past the capacity: skipped
    ws_k = torch.full((cap, H, 128), 0x5A, dtype=torch.uint8, device="cuda")
    ws_v = torch.full_like(ws_k, 0x5A)
    nk.fp8_rows_to_workspace(kd, vd, torch.from_numpy(rows).cuda(), ks, vs, ws_k, ws_v)
    torch.cuda.synchronize()
    ref_k = np.full((cap, H, 128), 0x5A, np.uint8)
    ref_v = np.full_like(ref_k, 0x5A)
    oracle.fp8_quantize_rows(host_f32(kt), np.where(rows < cap, rows, -1), ks, ref_k)
    oracle.fp8_quantize_rows(host_f32(vt), np.where(rows < cap, rows, -1), vs, ref_v)
    assert np.array_equal(ws_k.cpu().numpy(), ref_k)
    assert np.array_equal(ws_v.cpu().numpy(), ref_v)


# ----------------------------------------------------------- extend attention
def _case(rng, prefixes, chunks, H, gap=5):
    """Workspace rows [prefix | chunk] per sequence (gaps between), FP8 bytes from the oracle."""
    offs, at = [], 0
    for p, c in zip(prefixes, chunks):
        offs.append(at)
        at += p + c + gap
    cap = at
    k, v = _kv_values(rng, cap, H)
    ks, vs = float(np.abs(k).max() / 448), float(np.abs(v).max() / 448)
    ws_k = np.zeros((cap, H, 128), np.uint8)
    ws_v = np.zeros_like(ws_k)
    oracle.fp8_quantize_rows(k, np.arange(cap), ks, ws_k)
    oracle.fp8_quantize_rows(v, np.arange(cap), vs, ws_v)
    qo = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return ws_k, ws_v, ks, vs, np.array(offs, np.int32), qo


def _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, qdt, seed, q_scale=1.0, sm=0.088, rows=None,
                 max_chunk=None, extra_q_rows=0, q=None, split_max_prefix=None, oracle_ref=True):
    """The extend through the C ABI (the split entry point when split_max_prefix
    is given, its workspace pre-filled with NaN bytes) and the oracle's rows."""
    import nvfp4_quantized_paged_kv_amd as nk

    Tq = int(qo[-1]) + extra_q_rows
    if q is None:
        q = synth.queries(Tq, Hq, qdt, "cpu", seed, 7)
    if q_scale != 1.0:
        q = (q.float() * q_scale).to(qdt)
    pl = np.asarray(prefixes, np.int32)
    mc = int(np.diff(qo).max()) if max_chunk is None else max_chunk
    out = torch.full((Tq, Hq, 128), 12345.0, dtype=torch.float32, device="cuda")
    args = (q.cuda(), torch.from_numpy(qo).cuda(), torch.from_numpy(offs).cuda(), torch.from_numpy(pl).cuda(), mc)
    wsk, wsv = torch.from_numpy(ws_k).cuda(), torch.from_numpy(ws_v).cuda()
    if split_max_prefix is None:
        nk.fp8_extend_attn(*args, wsk, wsv, ks, vs, sm, out=out)
    else:
        need = nk.fp8_extend_attn_split_workspace_bytes(qdt, Tq, Hq, ws_k.shape[1], len(prefixes), mc,
                                                        split_max_prefix)
        _say(f"  split workspace {need} bytes")
        assert need > 0, "the split extend chose no split for this case"
        part = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        nk.fp8_extend_attn_split(*args, split_max_prefix, wsk, wsv, ks, vs, sm, out=out, workspace=part)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(Tq * Hq, 128)
    qf = host_f32(q)[: int(qo[-1])]
    if rows is None:
        rows = np.arange(int(qo[-1]) * Hq, dtype=np.int64)
    ref = oracle.extend_attention(ws_k, ws_v, ks, vs, qf, qo, offs, pl, sm, rows=rows) if oracle_ref else None
    return got, rows, ref


def test_fp8_rows_ties_non_power_of_two_scale():
    """Quotients exactly on E4M3 midpoints with a 12-bit workspace scale that is
    not a power of two (1/scale is inexact): ties go to the even byte."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: fp8 rows ties, scale 1.234375")
    H, T, s = 2, 4, 1.234375
    e4 = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (e4[:-1] + e4[1:]) / 2  # at most 5 significant bits: mid * s is exact in float32
    x = np.resize(np.concatenate([mids, -mids]) * s, T * H * 128).astype(np.float32).reshape(T, H, 128)
    assert np.array_equal(x.astype(np.float64) / s, np.resize(np.concatenate([mids, -mids]), T * H * 128).reshape(T, H, 128))
    rows = np.arange(T, dtype=np.int32)
    ws_k = torch.zeros((T, H, 128), dtype=torch.uint8, device="cuda")
    ws_v = torch.zeros_like(ws_k)
    xt = torch.from_numpy(x).cuda()
    nk.fp8_rows_to_workspace(xt, xt, torch.from_numpy(rows).cuda(), s, s, ws_k, ws_v)
    torch.cuda.synchronize()
    ref = np.zeros((T, H, 128), np.uint8)
    oracle.fp8_quantize_rows(x, rows, s, ref)
    assert np.array_equal(ws_k.cpu().numpy(), ref) and np.array_equal(ws_v.cpu().numpy(), ref)


@pytest.mark.parametrize("prefixes,chunks,H,G,qdt", [
    ([0], [100], 2, 4, torch.bfloat16),                 # prefill: the chunk only
    ([0, 37, 300], [1, 50, 33], 2, 8, torch.bfloat16),  # ragged extends, single-token chunk
    ([200], [40], 1, 16, torch.float32),                # 512-thread workgroups, float32 Q
    ([70, 5], [17, 64], 3, 3, torch.bfloat16),          # odd group: a half-empty wave
    ([31, 32, 33], [15, 16, 17], 1, 1, torch.float32),  # tile and page boundaries, one head
])
def test_extend_matches_oracle(prefixes, chunks, H, G, qdt):
    _say(f"case: extend prefixes={prefixes} chunks={chunks} H={H} G={G} q={qdt}")
    rng = np.random.default_rng(sum(prefixes) + sum(chunks) + G)
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H)
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, H * G, qdt, seed=G)
    err = row_rel_err(got[rows], ref)
    assert err.max() <= ATTN_TOL, (err.max(), int(np.argmax(err)))


@pytest.mark.parametrize("q_scale", [30.0, 300.0])
def test_extend_peaked_softmax(q_scale):
    _say(f"case: extend peaked q_scale={q_scale}")
    rng = np.random.default_rng(61)
    prefixes, chunks = [150, 9], [40, 70]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, 16, torch.bfloat16, seed=3,
                                  q_scale=q_scale)
    err = row_rel_err(got[rows], ref)
    assert err.max() <= ATTN_TOL, err.max()


def test_extend_huge_logits_stay_finite():
    """Logits far above 2^32 (a huge softmax scale): the weights come from the
    rounded logit, so the largest one is exactly 2^0 and none overflows; the
    output is a convex combination of V rows and matches the oracle."""
    _say("case: extend huge logits")
    rng = np.random.default_rng(67)
    prefixes, chunks = [90, 0], [33, 20]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, 16, torch.bfloat16, seed=5, sm=1e12)
    assert np.isfinite(got[rows]).all()
    err = row_rel_err(got[rows], ref)
    _say(f"  finite; max row rel err vs oracle {err.max():.2e}")
    assert err.max() <= ATTN_TOL, err.max()


def test_extend_cancelling_rows():
    """Rows whose output nearly cancels: in each sequence two prefix keys take
    almost all the weight (logits 20 and 19.990; every other key sits 40 lower)
    and have opposite V rows (+1 and -1 in every dim), so every output value is
    about 0.5% of a V value.  Rounding P to f16 alone (2^-12 relative) would
    leave about 2.5% of the row's largest value; the bound is 1e-3.  All
    products and sums of the logits are exact (powers of two)."""
    _say("case: extend cancelling rows")
    H, Hq = 2, 16
    prefixes, chunks = [40, 7], [37, 20]
    offs = np.array([0, prefixes[0] + chunks[0] + 3], np.int32)
    cap = int(offs[-1]) + prefixes[1] + chunks[1]
    rng = np.random.default_rng(71)
    ws_k = np.full((cap, H, 128), 0xB8, np.uint8)  # K = -1 in every dim
    mag = rng.integers(0, 0x7F, (cap, H, 128)).astype(np.uint8)  # any finite E4M3 V (0x7F is NaN)
    ws_v = mag | (rng.integers(0, 2, (cap, H, 128)).astype(np.uint8) << 7)
    for o in offs:
        ws_k[o] = 0x38  # key a: K = 1
        ws_k[o + 1] = 0x38
        ws_k[o + 1, :, 127] = 0x37  # key b: K = 1 except 0.9375 in one dim
        ws_v[o] = 0x38  # V = +1
        ws_v[o + 1] = 0xB8  # V = -1
    qo = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = torch.ones((int(qo[-1]), Hq, 128), dtype=torch.bfloat16)
    # logit of key a = 1.25 * 128 * 0.125 = 20
    got, rows, ref = _extend_both(ws_k, ws_v, 0.125, 1.0 / 64, offs, qo, prefixes, Hq, torch.bfloat16, seed=0,
                                  sm=1.25, q=q)
    assert np.abs(ref).max(axis=1).max() < 0.01 / 64  # every row cancels to below 1% of a V value
    err = row_rel_err(got[rows], ref)
    _say(f"  max row rel err vs oracle {err.max():.2e}")
    assert err.max() <= ATTN_TOL, err.max()


def test_extend_rows_outside_chunks_are_untouched():
    """Tokens past max_chunk_len and query rows after the last chunk are not written."""
    _say("case: extend untouched rows")
    rng = np.random.default_rng(62)
    prefixes, chunks = [20, 40], [30, 12]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, 8, torch.bfloat16, seed=4, max_chunk=16,
                                  extra_q_rows=5)
    Hq = 8
    got = got.reshape(-1, Hq, 128)
    ref = ref.reshape(-1, Hq, 128)
    computed = [t for i in range(2) for t in range(qo[i], qo[i] + min(16, chunks[i]))]
    assert row_rel_err(got[computed], ref[computed]).max() <= ATTN_TOL
    skipped = [t for t in range(got.shape[0]) if t not in computed]
    assert np.all(got[skipped] == 12345.0)


def test_extend_after_nvfp4_workspace_and_fp8_rows():
    """The whole extend flow: NVFP4 cache -> FP8 workspace prefix (dequant kernel),
    chunk K/V -> FP8 rows, then attention; bytes bit-exact, attention to 1e-3."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: extend full flow")
    H, G = 2, 8
    prefixes, chunks = [200, 45, 0], [33, 64, 20]
    c = build_cache(prefixes, H, torch.bfloat16, "chan50", 0.0, False, seed=71)
    ks, vs = 6 * c.g_k, 6 * c.g_v
    offs = np.concatenate([[0], np.cumsum(np.array(prefixes) + np.array(chunks))])[:-1].astype(np.int32)
    cap = int(sum(prefixes) + sum(chunks))
    ws_k = torch.zeros((cap, H, 128), dtype=torch.uint8, device="cuda")
    ws_v = torch.zeros_like(ws_k)
    pl = np.array(prefixes, np.int32)
    nk.dequant_to_fp8_workspace(c.layer, torch.from_numpy(c.bt).cuda(), torch.from_numpy(pl).cuda(),
                                torch.from_numpy(np.append(offs, cap).astype(np.int32)).cuda(), int(pl.max()), ks, vs,
                                ws_k, ws_v)
    rng = np.random.default_rng(72)
    T = int(sum(chunks))
    kn, vn = _kv_values(rng, T, H)
    knt, vnt = torch.from_numpy(kn).to(torch.bfloat16), torch.from_numpy(vn).to(torch.bfloat16)
    rows = np.concatenate([offs[i] + prefixes[i] + np.arange(chunks[i]) for i in range(3)]).astype(np.int32)
    nk.fp8_rows_to_workspace(knt.cuda(), vnt.cuda(), torch.from_numpy(rows).cuda(), ks, vs, ws_k, ws_v)
    torch.cuda.synchronize()
    wk = oracle.fp8_workspace(c.planes, False, c.g_k, c.bt, pl, np.append(offs, cap), ks, cap)
    wv = oracle.fp8_workspace(c.planes, True, c.g_v, c.bt, pl, np.append(offs, cap), vs, cap)
    oracle.fp8_quantize_rows(host_f32(knt), rows, ks, wk)
    oracle.fp8_quantize_rows(host_f32(vnt), rows, vs, wv)
    assert np.array_equal(ws_k.cpu().numpy(), wk)
    assert np.array_equal(ws_v.cpu().numpy(), wv)
    qo = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    got, r, ref = _extend_both(wk, wv, ks, vs, offs, qo, prefixes, H * G, torch.bfloat16, seed=5)
    assert row_rel_err(got[r], ref).max() <= ATTN_TOL


def test_extend_mixed_step_shape_sampled():
    """The mixed serving step's extend shape (64 q / 8 kv heads, 2048-token chunks over
    long prefixes), checked on a sample of output rows the oracle computes one by one."""
    _say("case: extend mixed-step shape, sampled rows")
    rng = np.random.default_rng(81)
    prefixes, chunks = [9000, 700], [2048, 2048]
    H, Hq = 8, 64
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H, gap=0)
    Tq = int(qo[-1])
    rows = np.unique(np.concatenate([
        rng.integers(0, Tq * Hq, 150),
        [0, Hq - 1, 2047 * Hq, 2048 * Hq, Tq * Hq - 1],  # first / last tokens of each chunk
    ])).astype(np.int64)
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, torch.bfloat16, seed=6, rows=rows)
    err = row_rel_err(got[rows], ref)
    assert err.max() <= ATTN_TOL, err.max()


# ------------------------------------------------- split extend (keys shared)
@pytest.mark.parametrize("prefixes,chunks,H,G,qdt,max_prefix", [
    ([5000, 3071], [1, 16], 2, 8, torch.bfloat16, None),          # verification-like: short chunks, long prefixes
    ([4000, 0, 2500], [7, 5, 33], 1, 16, torch.float32, None),    # 512-thread workgroups, float32 Q, 3-tile chunk
    ([2047, 2049, 3000], [4, 0, 9], 3, 3, torch.bfloat16, None),  # odd group, an empty chunk
    ([10, 3], [3, 2], 2, 4, torch.bfloat16, 1 << 20),             # over-stated prefix bound: most shares empty
])
def test_extend_split_matches_oracle_and_unsplit(prefixes, chunks, H, G, qdt, max_prefix):
    _say(f"case: split extend prefixes={prefixes} chunks={chunks} H={H} G={G} q={qdt} max_prefix={max_prefix}")
    rng = np.random.default_rng(sum(prefixes) + sum(chunks) + G + 1)
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H)
    mp = max(prefixes) if max_prefix is None else max_prefix
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, H * G, qdt, seed=G, split_max_prefix=mp)
    err = row_rel_err(got[rows], ref)
    assert err.max() <= ATTN_TOL, (err.max(), int(np.argmax(err)))
    whole, _, _ = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, H * G, qdt, seed=G, oracle_ref=False)
    d = row_rel_err(got[rows], whole[rows])
    _say(f"  max row rel err: vs oracle {err.max():.2e}, vs unsplit {d.max():.2e}")
    assert d.max() <= 2e-5, d.max()  # the same sums in another fp32 order


def test_extend_split_rows_outside_chunks_are_untouched():
    """With keys shared: tokens past max_chunk_len and query rows after the last chunk are not written."""
    _say("case: split extend untouched rows")
    rng = np.random.default_rng(63)
    prefixes, chunks = [5000, 300], [20, 12]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    Hq = 8
    got, rows, ref = _extend_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, torch.bfloat16, seed=4, max_chunk=16,
                                  extra_q_rows=5, split_max_prefix=5000)
    got = got.reshape(-1, Hq, 128)
    ref = ref.reshape(-1, Hq, 128)
    computed = [t for i in range(2) for t in range(qo[i], qo[i] + min(16, chunks[i]))]
    assert row_rel_err(got[computed], ref[computed]).max() <= ATTN_TOL
    skipped = [t for t in range(got.shape[0]) if t not in computed]
    assert np.all(got[skipped] == 12345.0)


def test_extend_split_workspace_reuse_smaller_call():
    """One workspace, two calls in a row, the second smaller: its results do not depend on the first's partials."""
    import nvfp4_quantized_paged_kv_amd as nk

    _say("case: split extend workspace reuse")
    rng = np.random.default_rng(64)
    H, Hq = 2, 16
    big = _case(rng, [6000, 4000], [9, 3], H)
    small = _case(rng, [3000], [2], H)
    bf = torch.bfloat16
    need = nk.fp8_extend_attn_split_workspace_bytes(bf, 12, Hq, H, 2, 9, 6000)
    assert need >= nk.fp8_extend_attn_split_workspace_bytes(bf, 2, Hq, H, 1, 2, 3000) > 0
    part = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for (ws_k, ws_v, ks, vs, offs, qo), prefixes in ((big, [6000, 4000]), (small, [3000])):
        Tq, mc = int(qo[-1]), int(np.diff(qo).max())
        q = synth.queries(Tq, Hq, torch.bfloat16, "cpu", 9, 7)
        out = nk.fp8_extend_attn_split(q.cuda(), torch.from_numpy(qo).cuda(), torch.from_numpy(offs).cuda(),
                                       torch.from_numpy(np.asarray(prefixes, np.int32)).cuda(), mc, max(prefixes),
                                       torch.from_numpy(ws_k).cuda(), torch.from_numpy(ws_v).cuda(), ks, vs, 0.088,
                                       workspace=part)
        torch.cuda.synchronize()
        ref = oracle.extend_attention(ws_k, ws_v, ks, vs, host_f32(q), qo, offs, np.asarray(prefixes, np.int32), 0.088,
                                      rows=np.arange(Tq * Hq, dtype=np.int64))
        outs.append(row_rel_err(out.cpu().numpy().reshape(-1, 128), ref).max())
    _say(f"  max row rel err per call {outs}")
    assert max(outs) <= ATTN_TOL, outs


# ------------------------------------------- extend attention in FP8 arithmetic
def _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, qdt, seed, q_scale=1.0, sm=0.088, rows=None,
                    max_chunk=None, max_prefix=None, extra_q_rows=0):
    """The FP8-arithmetic extend through the C ABI (a needed split workspace pre-filled
    with NaN bytes), the oracle's FP8 statement with its per-row bound, and the exact oracle."""
    import nvfp4_quantized_paged_kv_amd as nk

    Tq = int(qo[-1]) + extra_q_rows
    q = synth.queries(Tq, Hq, qdt, "cpu", seed, 7)
    if q_scale != 1.0:
        q = (q.float() * q_scale).to(qdt)
    pl = np.asarray(prefixes, np.int32)
    mc = int(np.diff(qo).max()) if max_chunk is None else max_chunk
    mp = int(pl.max()) if max_prefix is None else max_prefix
    out = torch.full((Tq, Hq, 128), 12345.0, dtype=torch.float32, device="cuda")
    need = nk.fp8_extend_attn_f8_workspace_bytes(qdt, Tq, Hq, ws_k.shape[1], len(prefixes), mc, mp)
    part = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    _say(f"  f8 split workspace {need} bytes")
    nk.fp8_extend_attn_f8(q.cuda(), torch.from_numpy(qo).cuda(), torch.from_numpy(offs).cuda(),
                          torch.from_numpy(pl).cuda(), mc, mp, torch.from_numpy(ws_k).cuda(),
                          torch.from_numpy(ws_v).cuda(), ks, vs, sm, out=out, workspace=part)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(Tq * Hq, 128)
    qf = host_f32(q)[: int(qo[-1])]
    if rows is None:
        rows = np.arange(int(qo[-1]) * Hq, dtype=np.int64)
    emul, tol = oracle.extend_attention_fp8(ws_k, ws_v, ks, vs, qf, qo, offs, pl, sm, rows=rows)
    exact = oracle.extend_attention(ws_k, ws_v, ks, vs, qf, qo, offs, pl, sm, rows=rows)
    return got, rows, emul, tol, exact, need


def _check_f8(got, rows, emul, tol, exact):
    d = np.abs(got[rows] - emul).max(axis=1)
    scale = np.abs(emul).max(axis=1)
    bad = np.nonzero(d > tol + 1e-6 * scale)[0]
    rel = d / np.maximum(scale, 1e-30)
    ex = row_rel_err(got[rows], exact)
    _say(f"  vs FP8 statement: max row err {rel.max():.2e} (median {np.median(rel):.2e}), bound median "
         f"{np.median(tol / np.maximum(scale, 1e-30)):.2e}; vs exact attention: max {ex.max():.2e} "
         f"(median {np.median(ex):.2e})")
    assert bad.size == 0, (bad[:5], d[bad[:5]], tol[bad[:5]])
    return ex


@pytest.mark.parametrize("prefixes,chunks,H,G,qdt", [
    ([0], [100], 2, 4, torch.bfloat16),                 # prefill: the chunk only
    ([0, 37, 300], [1, 50, 33], 2, 8, torch.bfloat16),  # ragged extends, single-token chunk
    ([200], [40], 1, 16, torch.float32),                # 512-thread workgroups, float32 Q
    ([70, 5], [17, 64], 3, 3, torch.bfloat16),          # odd group: a half-empty wave
    ([31, 32, 33], [15, 16, 17], 1, 1, torch.float32),  # tile and page boundaries, one head
    ([63, 64, 65, 127], [1, 64, 65, 2], 2, 8, torch.bfloat16),  # 64-key tile boundaries
])
def test_extend_f8_matches_fp8_statement(prefixes, chunks, H, G, qdt):
    _say(f"case: f8 extend prefixes={prefixes} chunks={chunks} H={H} G={G} q={qdt}")
    rng = np.random.default_rng(sum(prefixes) + sum(chunks) + G + 2)
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H)
    got, rows, emul, tol, exact, _ = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, H * G, qdt, seed=G)
    ex = _check_f8(got, rows, emul, tol, exact)
    assert ex.max() <= 0.1  # the E4M3 roundings of Q and of the weights (2^-4 each), well inside


@pytest.mark.parametrize("prefixes,chunks,H,G,qdt,max_prefix", [
    ([5000, 3071], [1, 16], 2, 8, torch.bfloat16, None),          # short chunks over long prefixes: keys split
    ([4000, 0, 2500], [7, 5, 33], 1, 16, torch.float32, None),    # 512-thread workgroups, float32 Q
    ([10, 3], [3, 2], 2, 4, torch.bfloat16, 1 << 20),             # over-stated prefix bound: most shares empty
])
def test_extend_f8_split_matches_fp8_statement(prefixes, chunks, H, G, qdt, max_prefix):
    _say(f"case: f8 split extend prefixes={prefixes} chunks={chunks} H={H} G={G} q={qdt} max_prefix={max_prefix}")
    rng = np.random.default_rng(sum(prefixes) + sum(chunks) + G + 3)
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H)
    got, rows, emul, tol, exact, need = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, H * G, qdt, seed=G,
                                                        max_prefix=max_prefix)
    assert need > 0, "no split chosen"
    _check_f8(got, rows, emul, tol, exact)


@pytest.mark.parametrize("q_scale", [30.0, 300.0])
def test_extend_f8_peaked_softmax(q_scale):
    _say(f"case: f8 extend peaked q_scale={q_scale}")
    rng = np.random.default_rng(161)
    prefixes, chunks = [150, 9], [40, 70]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    got, rows, emul, tol, exact, _ = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, 16, torch.bfloat16, 3,
                                                     q_scale=q_scale)
    _check_f8(got, rows, emul, tol, exact)


def test_extend_f8_huge_logits_stay_finite():
    _say("case: f8 extend huge logits")
    rng = np.random.default_rng(167)
    prefixes, chunks = [90, 0], [33, 20]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    got, rows, emul, tol, exact, _ = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, 16, torch.bfloat16, 5,
                                                     sm=1e12)
    assert np.isfinite(got[rows]).all()
    _check_f8(got, rows, emul, tol, exact)


def test_extend_f8_rows_outside_chunks_are_untouched():
    _say("case: f8 extend untouched rows")
    rng = np.random.default_rng(162)
    prefixes, chunks = [20, 40], [30, 12]
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, 2)
    Hq = 8
    got, rows, emul, tol, exact, _ = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, torch.bfloat16, 4,
                                                     max_chunk=16, extra_q_rows=5)
    got = got.reshape(-1, Hq, 128)
    computed = [t for i in range(2) for t in range(qo[i], qo[i] + min(16, chunks[i]))]
    crow = np.array([t * Hq + h for t in computed for h in range(Hq)], np.int64)
    _check_f8(got.reshape(-1, 128), crow, emul[crow], tol[crow], exact[crow])
    skipped = [t for t in range(got.shape[0]) if t not in computed]
    assert np.all(got[skipped] == 12345.0)


def test_extend_f8_mixed_step_shape_sampled():
    """The mixed serving step's extend shape (64 q / 8 kv heads, 2048-token chunks over
    long prefixes) in FP8 arithmetic, on sampled rows."""
    _say("case: f8 extend mixed-step shape, sampled rows")
    rng = np.random.default_rng(181)
    prefixes, chunks = [9000, 700], [2048, 2048]
    H, Hq = 8, 64
    ws_k, ws_v, ks, vs, offs, qo = _case(rng, prefixes, chunks, H, gap=0)
    Tq = int(qo[-1])
    rows = np.unique(np.concatenate([rng.integers(0, Tq * Hq, 150),
                                     [0, Hq - 1, 2047 * Hq, 2048 * Hq, Tq * Hq - 1]])).astype(np.int64)
    got, rows, emul, tol, exact, _ = _extend_f8_both(ws_k, ws_v, ks, vs, offs, qo, prefixes, Hq, torch.bfloat16, 6,
                                                     rows=rows)
    _check_f8(got, rows, emul, tol, exact)
