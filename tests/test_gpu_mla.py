"""GPU parity of the Sparse-MLA latent cache against the oracle: latent rows
quantize-appended bit for bit (bf16 and float32 inputs, strided rows,
skipped slots), and sparse decode attention to 1e-3 over top-k slot lists with
skipped, out-of-range and repeated entries, ragged list tails, several head
counts (1 to 4 waves, two head blocks), lists split over several workgroups
and merged, rows whose output nearly cancels, and empty lists."""
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


def _fill(n_slots, g, rows, slots, dtype=torch.bfloat16):
    """The same rows into a GPU layer and the oracle's planes; returns both."""
    import nvfp4_quantized_paged_kv_amd as nk
    layer = nk.MlaCacheLayer.allocate(n_slots, g, "cuda")
    nk.mla_quantize_append(layer, rows.to(dtype).cuda(), torch.as_tensor(slots, dtype=torch.int32).cuda())
    planes = oracle.MlaPlanes(n_slots)
    oracle.mla_quantize_append(planes, host_f32(rows.to(dtype)), np.asarray(slots), g)
    torch.cuda.synchronize()
    return layer, planes


def _planes_equal(layer, planes):
    return (np.array_equal(layer.codes.cpu().numpy(), planes.codes)
            and np.array_equal(layer.scales.cpu().numpy(), planes.scales))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mla_append_bitexact(dtype):
    import nvfp4_quantized_paged_kv_amd as nk
    _say(f"case: mla append {dtype}")
    n_slots, T = 700, 520
    rows = synth.mla_rows(T, 0.01, torch.float32, "cpu", 31)
    rows[3, :64] = 0.0
    rows[4, 10] = -0.0
    rows[5] *= 1e-6                      # tiny values: subnormal block scales
    rows[6, 512:] *= 300.0               # a loud rotary part
    g = synth.global_scale(float(rows.abs().max()))
    rng = np.random.default_rng(3)
    slots = rng.permutation(n_slots)[:T].astype(np.int32)
    slots[7] = -1                        # skipped
    slots[8] = n_slots                   # past the cache: skipped
    layer, planes = _fill(n_slots, g, rows, slots, dtype)
    assert _planes_equal(layer, planes)
    # strided rows (token stride 640 elements) write the same bytes
    wide = torch.zeros((T, 640), dtype=dtype)
    wide[:, :576] = rows.to(dtype)
    layer2 = nk.MlaCacheLayer.allocate(n_slots, g, "cuda")
    nk.mla_quantize_append(layer2, wide.cuda()[:, :576], torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert _planes_equal(layer2, planes)


def _decode_case(T, Hq, topk, n_slots, seed, q_scale=1.0, lens=None, idx=None, rows=None):
    import nvfp4_quantized_paged_kv_amd as nk
    _say(f"case: mla decode T={T} Hq={Hq} topk={topk} slots={n_slots} seed={seed}")
    if rows is None:
        rows = synth.mla_rows(n_slots, 0.005, torch.float32, "cpu", seed)
    g = synth.global_scale(float(rows.abs().max()))
    layer, planes = _fill(n_slots, g, rows, np.arange(n_slots, dtype=np.int32))
    assert _planes_equal(layer, planes)
    if idx is None:
        rng = np.random.default_rng(seed)
        idx = rng.integers(0, n_slots, (T, topk)).astype(np.int32)
    q = (synth.mla_queries(T, Hq, torch.float32, "cpu", seed) * q_scale).to(torch.bfloat16)
    sm = 1 / math.sqrt(192)
    out = nk.mla_sparse_decode(layer, q.cuda(), torch.from_numpy(np.ascontiguousarray(idx)).cuda(), sm)
    torch.cuda.synchronize()
    ref = oracle.mla_sparse_decode(planes, g, host_f32(q), idx, sm)
    got = out.cpu().numpy()
    err = row_rel_err(got.reshape(-1, 512), ref.reshape(-1, 512))
    _say(f"  max row rel err {err.max():.2e}")
    assert err.max() <= ATTN_TOL, err.max()
    return got, ref


@pytest.mark.parametrize("Hq", [16, 32, 48, 64, 128])
def test_mla_decode_head_counts(Hq):
    """1, 2, 3 and 4 waves per workgroup, and two head blocks (128 heads)."""
    _decode_case(T=3, Hq=Hq, topk=77, n_slots=400, seed=40 + Hq)


def test_mla_decode_skipped_and_repeated_entries():
    rng = np.random.default_rng(41)
    T, topk, n = 6, 100, 500
    idx = rng.integers(0, n, (T, topk)).astype(np.int32)
    idx[0, ::3] = -1                  # skipped
    idx[1, 5:40] = n + 7              # past the cache: skipped
    idx[2, :60] = idx[2, 0]           # one slot repeated
    idx[3, :] = -1                    # nothing valid: zeros
    idx[4, :99] = -5                  # a single valid entry, last in the list
    got, ref = _decode_case(T, 64, topk, n, 41, idx=idx)
    assert not got[3].any()


def test_mla_decode_split_lists_merge():
    """Few query tokens with long lists: each list is split over several
    workgroups and the shares are merged by a second launch."""
    import nvfp4_quantized_paged_kv_amd as nk
    assert nk.mla_sparse_decode_workspace_bytes(2, 64, 2048) > nk.mla_sparse_decode_workspace_bytes(512, 64, 2048)
    _decode_case(T=2, Hq=64, topk=2048, n_slots=6000, seed=42)
    _decode_case(T=1, Hq=128, topk=1000, n_slots=3000, seed=43)   # ragged last share


def test_mla_decode_peaked_and_needle():
    """A large query scale makes the softmax nearly one-hot."""
    _decode_case(T=4, Hq=32, topk=256, n_slots=1000, seed=44, q_scale=40.0)


def test_mla_decode_cancelling_rows():
    """Two entries carry almost all the weight with opposite latent values, so
    each output is a fraction of a value: P must enter with more than f16's
    11 bits.  Row 0's rotary value 2.0 sits in block 32, row 1's in block 33;
    the query weighs them 64 and 63.75, so the logits are 128 and 127.5
    (every value is exact in NVFP4 and bf16)."""
    import nvfp4_quantized_paged_kv_amd as nk
    n = 64
    rows = torch.zeros((n, 576))
    rows[:, 512:] = torch.randn((n, 64), generator=torch.Generator().manual_seed(45)) * 0.01
    rows[0, :512] = 1.0
    rows[1, :512] = -1.0
    rows[0, 512:544] = 0.0
    rows[1, 512:544] = 0.0
    rows[0, 512] = 2.0
    rows[1, 528] = 2.0
    q = torch.zeros((1, 16, 576))
    q[:, :, 512] = 64.0
    q[:, :, 528] = 63.75
    idx = np.arange(n, dtype=np.int32)[None]
    g = synth.global_scale(float(rows.abs().max()))
    layer, planes = _fill(n, g, rows, np.arange(n, dtype=np.int32))
    out = nk.mla_sparse_decode(layer, q.to(torch.bfloat16).cuda(), torch.from_numpy(idx).cuda(), 1.0)
    torch.cuda.synchronize()
    ref = oracle.mla_sparse_decode(planes, g, host_f32(q.to(torch.bfloat16)), idx, 1.0)
    err = row_rel_err(out.cpu().numpy().reshape(-1, 512), ref.reshape(-1, 512))
    _say(f"case: mla cancelling rows, max |out| {np.abs(ref).max():.3f}, max row rel err {err.max():.2e}")
    assert 0.1 < np.abs(ref).max() < 0.5 and err.max() <= ATTN_TOL


def test_mla_decode_empty_list_and_no_tokens():
    import nvfp4_quantized_paged_kv_amd as nk
    layer = nk.MlaCacheLayer.allocate(16, 0.01, "cuda")
    q = torch.ones((2, 16, 576), dtype=torch.bfloat16, device="cuda")
    out = nk.mla_sparse_decode(layer, q, torch.zeros((2, 0), dtype=torch.int32, device="cuda"), 0.1)
    torch.cuda.synchronize()
    assert not out.any()
    out0 = nk.mla_sparse_decode(layer, q[:0], torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 0.1)
    assert out0.shape == (0, 16, 512)


def test_mla_full_size_sampled():
    """The bench's sparse-MLA shape at full size (4,194,304 cached tokens in
    random 64-token pages, 128 query tokens, top-2048 lists): the rows the
    first and last query tokens list are checked byte for byte against the
    oracle's quantizer of the raw rows, and those tokens' outputs at 128 heads
    (one workgroup per 64 heads, unsplit) and at 16 heads (lists split over
    workgroups and merged) against the oracle's attention."""
    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic.workloads import MLA_SHAPE, build_mla_layer

    T, ctx, topk = MLA_SHAPE["T"], MLA_SHAPE["ctx"], MLA_SHAPE["topk"]
    samples = [0, T - 1]
    _say(f"case: mla full size T={T} ctx={ctx} topk={topk}, samples {samples}")
    pos = synth.mla_topk_positions(T, [ctx] * T, topk, "cuda", 62, 0)  # the lists build_mla_layer draws
    want = torch.unique(torch.cat([t * ctx + pos[t][pos[t] >= 0] for t in samples]))
    kept = {}

    def keep(c0, rows):
        sel = want[(want >= c0) & (want < c0 + rows.shape[0])]
        if sel.numel():
            for tok, row in zip(sel.tolist(), rows[sel - c0].float().cpu().numpy()):
                kept[tok] = row

    filled = build_mla_layer(0, "cuda", on_chunk=keep)
    assert len(kept) == want.numel()
    layer, g = filled.layer, filled.layer.global_scale
    sm = 1 / math.sqrt(192)
    for Hq in (128, 16):
        q = synth.mla_queries(T, Hq, torch.bfloat16, "cuda", 63, 0)
        out = nk.mla_sparse_decode(layer, q, filled.indices, sm)
        torch.cuda.synchronize()
        for t in samples:
            idx = filled.indices[t].cpu().numpy()
            toks = (t * ctx + pos[t].cpu().numpy())
            valid = idx >= 0
            raw = np.stack([kept[int(x)] for x in toks[valid]])
            oc, osc = oracle.mla_quantize_rows(raw, g)
            sl = torch.from_numpy(idx[valid].astype(np.int64)).cuda()
            assert np.array_equal(layer.codes[sl].cpu().numpy(), oc), f"codes differ, token {t}"
            assert np.array_equal(layer.scales[sl].cpu().numpy(), osc), f"scales differ, token {t}"
            planes = oracle.MlaPlanes(int(valid.sum()))
            planes.codes[:], planes.scales[:] = oc, osc
            local = np.full(topk, -1, np.int32)
            local[valid] = np.arange(int(valid.sum()), dtype=np.int32)
            ref = oracle.mla_sparse_decode(planes, g, host_f32(q[t:t + 1]), local[None], sm)
            err = row_rel_err(out[t].cpu().numpy().reshape(-1, 512), ref.reshape(-1, 512))
            _say(f"  Hq={Hq} token {t}: {int(valid.sum())} rows bit-exact, max row rel err {err.max():.2e}")
            assert err.max() <= ATTN_TOL
