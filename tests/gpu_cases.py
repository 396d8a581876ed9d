"""Shared helpers for the GPU parity tests: run one case through the HIP
library (via its C ABI) and through the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import oracle
from synthetic import synth

ATTN_TOL = 1e-3  # row-normalised max relative error of the fp32 decode output


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max_d |got - ref| / max_d |ref| per row (rows of 128)."""
    got = got.reshape(-1, 128).astype(np.float64)
    ref = ref.reshape(-1, 128).astype(np.float64)
    den = np.abs(ref).max(1)
    num = np.abs(got - ref).max(1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).contiguous().numpy()


def planes_equal(layer, planes: oracle.Planes):
    """Return the list of planes that differ (empty = bit-exact)."""
    bad = []
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        g = getattr(layer, name).cpu().numpy()
        o = getattr(planes, name)
        if not np.array_equal(g, o):
            idx = np.flatnonzero(g != o)
            bad.append((name, int(idx.size), int(idx[0]), int(g[idx[0]]), int(o[idx[0]])))
    return bad


@dataclass
class Cache:
    layer: object          # nvfp4_quantized_paged_kv_amd.KVCacheLayer (device)
    planes: oracle.Planes  # oracle's own planes
    bt: np.ndarray
    lens: list
    g_k: float
    g_v: float


def build_cache(lens, H, dtype, dist, outlier_frac, g_one, seed, extra_pages=3, device="cuda", kv=None):
    """Quantize-append every sequence's tokens with both implementations
    (kv: optional per-sequence (k, v) tensors [n, H, 128] in place of synthetic ones)."""
    import nvfp4_quantized_paged_kv_amd as nk

    bt, pool = synth.page_tables(lens, sum((n + 15) // 16 for n in lens) + extra_pages, seed=seed)
    ks, vs, slots = [], [], []
    for b, n in enumerate(lens):
        if n == 0:
            continue
        if kv is not None:
            ks.append(kv[b][0].to(dtype))
            vs.append(kv[b][1].to(dtype))
        else:
            ks.append(synth.kv_values(n, H, dist, outlier_frac, 0, dtype, "cpu", seed, b))
            vs.append(synth.kv_values(n, H, dist, outlier_frac, 1, dtype, "cpu", seed, b))
        slots.append(synth.slots_for(bt[b], 0, n))
    k = torch.cat(ks) if ks else torch.zeros((0, H, 128), dtype=dtype)
    v = torch.cat(vs) if vs else torch.zeros((0, H, 128), dtype=dtype)
    sl = np.concatenate(slots) if slots else np.zeros(0, np.int32)
    if g_one:
        g_k = g_v = 1.0
    else:
        g_k = synth.global_scale(float(k.float().abs().max()) if k.numel() else 1.0)
        g_v = synth.global_scale(float(v.float().abs().max()) if v.numel() else 1.0)
    planes = oracle.Planes(pool, H)
    oracle.quantize_append(planes, host_f32(k), host_f32(v), sl, g_k, g_v)
    layer = nk.KVCacheLayer.allocate(pool, H, g_k, g_v, device)
    nk.quantize_append(layer, k.to(device), v.to(device), torch.from_numpy(sl).to(device))
    torch.cuda.synchronize()
    return Cache(layer, planes, bt, list(lens), g_k, g_v)


def decode_both(cache: Cache, Hq, q_dtype, seed, rows=None, max_seq_len=None, q_scale=1.0, device="cuda", q=None):
    import nvfp4_quantized_paged_kv_amd as nk

    B = len(cache.lens)
    if q is None:
        q = synth.queries(B, Hq, q_dtype, "cpu", seed, 1) * q_scale
    q = q.to(q_dtype)
    msl = max(max(cache.lens), 1) if max_seq_len is None else max_seq_len
    bt = cache.bt
    need = (msl + 15) // 16
    if bt.shape[1] < need:
        bt = np.concatenate([bt, np.zeros((B, need - bt.shape[1]), np.int32)], 1)
    bt_d = torch.from_numpy(np.ascontiguousarray(bt)).to(device)
    sl_d = torch.tensor(cache.lens, dtype=torch.int32, device=device)
    out = nk.paged_decode_attn(cache.layer, q.to(device).contiguous(), bt_d, sl_d, msl, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    ref = oracle.decode_attention(cache.planes, cache.g_k, cache.g_v, host_f32(q), cache.bt,
                                  np.array(cache.lens, np.int32), float(np.float32(1 / math.sqrt(128))), rows)
    got = out.cpu().numpy().reshape(B * Hq, 128)
    if rows is not None:
        got = got[np.asarray(rows)]
    return got, ref
