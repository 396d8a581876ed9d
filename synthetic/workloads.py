"""Device-side construction of the synthetic workloads' caches, shared by the
bench and the full-size parity tests: every layer is filled by bulk
quantize-append of seeded synthetic K/V (see ``synth``), chunk by chunk, in
(sequence, position) order, at slots from a seeded random page permutation."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from nvfp4_quantized_paged_kv_amd import KVCacheLayer, MxKVCacheLayer, mx_quantize_append, quantize_append
from synthetic import synth


@dataclass
class FilledLayer:
    layer: KVCacheLayer         # (MxKVCacheLayer for an MXFP4 fill)
    block_table: np.ndarray     # [B, width] int32 (host)
    block_table_dev: torch.Tensor
    append_ms: list             # per-chunk append durations (HIP events), if timed
    append_bytes: list          # per-chunk algorithmic bytes


def build_layer(wl: synth.Workload, fill_lens, pool_lens, layer_idx: int, device="cuda", on_chunk=None,
                timed: bool = False, mx: bool = False, hadamard: bool = False) -> FilledLayer:
    """Quantize-append the first fill_lens[b] tokens of every sequence b.

    pool_lens[b] >= fill_lens[b] sizes each sequence's pages (room for tokens
    appended later).  on_chunk(c0, n, k, v, seq, pos) sees every generated chunk.
    mx: fill an MXFP4 layer with the same tokens, slots and page table.
    hadamard: store K Hadamard-rotated (the global scales stay those of the unrotated K)."""
    pool_lens = [int(x) for x in pool_lens]
    bt, pool = synth.page_tables(pool_lens, seed=1000 + layer_idx)
    if mx:
        layer = MxKVCacheLayer.allocate(pool, wl.kv_heads, device)
        append, per_head = mx_quantize_append, 2 * 68
    else:
        g_k, g_v = synth.layer_global_scales(wl, fill_lens, layer_idx, device)
        layer = KVCacheLayer.allocate(pool, wl.kv_heads, g_k, g_v, device)
        append, per_head = quantize_append, 2 * 72
    seq_all, pos_all = synth.token_positions(fill_lens)
    stream = torch.cuda.current_stream()
    ms, by = [], []
    for c0, n, k, v in synth.layer_token_chunks(wl, fill_lens, layer_idx, device):
        seq, pos = seq_all[c0:c0 + n], pos_all[c0:c0 + n]
        slots = (bt[seq, pos // synth.PAGE].astype(np.int64) * synth.PAGE + pos % synth.PAGE).astype(np.int32)
        sl = torch.from_numpy(slots).to(device)
        if timed:
            # keep the GPU busy while the host prepares the launch, so the
            # events bracket the kernel and not the host-side call overhead
            torch.cuda._sleep(1 << 20)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        append(layer, k, v, sl, hadamard=hadamard)
        if timed:
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
            by.append(n * wl.kv_heads * (2 * 128 * k.element_size() + per_head) + 4 * n)
        if on_chunk is not None:
            on_chunk(c0, n, k, v, seq, pos)
        del k, v
    return FilledLayer(layer, bt, torch.from_numpy(bt).to(device), ms, by)


def first_chunk(wl: synth.Workload, fill_lens, layer_idx: int, block_table: np.ndarray, device="cuda"):
    """The first chunk build_layer appends to layer layer_idx: (k, v, slots) on
    the device, the same tokens and slots, so appending it again rewrites the
    same bytes."""
    seq_all, pos_all = synth.token_positions(fill_lens)
    c0, n, k, v = next(iter(synth.layer_token_chunks(wl, fill_lens, layer_idx, device)))
    seq, pos = seq_all[c0:c0 + n], pos_all[c0:c0 + n]
    slots = (block_table[seq, pos // synth.PAGE].astype(np.int64) * synth.PAGE + pos % synth.PAGE).astype(np.int32)
    return k, v, torch.from_numpy(slots).to(device)


@dataclass
class MixedStep:
    """One layer of the mixed serving step, ready to run."""
    filled: FilledLayer
    lens: list                  # cached tokens per sequence before the step
    extend: np.ndarray          # indices of the extended sequences
    decode: np.ndarray          # indices of the decoding sequences
    new_k: torch.Tensor         # [T_new, H, 128] all new tokens of the step
    new_v: torch.Tensor
    new_slots: torch.Tensor     # [T_new] int32
    new_seq: np.ndarray         # sequence of each new token
    new_pos: np.ndarray         # position of each new token
    dec_table: torch.Tensor     # [56, width] block-table rows of the decoding sequences
    dec_lens: torch.Tensor      # [56] lengths after the append (L + 16)
    dec_q: torch.Tensor         # [56, Hq, 128]
    ext_table: torch.Tensor     # [8, width] block-table rows of the extended sequences
    ext_prefix: torch.Tensor    # [8] cached prefix lengths (L)
    ext_offsets: torch.Tensor   # [9] workspace token offsets: sequence i's rows [prefix | 2048-token chunk]
    ext_rows: torch.Tensor      # [T_new] workspace row of each new token of an extended sequence, -1 otherwise
    ext_q: torch.Tensor         # [8 * 2048, Hq, 128] queries of the extend chunks
    ext_q_offsets: torch.Tensor  # [9] chunk query rows per extended sequence
    max_dec_len: int
    max_prefix: int
    ext_chunk: int              # tokens per extend chunk


def build_mixed_step(wl: synth.Workload, layer_idx: int, device="cuda", on_chunk=None, timed=False) -> MixedStep:
    lens = list(wl.lens)
    ext, dec = synth.mixed_roles(len(lens))
    grow = np.full(len(lens), synth.MIXED_DECODE_NEW, np.int64)
    grow[ext] = synth.MIXED_EXTEND_NEW
    pool_lens = (np.asarray(lens) + grow).tolist()
    fl = build_layer(wl, lens, pool_lens, layer_idx, device, on_chunk=on_chunk, timed=timed)
    bt = fl.block_table
    new_seq = np.repeat(np.arange(len(lens)), grow)
    new_pos = np.concatenate([np.arange(lens[b], lens[b] + grow[b]) for b in range(len(lens))])
    T_new = new_seq.size
    new_k = synth.kv_values(T_new, wl.kv_heads, wl.dist, wl.outlier_frac, 0, wl.in_dtype, device, 3, layer_idx)
    new_v = synth.kv_values(T_new, wl.kv_heads, wl.dist, wl.outlier_frac, 1, wl.in_dtype, device, 3, layer_idx)
    slots = (bt[new_seq, new_pos // synth.PAGE].astype(np.int64) * synth.PAGE + new_pos % synth.PAGE).astype(np.int32)
    dec_lens = np.asarray(lens)[dec] + synth.MIXED_DECODE_NEW
    prefix = np.asarray(lens)[ext]
    chunk = synth.MIXED_EXTEND_NEW
    offs = np.concatenate([[0], np.cumsum(prefix + chunk)]).astype(np.int32)  # room for prefix and chunk
    ext_rows = np.full(T_new, -1, np.int64)
    for i, b in enumerate(ext):
        mine = np.flatnonzero(new_seq == b)
        ext_rows[mine] = offs[i] + new_pos[mine]  # new_pos runs lens[b] .. lens[b] + chunk - 1
    return MixedStep(
        filled=fl, lens=lens, extend=ext, decode=dec, new_k=new_k, new_v=new_v,
        new_slots=torch.from_numpy(slots).to(device), new_seq=new_seq, new_pos=new_pos,
        dec_table=torch.from_numpy(np.ascontiguousarray(bt[dec])).to(device),
        dec_lens=torch.from_numpy(dec_lens.astype(np.int32)).to(device),
        dec_q=synth.queries(dec.size, wl.q_heads, wl.in_dtype, device, 4, layer_idx),
        ext_table=torch.from_numpy(np.ascontiguousarray(bt[ext])).to(device),
        ext_prefix=torch.from_numpy(prefix.astype(np.int32)).to(device),
        ext_offsets=torch.from_numpy(offs).to(device),
        ext_rows=torch.from_numpy(ext_rows.astype(np.int32)).to(device),
        ext_q=synth.queries(ext.size * chunk, wl.q_heads, wl.in_dtype, device, 5, layer_idx),
        ext_q_offsets=torch.from_numpy((np.arange(ext.size + 1) * chunk).astype(np.int32)).to(device),
        max_dec_len=int(dec_lens.max()), max_prefix=int(prefix.max()), ext_chunk=chunk)


# ------------------------------------------------------- Sparse-MLA latent cache
# DeepSeek-V3.2-class sparse-MLA decode: T query tokens (one per sequence),
# each sequence holds ctx cached tokens in `page`-token pages of a seeded random
# permutation; each query token attends to topk distinct positions of its own
# sequence.
MLA_SHAPE = dict(T=128, Hq=128, ctx=32768, topk=2048, page=64, layers=4)
MLA_CHUNK = 1 << 17
MLA_OUTLIERS = 0.002


@dataclass
class MlaFilled:
    layer: object               # nvfp4_quantized_paged_kv_amd.MlaCacheLayer
    block_table: torch.Tensor   # [T, ctx / page] int64 page indices
    indices: torch.Tensor       # [T, topk] int32 cache slots of each query token's list
    append_ms: list             # per-chunk append durations (HIP events), if timed


def mla_slots(bt: torch.Tensor, tok: torch.Tensor, ctx: int, page: int) -> torch.Tensor:
    """Cache slots of flattened token indices tok (sequence tok // ctx, position tok % ctx)."""
    pos = tok % ctx
    return (bt[tok // ctx, pos // page] * page + pos % page).to(torch.int32)


def build_mla_layer(layer_idx: int, device="cuda", shape=None, on_chunk=None, timed: bool = False) -> MlaFilled:
    """Fill one layer's latent cache by bulk quantize-append of seeded rows,
    chunk by chunk in (sequence, position) order.  on_chunk(c0, rows) sees every
    generated chunk (rows [n, 576] bf16 of tokens c0 .. c0+n-1)."""
    from nvfp4_quantized_paged_kv_amd import MlaCacheLayer, mla_quantize_append

    sh = dict(MLA_SHAPE if shape is None else shape)
    T, ctx, topk, page = sh["T"], sh["ctx"], sh["topk"], sh["page"]
    n_slots = T * ctx
    amax = 0.0
    for c0 in range(0, n_slots, MLA_CHUNK):
        rows = synth.mla_rows(min(MLA_CHUNK, n_slots - c0), MLA_OUTLIERS, torch.bfloat16, device, 60, layer_idx, c0)
        amax = max(amax, float(rows.float().abs().max()))
    layer = MlaCacheLayer.allocate(n_slots, synth.global_scale(amax), device)
    perm = np.random.default_rng(synth.seed_of(layer_idx, 61)).permutation(n_slots // page).astype(np.int64)
    bt = torch.from_numpy(perm).to(device).reshape(T, ctx // page)
    stream = torch.cuda.current_stream()
    ms = []
    for c0 in range(0, n_slots, MLA_CHUNK):
        n = min(MLA_CHUNK, n_slots - c0)
        rows = synth.mla_rows(n, MLA_OUTLIERS, torch.bfloat16, device, 60, layer_idx, c0)
        slots = mla_slots(bt, torch.arange(c0, c0 + n, device=device), ctx, page)
        if timed:
            torch.cuda._sleep(1 << 20)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        mla_quantize_append(layer, rows, slots)
        if timed:
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        if on_chunk is not None:
            on_chunk(c0, rows)
    pos = synth.mla_topk_positions(T, [ctx] * T, topk, device, 62, layer_idx)
    idx = synth.slots_of_positions(pos, bt, page)
    return MlaFilled(layer, bt, idx, ms)
