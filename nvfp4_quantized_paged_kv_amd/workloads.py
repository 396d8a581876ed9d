"""Device-side construction of the synthetic workloads' caches, shared by the
bench and the full-size parity tests: every layer is filled by bulk
quantize-append of seeded synthetic K/V (see ``synth``), chunk by chunk, in
(sequence, position) order, at slots from a seeded random page permutation."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import KVCacheLayer, quantize_append
from . import synth


@dataclass
class FilledLayer:
    layer: KVCacheLayer
    block_table: np.ndarray     # [B, width] int32 (host)
    block_table_dev: torch.Tensor
    append_ms: list             # per-chunk append durations (HIP events), if timed
    append_bytes: list          # per-chunk algorithmic bytes


def build_layer(wl: synth.Workload, fill_lens, pool_lens, layer_idx: int, device="cuda", on_chunk=None,
                timed: bool = False) -> FilledLayer:
    """Quantize-append the first fill_lens[b] tokens of every sequence b.

    pool_lens[b] >= fill_lens[b] sizes each sequence's pages (room for tokens
    appended later).  on_chunk(c0, n, k, v, seq, pos) sees every generated chunk."""
    pool_lens = [int(x) for x in pool_lens]
    bt, pool = synth.page_tables(pool_lens, seed=1000 + layer_idx)
    g_k, g_v = synth.layer_global_scales(wl, fill_lens, layer_idx, device)
    layer = KVCacheLayer.allocate(pool, wl.kv_heads, g_k, g_v, device)
    seq_all, pos_all = synth.token_positions(fill_lens)
    stream = torch.cuda.current_stream()
    ms, by = [], []
    for c0, n, k, v in synth.layer_token_chunks(wl, fill_lens, layer_idx, device):
        seq, pos = seq_all[c0:c0 + n], pos_all[c0:c0 + n]
        slots = (bt[seq, pos // synth.PAGE].astype(np.int64) * synth.PAGE + pos % synth.PAGE).astype(np.int32)
        sl = torch.from_numpy(slots).to(device)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        quantize_append(layer, k, v, sl)
        if timed:
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
            by.append(n * wl.kv_heads * (2 * 128 * k.element_size() + 144) + 4 * n)
        if on_chunk is not None:
            on_chunk(c0, n, k, v, seq, pos)
        del k, v
    return FilledLayer(layer, bt, torch.from_numpy(bt).to(device), ms, by)
