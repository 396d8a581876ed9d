"""Seeded synthetic workloads for tests and the bench (no NVFP4 arithmetic here).

The shapes and value distributions stand in for the pages' workloads: 80-layer
/ 8-KV-head / head_dim-128 GQA models, 32K-1M-token contexts and
multi-million-token agentic sessions (grer.cn blog "NVFP4 KV cache and the
memory wall", sections 1 and 4).  K/V values are mostly small Gaussians with
rare large outliers, as in the blog's section-2 experiment (gauss(0, 0.02)
with a few values of 6.0).  Nothing here reads a dataset; every tensor comes
from a seeded torch generator, so the oracle and the GPU path can be given the
same inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 20261106  # the seed of the blog's section-2 experiment
HEAD_DIM = 128
PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    ctx: int                  # context length per sequence (max for ragged)
    layers: int               # layers the bench rotates over
    in_dtype: torch.dtype     # K/V/Q input dtype
    dist: str                 # "sparse6" (random +-6.0 entries) or "chan50" (2 K channels x50)
    outlier_frac: float = 0.0
    global_one: bool = False  # g = 1.0 instead of amax / (6*448)
    lens: tuple = field(default=())  # ragged lengths (mixed step); empty = all `ctx`

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 1, 256, 1, torch.float32, "sparse6", 0.005, True),
    "gqa70b_b32_8k": Workload("gqa70b_b32_8k", 32, 64, 8, 8192, 4, torch.bfloat16, "chan50"),
    "long_b8_128k": Workload("long_b8_128k", 8, 64, 8, 131072, 4, torch.bfloat16, "chan50"),
    "agentic_b1_2m": Workload("agentic_b1_2m", 1, 96, 8, 2_000_000, 8, torch.bfloat16, "sparse6", 0.002),
}


# Mixed serving step: 64 ragged sequences (log-uniform 512..65536 tokens);
# 8 of them are extended by a 2048-token chunk (their cached prefix goes
# through the FP8 workspace), the other 56 append 16 tokens and decode.
MIXED_N_EXTEND = 8
MIXED_EXTEND_NEW = 2048
MIXED_DECODE_NEW = 16


def mixed_roles(n: int = 64, n_extend: int = MIXED_N_EXTEND, seed: int = BASE_SEED + 6):
    """(extend sequence indices, decode sequence indices), both sorted."""
    rng = np.random.default_rng(seed)
    ext = np.sort(rng.choice(n, n_extend, replace=False)).astype(np.int64)
    dec = np.setdiff1d(np.arange(n), ext).astype(np.int64)
    return ext, dec


def chunk_tokens(H: int) -> int:
    """Tokens per generated chunk (about 2^27 values, 256 MiB of bf16)."""
    return max(1, (1 << 27) // (H * HEAD_DIM))


def layer_token_chunks(wl: Workload, lens, layer: int, device):
    """Yield (first_index, n, k, v) over the tokens of one layer's fill, in
    (sequence, position) order: index i is token i % n_fill... of the flattened
    list of every sequence's tokens.  k, v: [n, H, 128] in wl.in_dtype."""
    total = int(sum(lens))
    step = chunk_tokens(wl.kv_heads)
    for c0 in range(0, total, step):
        n = min(step, total - c0)
        k = kv_values(n, wl.kv_heads, wl.dist, wl.outlier_frac, 0, wl.in_dtype, device, 2, layer, c0)
        v = kv_values(n, wl.kv_heads, wl.dist, wl.outlier_frac, 1, wl.in_dtype, device, 2, layer, c0)
        yield c0, n, k, v


def token_positions(lens):
    """(sequence index, position) of every token of the flattened fill order."""
    lens = np.asarray(lens, np.int64)
    seq = np.repeat(np.arange(lens.size), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    pos = np.arange(int(lens.sum()), dtype=np.int64) - np.repeat(starts, lens)
    return seq, pos


def layer_global_scales(wl: Workload, lens, layer: int, device):
    """Calibrated (g_k, g_v) = amax/(6*448) over the layer's K and V (1.0 if wl.global_one)."""
    if wl.global_one:
        return 1.0, 1.0
    amax = [0.0, 0.0]
    for _, _, k, v in layer_token_chunks(wl, lens, layer, device):
        amax[0] = max(amax[0], float(k.float().abs().max()))
        amax[1] = max(amax[1], float(v.float().abs().max()))
    return global_scale(amax[0]), global_scale(amax[1])


def mixed_lengths(n: int = 64, lo: int = 512, hi: int = 65536, seed: int = BASE_SEED + 5) -> list[int]:
    """Log-uniform ragged lengths for the mixed serving step."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in np.exp(rng.uniform(math.log(lo), math.log(hi), n)).astype(np.int64)]


WORKLOADS["mixed_64"] = Workload("mixed_64", 64, 64, 8, 65536, 4, torch.bfloat16, "chan50",
                                 lens=tuple(mixed_lengths()))


def seed_of(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (the blog's seed first)."""
    h = BASE_SEED
    for p in parts:
        h = (h * 1_000_003 + int(p) + 0x9E3779B9) % (1 << 63)
    return h


def generator(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def kv_values(n_tokens: int, H: int, dist: str, outlier_frac: float, which: int, dtype: torch.dtype, device,
              *seed_parts: int) -> torch.Tensor:
    """K (which=0) or V (which=1) values [n_tokens, H, 128] in `dtype` (generated in f32, RNE-rounded)."""
    g = generator(device, *seed_parts, which)
    x = torch.randn((n_tokens, H, HEAD_DIM), generator=g, device=device, dtype=torch.float32) * 0.02
    if dist == "sparse6" and outlier_frac > 0:
        u = torch.rand((n_tokens, H, HEAD_DIM), generator=g, device=device)
        sign = torch.where(torch.rand((n_tokens, H, HEAD_DIM), generator=g, device=device) < 0.5, -6.0, 6.0)
        x = torch.where(u < outlier_frac, sign, x)
    elif dist == "chan50" and which == 0:
        ch = channel_outliers(seed_parts[0] if seed_parts else 0)
        x[:, :, ch] *= 50.0
    return x.to(dtype)


def channel_outliers(cfg_id: int) -> list[int]:
    """The 2 (of 128) K channels scaled by 50, the same for every head and token."""
    rng = np.random.default_rng(seed_of(cfg_id, 777))
    return sorted(int(c) for c in rng.choice(HEAD_DIM, 2, replace=False))


def queries(B: int, Hq: int, dtype: torch.dtype, device, *seed_parts: int) -> torch.Tensor:
    g = generator(device, *seed_parts, 99)
    q = torch.randn((B, Hq, HEAD_DIM), generator=g, device=device, dtype=torch.float32) / math.sqrt(HEAD_DIM)
    return q.to(dtype)


def global_scale(amax: float) -> float:
    """Calibrated FP32 global scale amax / (6 * 448) (E2M1 max times E4M3 max)."""
    return float(np.float32(amax) / np.float32(6 * 448))


def page_tables(lens, num_pages: int | None = None, seed: int = 0):
    """Block table [B, max_pages] int32 drawn from a seeded random permutation of the page pool."""
    pages_per = [(int(n) + PAGE - 1) // PAGE for n in lens]
    total = sum(pages_per)
    pool = total if num_pages is None else int(num_pages)
    assert pool >= total
    rng = np.random.default_rng(seed_of(seed, 4242))
    perm = rng.permutation(pool).astype(np.int32)
    width = max(max(pages_per), 1)
    bt = np.zeros((len(lens), width), np.int32)
    at = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, pool


def slots_for(bt_row: np.ndarray, start: int, n: int) -> np.ndarray:
    """Slots of tokens start..start+n-1 of one sequence."""
    t = np.arange(start, start + n, dtype=np.int64)
    return (bt_row[t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)


# ------------------------------------------------------- Sparse-MLA latent cache
# Stand-in for a DeepSeek-V3.2-class sparse-MLA decode: every token caches one
# latent row (512 latent + 64 rotary-key values) shared by all query heads; each
# query token attends to a top-k list of positions of its own sequence (the
# selection itself is made outside this path: here a seeded uniform draw of
# distinct positions).  Values follow the pages' cache distribution.
MLA_DIM = 576
MLA_LATENT = 512


def mla_rows(n_tokens: int, outlier_frac: float, dtype: torch.dtype, device, *seed_parts: int) -> torch.Tensor:
    """Latent rows [n_tokens, 576] in `dtype`: N(0, 0.02) with a fraction of +-6.0 entries."""
    g = generator(device, *seed_parts, 55)
    x = torch.randn((n_tokens, MLA_DIM), generator=g, device=device, dtype=torch.float32) * 0.02
    if outlier_frac > 0:
        u = torch.rand((n_tokens, MLA_DIM), generator=g, device=device)
        sign = torch.where(torch.rand((n_tokens, MLA_DIM), generator=g, device=device) < 0.5, -6.0, 6.0)
        x = torch.where(u < outlier_frac, sign, x)
    return x.to(dtype)


def mla_queries(T: int, Hq: int, dtype: torch.dtype, device, *seed_parts: int) -> torch.Tensor:
    """Absorbed queries [T, Hq, 576] ~ N(0, 1)."""
    g = generator(device, *seed_parts, 56)
    return torch.randn((T, Hq, MLA_DIM), generator=g, device=device, dtype=torch.float32).to(dtype)


def mla_topk_positions(T: int, lens, topk: int, device, *seed_parts: int) -> torch.Tensor:
    """Per query token t: min(topk, lens[t]) distinct positions of [0, lens[t]) in random order,
    padded with -1 to topk entries; int64 [T, topk]."""
    g = generator(device, *seed_parts, 57)
    out = torch.full((T, topk), -1, dtype=torch.int64, device=device)
    for t in range(T):
        n = int(lens[t])
        k = min(topk, n)
        if k > 0:
            out[t, :k] = torch.randperm(n, generator=g, device=device)[:k]
    return out


def slots_of_positions(pos: torch.Tensor, block_table: torch.Tensor, page: int) -> torch.Tensor:
    """Cache slots of positions pos [T, k] (-1 stays -1) through block_table [T, width] of `page`-token pages."""
    p = pos.clamp(min=0)
    pages = torch.gather(block_table.to(torch.int64), 1, p // page)
    return torch.where(pos >= 0, pages * page + p % page, torch.full_like(pos, -1)).to(torch.int32)
