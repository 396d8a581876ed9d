"""Pins of the oracle against the numbers the memory-wall blog prints.

* Section 2: the two-level-scaling experiment (seeded Gaussian data with a few
  outliers, printed RMSE of block+global versus global-only quantization) --
  reproduced exactly by the oracle's unrounded two-level rule, and the oracle's
  own rule (E4M3-rounded block scale, FP32 global scale, ties to even) must
  keep the large advantage.
* Section 1: the KV-cache accounting table, computed from the oracle's own
  cache layout size (bytes per token and head).
"""
import math
import os
import random

import numpy as np
import pytest

import oracle


def _kv(path):
    out = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            t = ln.split()
            out[t[0]] = t[1:]
    return out


def _page_data(cfg):
    """The section-2 data, as the page describes it: one Mersenne-Twister stream
    (Python's `random`) seeded with the page's seed gives `n` normal draws of
    standard deviation `sigma`, then `outliers` uniform positions, each set to
    `outlier_value` (a position drawn twice is set once)."""
    rng = random.Random(int(cfg["seed"][0]))
    n, sigma = int(cfg["n"][0]), float(cfg["sigma"][0])
    x = np.array([rng.gauss(0.0, sigma) for _ in range(n)], dtype=np.float64)
    for _ in range(int(cfg["outliers"][0])):
        x[rng.randrange(n)] = float(cfg["outlier_value"][0])
    return x


def _rmse(a, b):
    d = np.asarray(a, np.float64) - np.asarray(b, np.float64)
    return float(np.sqrt(np.mean(d * d)))


def test_page_rmse_reproduced_exactly(golden_dir):
    cfg = _kv(os.path.join(golden_dir, "mw_rmse.txt"))
    values = _page_data(cfg)
    blk = oracle.unrounded_block_dequant(values, int(cfg["block"][0]))
    glb = oracle.unrounded_block_dequant(values, len(values))
    assert f"{_rmse(values, blk):.6f}" == cfg["rmse_block_global"][0]
    assert f"{_rmse(values, glb):.6f}" == cfg["rmse_global_only"][0]


@pytest.mark.parametrize("gmode", ["one", "calibrated"])
def test_two_level_rule_beats_global_only(golden_dir, gmode):
    """The oracle's rule on the page's data: block+global RMSE several times lower."""
    cfg = _kv(os.path.join(golden_dir, "mw_rmse.txt"))
    values = _page_data(cfg)
    x = np.array(values, np.float32)  # the quantizer takes float32 inputs
    amax = float(np.abs(x).max())
    g = 1.0 if gmode == "one" else float(np.float32(amax) / np.float32(6 * 448))
    codes, scales = oracle.quantize_rows(x.reshape(-1, 128), g)
    deq = oracle.dequantize_rows(codes, scales, g).reshape(-1)
    xd = x.astype(np.float64)
    ours = _rmse(xd, deq)
    glb = _rmse(xd, oracle.unrounded_block_dequant(xd, xd.size))
    assert ours * 4.0 < glb, (ours, glb)
    # and it is within a few percent of the page's own unrounded-scale block result
    assert ours < 1.05 * float(cfg["rmse_block_global"][0])


def test_kv_accounting_from_layout(golden_dir):
    cfg = _kv(os.path.join(golden_dir, "mw_accounting.txt"))
    L, H, D = int(cfg["layers"][0]), int(cfg["kv_heads"][0]), int(cfg["head_dim"][0])
    gpu_gb, frac = float(cfg["gpu_gb"][0]), float(cfg["static_frac"][0])
    # the oracle's cache layout: bytes per (token, kv head) for K and V together
    nv_bytes = oracle.bytes_per_token_head()
    assert nv_bytes == 144 and nv_bytes / (2 * D) == 9 / 16
    bpv = {"bf16": 2.0, "fp8": 1.0, "nvfp4": nv_bytes / (2 * D)}
    exp_kb = dict(zip(cfg["per_token_kb"][0::2], cfg["per_token_kb"][1::2]))
    exp_sess = dict(zip(cfg["session_128k_gb"][0::2], cfg["session_128k_gb"][1::2]))
    exp_n = dict(zip(cfg["sessions_per_card"][0::2], cfg["sessions_per_card"][1::2]))
    budget = gpu_gb * 1024 ** 3 * frac
    for dt, b in bpv.items():
        per_token = 2 * L * H * D * b
        ctx = 128 * 1024
        assert f"{per_token / 1024:.1f}" == exp_kb[dt]
        assert f"{per_token * ctx / 2 ** 30:.1f}" == exp_sess[dt]
        assert str(int(budget // (per_token * ctx))) == exp_n[dt]
    exp_3m = dict(zip(cfg["session_3m_gb"][0::2], cfg["session_3m_gb"][1::2]))
    exp_cards = dict(zip(cfg["cards_3m"][0::2], cfg["cards_3m"][1::2]))
    for dt in ("fp8", "nvfp4"):
        total = 2 * L * H * D * bpv[dt] * 3_000_000 / 2 ** 30
        assert f"{total:.0f}" == exp_3m[dt]
        assert str(int(-(-total // (gpu_gb * frac)))) == exp_cards[dt]
    ratios = dict(zip(cfg["capacity_ratio"][0::2], cfg["capacity_ratio"][1::2]))
    assert f"{bpv['fp8'] / bpv['nvfp4']:.2f}" == ratios["fp8_to_nvfp4"]
    assert f"{bpv['bf16'] / bpv['nvfp4']:.2f}" == ratios["bf16_to_nvfp4"]
