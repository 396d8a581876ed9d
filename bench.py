"""Benchmark of the NVFP4 paged-KV hot path on one MI355X.

Default workload: agentic single-session decode -- batch 1, 96 query heads /
8 KV heads, head_dim 128, a 2,000,000-token context resident as NVFP4 pages in
random page order, bf16 K/V ~ N(0, 0.02) with 0.2% of entries set to +-6.0,
FP32 global scales amax/(6*448).  Eight layer caches (2.3 GB of pages each)
are filled by bulk quantize-append and the timed step rotates over them, so a
step never finds its layer in the 256 MB Infinity Cache.  One step = append
the sequence's new token + decode attention over the whole context, as one
call of the library's decode step (the same step as two explicit calls is
reported beside it).  `--workload` selects the other shapes (70B-class batch
32 at 8K, batch 8 at 128K, the mixed serving step, the tiny case).

Timing.  `value` and `ms_per_step` come from the median of several windows of
exactly --steps step calls, each window bracketed by torch.cuda.synchronize()
on both sides and timed by the wall clock (min and max beside it).  Kernel
rooflines use HIP events on the launch stream around calls queued back to
back (median of several windows, each led by untimed calls so that the GPU is
already busy with the same work when the first event is taken).

Printed: one JSON line -- decode-step effective HBM GB/s (algorithmic bytes of
append + decode per step / step time), the decode kernel's roofline, the bulk
quantize-append GB/s and its roofline, the FP8 workspace dequant, multi-token
decode, the MXFP4 comparison format and Hadamard-rotated K on the same tokens,
and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0  # dense f16 / bf16 MFMA
PEAK_F8_TFLOPS = 5000.0   # dense fp8 MFMA
METRIC = "decode-attn effective HBM GB/s (% of 8 TB/s) + quantize-append GB/s"
# Windows of the headline step timing (each exactly --steps calls between two synchronizations)
STEP_WINDOWS = 7
# Back-to-back kernel timing: untimed calls queued ahead of each timed window, and windows per figure
LEAD_CALLS = 8
SUSTAIN_S = 0.75  # seconds of the same call before each timed section (see sustain())
B2B_WINDOWS = 5
# Layer caches larger than this are already far beyond the 256 MB Infinity Cache in pairs:
# the comparison formats (MXFP4, rotated K) rotate over two of them instead of every layer
BIG_LAYER_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="agentic_b1_2m",
                    choices=["agentic_b1_2m", "gqa70b_b32_8k", "long_b8_128k", "mixed_64", "tiny"])
    ap.add_argument("--layers", type=int, default=0, help="override the number of rotated layer caches")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step, the decode and the bulk append (no MXFP4 / rotated / workspace)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--sustain", type=float, default=None,
                    help="seconds of the same call, untimed, before each timed section (default %.2f)" % SUSTAIN_S)
    ap.add_argument("--calibrate", action="store_true",
                    help="after the timed region, run a 1 GiB float32 elementwise add (reads 1 GiB, writes "
                         "1 GiB) so hardware byte counters can be scaled against a kernel of known size")
    return ap.parse_args()


def src_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = os.path.join(ROOT, "nvfp4_quantized_paged_kv_amd", "csrc")
# The decode kernel's source: the kernel file and the headers it includes.
DECODE_SOURCES = [os.path.join(_CSRC, n)
                  for n in ("decode_attn.hip", "nvfp4_kv_internal.h", "nvfp4_device.h", "nvfp4_quant_device.h")]
# The bulk quantize-append kernel's source.
APPEND_SOURCES = [os.path.join(_CSRC, n)
                  for n in ("quant_append.hip", "nvfp4_kv_internal.h", "nvfp4_device.h", "nvfp4_quant_device.h")]


def spread(xs, scale=1.0, nd=3):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64) * scale
    return {"n": int(a.size), "median": round(float(np.median(a)), nd), "min": round(float(a.min()), nd),
            "max": round(float(a.max()), nd)}


def sustain(launch, seconds=None):
    """Untimed: run `launch` continuously for `seconds` of wall time (batches of
    16 calls between synchronizations).  After even a short idle (host-side
    set-up between two timed sections is enough) the GPU's power management
    runs the next milliseconds of work at lower clocks: the 70B-class decode
    measured 64-79 us per call in windows right after 1-3 s idle, and 57 us
    after a few seconds of any sustained work (the same decode, elementwise
    adds or GEMMs).  A serving loop runs in the sustained state, so every timed
    section starts from it."""
    import torch
    seconds = SUSTAIN_S if seconds is None else seconds
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            launch(i)
            i += 1
        torch.cuda.synchronize()


def sync_windows(launch, steps: int, windows: int):
    """The headline timing: `windows` windows of exactly `steps` calls, each
    bracketed by torch.cuda.synchronize() on both sides.  Returns the wall
    seconds per call of every window and the HIP-event seconds per call (events
    on the launch stream, recorded at the window's first and last call)."""
    import torch
    stream = torch.cuda.current_stream()
    wall, ev = [], []
    sustain(launch)
    for w in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            launch(w * steps + i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t0) / steps)
        ev.append(e0.elapsed_time(e1) / 1e3 / steps)
    return wall, ev


def back_to_back(stream, n, launch, windows=B2B_WINDOWS, spread_out=None):
    """Per-call GPU time of n calls queued back to back between one event pair
    on `stream`: the median over `windows` windows.  Each window is led by
    LEAD_CALLS untimed calls, so the GPU is already busy with the same work
    (no idle gap, no clock ramp) when the first event is taken and the host
    queues the timed calls while earlier ones run.  Warns on stderr if the host
    took longer to queue a window than the GPU took to run it.  spread_out, if
    a list, receives every window's per-call seconds."""
    import numpy as np
    import torch
    per_call = []
    sustain(launch)
    for w in range(windows):
        torch.cuda.synchronize()
        for i in range(LEAD_CALLS):
            launch(i)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        t0 = time.perf_counter()
        for i in range(n):
            launch(LEAD_CALLS + i)
        host_s = time.perf_counter() - t0
        d1.record(stream)
        torch.cuda.synchronize()
        gpu_s = d0.elapsed_time(d1) / 1e3
        if host_s > gpu_s:
            print(f"[bench] warning: queueing {n} calls took {host_s * 1e3:.2f} ms, longer than their "
                  f"{gpu_s * 1e3:.2f} ms on the GPU; the back-to-back time includes host gaps", file=sys.stderr)
        per_call.append(gpu_s / n)
    if spread_out is not None:
        spread_out.extend(per_call)
    return float(np.median(per_call))


def append_b2b(stream, steps, chunks, targets, append, per_head, **kw):
    """Bulk quantize-append timed like decode: calls queued back to back, each
    re-appending the first fill chunk of a layer (the same tokens into the same
    slots, so the cache keeps its bytes), alternating over the layers so that
    no call finds its inputs in the caches.  Returns (us per call, GB/s of
    algorithmic bytes, algorithmic bytes per call)."""
    def launch(i):
        j = i % len(chunks)
        k, v, sl = chunks[j]
        append(targets[j], k, v, sl, **kw)
    s = back_to_back(stream, steps, launch)
    k0 = chunks[0][0]
    n, H = k0.shape[0], k0.shape[1]
    b = n * H * (2 * 128 * k0.element_size() + per_head) + 4 * n
    return s * 1e6, b / s / 1e9, b


def read_profile(workload: str):
    """key: value lines of the committed rocprofv3 HBM-counter summary of a workload."""
    prof = os.path.join(ROOT, "profiles", f"decode_attn_{workload}_pmc.txt")
    vals = {}
    if os.path.exists(prof):
        with open(prof) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    vals[k.strip()] = v.strip()
    return vals


def read_traffic(kernel_files, workload: str, key: str = "hbm_bytes_per_call",
                 hash_key: str = "kernel_source_sha256_16"):
    """HBM traffic per call (decode by default; `key` picks another kernel's
    figure) from the committed rocprofv3 PMC summary, if it was taken on the
    current kernel source; else None."""
    vals = read_profile(workload)
    if not vals or vals.get(hash_key) != src_hash(kernel_files):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, target_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    sequences of up to 8192 tokens (all KV heads) generated on the host with the
    workload's value distribution, quantized and attended by the oracle; rate in
    the metric's unit (decode GB/s over the same algorithmic bytes as the GPU)."""
    import numpy as np
    import torch

    import oracle
    from synthetic import synth

    H, ctx = wl.kv_heads, min(wl.ctx, 8192)
    in_b = 2 if wl.in_dtype == torch.bfloat16 else 4
    sm = float(np.float32(1 / math.sqrt(128)))
    done_bytes = 0
    t_dec = 0.0
    t_q = 0.0
    q_bytes = 0
    seqs = 0
    while t_dec + t_q < target_s and seqs < max(wl.batch, 64):
        k = synth.kv_values(ctx, H, wl.dist, wl.outlier_frac, 0, wl.in_dtype, "cpu", 900 + seqs)
        v = synth.kv_values(ctx, H, wl.dist, wl.outlier_frac, 1, wl.in_dtype, "cpu", 900 + seqs)
        g_k = 1.0 if wl.global_one else synth.global_scale(float(k.float().abs().max()))
        g_v = 1.0 if wl.global_one else synth.global_scale(float(v.float().abs().max()))
        kf = k.float().numpy()
        vf = v.float().numpy()
        n_pages = (ctx + 15) // 16
        planes = oracle.Planes(n_pages, H)
        slots = np.arange(ctx, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.quantize_append(planes, kf, vf, slots, g_k, g_v)
        t_q += time.perf_counter() - t0
        q_bytes += ctx * H * (2 * 128 * k.element_size() + 144) + 4 * ctx
        q = synth.queries(1, wl.q_heads, wl.in_dtype, "cpu", 900 + seqs).float().numpy()
        bt = np.arange(n_pages, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        oracle.decode_attention(planes, g_k, g_v, q, bt, np.array([ctx], np.int32), sm)
        t_dec += time.perf_counter() - t0
        done_bytes += ctx * H * 144 + n_pages * 4 + wl.q_heads * 128 * (in_b + 4)
        seqs += 1
    return {
        "value": round(done_bytes / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{seqs} sequence(s) x {ctx} tokens x {H} kv heads x {wl.q_heads} q heads "
                  f"(the workload's value distribution): oracle decode {t_dec:.2f} s; oracle quantize "
                  f"{t_q:.2f} s ({q_bytes / t_q / 1e9:.4f} GB/s)",
        "quantize_gbps": round(q_bytes / t_q / 1e9, 4),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def warm_kernels(wl, dev):
    """One tiny call of each library kernel before anything is timed: the first
    launch of a kernel pays a one-time code-object load (about 1 ms), which is
    not part of the per-call cost."""
    import torch
    import nvfp4_quantized_paged_kv_amd as nk

    H = wl.kv_heads
    layer = nk.KVCacheLayer.allocate(2, H, 1e-3, 1e-3, dev)
    x = torch.zeros((4, H, 128), dtype=wl.in_dtype, device=dev)
    nk.quantize_append(layer, x, x, torch.arange(4, dtype=torch.int32, device=dev))
    bt = torch.zeros((1, 2), dtype=torch.int32, device=dev)
    sl = torch.full((1,), 4, dtype=torch.int32, device=dev)
    q = torch.zeros((1, wl.q_heads, 128), dtype=wl.in_dtype, device=dev)
    nk.paged_decode_attn(layer, q, bt, sl, 4, 0.088)
    ws = torch.zeros((4, H, 128), dtype=torch.uint8, device=dev)
    nk.dequant_to_fp8_workspace(layer, bt, sl, torch.tensor([0, 4], dtype=torch.int32, device=dev), 4, 1.0, 1.0,
                                ws, ws.clone())
    rows = torch.arange(4, dtype=torch.int32, device=dev)
    nk.fp8_rows_to_workspace(x, x, rows, 1.0, 1.0, ws, ws.clone())
    qx = torch.zeros((4, wl.q_heads, 128), dtype=wl.in_dtype, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    nk.fp8_extend_attn(qx, torch.tensor([0, 4], dtype=torch.int32, device=dev), zero, zero, 4, ws, ws.clone(), 1.0,
                       1.0, 0.088)
    mx = nk.MxKVCacheLayer.allocate(2, H, dev)
    for rot in (False, True):
        nk.quantize_append(layer, x, x, torch.arange(4, dtype=torch.int32, device=dev), hadamard=rot)
        nk.paged_decode_attn(layer, q, bt, sl, 4, 0.088, hadamard=rot)
        nk.mx_quantize_append(mx, x, x, torch.arange(4, dtype=torch.int32, device=dev), hadamard=rot)
        nk.mx_paged_decode_attn(mx, q, bt, sl, 4, 0.088, hadamard=rot)
    torch.cuda.synchronize()


def bench_mixed(args, wl, dev):
    """Mixed serving step per layer: quantize-append every new token (16 per
    decoding sequence, 2048 per extended sequence), dequantize the extended
    sequences' cached prefixes into the one FP8 workspace pair every layer
    reuses, then decode attention for the 56 decoding sequences.  The extend
    chunks' attention (compute-bound, on MFMA) and the FP8 rows of their K/V
    are timed beside the step and reported with their own roofline; the
    step's GB/s value covers the memory-bound kernels above."""
    import numpy as np
    import torch

    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic.workloads import build_mixed_step, first_chunk
    warm_kernels(wl, dev)

    L = args.layers or wl.layers
    stream = torch.cuda.current_stream()
    steps = []
    append_ms, append_bytes = [], []
    for l in range(L):
        st = build_mixed_step(wl, l, dev, timed=True)
        append_ms += st.filled.append_ms
        append_bytes += st.filled.append_bytes
        steps.append(st)
        print(f"[bench] layer {l} filled", file=sys.stderr, flush=True)
    s0 = steps[0]
    H, Hq = wl.kv_heads, wl.q_heads
    n_dec, n_ext = s0.decode.size, s0.extend.size
    ws_cap = int(s0.ext_offsets[-1].item())  # prefix and chunk rows of the 8 extended sequences
    ws_prefix = int(s0.ext_prefix.sum().item())
    ws_k = torch.empty((ws_cap, H, 128), dtype=torch.uint8, device=dev)  # one pair for every layer
    ws_v = torch.empty_like(ws_k)
    out = torch.empty((n_dec, Hq, 128), dtype=torch.float32, device=dev)
    dws = nk.decode_workspace(n_dec, Hq, H, s0.max_dec_len, dev)
    in_b = s0.new_k.element_size()
    t_new = s0.new_slots.numel()
    dec_tokens = int(s0.dec_lens.sum().item())
    dec_pages = int(((s0.dec_lens + 15) // 16).sum().item())
    ext_pages = int(((s0.ext_prefix + 15) // 16).sum().item())
    b_app = t_new * H * (2 * 128 * in_b + 144) + 4 * t_new
    b_ws = ws_prefix * H * (144 + 256) + ext_pages * 4
    b_dec = dec_tokens * H * 144 + dec_pages * 4 + n_dec * Hq * 128 * (in_b + 4)
    sm = 1 / math.sqrt(128)

    def app_call(i):
        st = steps[i % L]
        nk.quantize_append(st.filled.layer, st.new_k, st.new_v, st.new_slots)

    def ws_call(i):
        st = steps[i % L]
        nk.dequant_to_fp8_workspace(st.filled.layer, st.ext_table, st.ext_prefix, st.ext_offsets, st.max_prefix,
                                    6 * st.filled.layer.k_global, 6 * st.filled.layer.v_global, ws_k, ws_v)

    def dec_call(i):
        st = steps[i % L]
        nk.paged_decode_attn(st.filled.layer, st.dec_q, st.dec_table, st.dec_lens, st.max_dec_len, sm, out=out,
                             workspace=dws)

    def step(i):
        app_call(i)
        ws_call(i)
        dec_call(i)

    for l in range(L):  # set-up: touch every layer once
        step(l)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    wall, ev = sync_windows(step, args.steps, STEP_WINDOWS)
    per_step = float(np.median(wall))
    step_b2b = back_to_back(stream, args.steps, step)
    dec_spread = []
    dec_b2b = back_to_back(stream, args.steps, dec_call, spread_out=dec_spread)
    app_b2b = back_to_back(stream, args.steps, app_call)
    ws_b2b = back_to_back(stream, args.steps, ws_call)
    # bulk append back to back over the first fill chunk of two layers
    b2b_layers = list(range(min(L, 2)))
    bulk_us, bulk_gbs, _ = append_b2b(stream, args.steps,
                                      [first_chunk(wl, list(wl.lens), l, steps[l].filled.block_table, dev)
                                       for l in b2b_layers],
                                      [steps[l].filled.layer for l in b2b_layers], nk.quantize_append, 144)

    # ---- extend chunks: their K/V as FP8 rows after each prefix, then causal
    # attention of the chunk queries over [prefix | chunk] in the workspace
    ext_out = torch.empty((s0.ext_q.shape[0], Hq, 128), dtype=torch.float32, device=dev)
    scales = lambda st: (6 * st.filled.layer.k_global, 6 * st.filled.layer.v_global)

    def rows_call(i):
        st = steps[i % L]
        nk.fp8_rows_to_workspace(st.new_k, st.new_v, st.ext_rows, *scales(st), ws_k, ws_v)
    rows_s = back_to_back(stream, args.steps, rows_call)
    t_ext = int(s0.ext_q.shape[0])
    b_rows = t_ext * H * 128 * (2 * in_b + 2) + 4 * t_new

    def ext_call(i):
        st = steps[i % L]
        nk.fp8_extend_attn(st.ext_q, st.ext_q_offsets, st.ext_offsets[:-1], st.ext_prefix, st.ext_chunk, ws_k, ws_v,
                           *scales(st), sm, out=ext_out)
    ext_s = back_to_back(stream, max(4, args.steps // 5), ext_call, windows=3)
    ext8_out = torch.empty_like(ext_out)

    def ext8_call(i):  # the same attention in FP8 arithmetic (Q and the weights in E4M3, FP8 MFMA)
        st = steps[i % L]
        nk.fp8_extend_attn_f8(st.ext_q, st.ext_q_offsets, st.ext_offsets[:-1], st.ext_prefix, st.ext_chunk,
                              st.max_prefix, ws_k, ws_v, *scales(st), sm, out=ext8_out)
    ext8_s = back_to_back(stream, max(4, args.steps // 5), ext8_call, windows=3)
    C = s0.ext_chunk
    pairs = sum(C * int(p) + C * (C + 1) // 2 for p in s0.ext_prefix.cpu().numpy())  # (query token, key) pairs
    ext_flops = pairs * Hq * 4 * 128  # QK^T and PV: 2 x 128 multiply-adds per (query row, key)
    ext_tf = ext_flops / ext_s / 1e12
    ext8_tf = ext_flops / ext8_s / 1e12

    b_step = b_app + b_ws + b_dec
    achieved = b_dec / dec_b2b / 1e9
    return {
        "value": round(b_step / per_step / 1e9, 2),
        "ms_per_step": round(per_step * 1e3, 5),
        "ms_per_step_windows": spread(wall, 1e3, 5),
        "ms_per_step_events_windows": spread(ev, 1e3, 5),
        "step_us_b2b": round(step_b2b * 1e6, 3),
        "config": {"workload": wl.name, "sequences": len(s0.lens), "decode_sequences": int(n_dec),
                   "extend_sequences": int(n_ext), "q_heads": Hq, "kv_heads": H, "head_dim": 128, "page_size": 16,
                   "layers_rotated": L, "new_tokens": int(t_new), "decode_tokens": dec_tokens,
                   "workspace_tokens": ws_prefix, "workspace_rows": ws_cap,
                   "step": "append 16/2048 tokens + FP8 workspace dequant of 8 prefixes + decode of 56, one layer"},
        "pct_of_peak": round(100 * b_step / per_step / 1e9 / PEAK_HBM_GBS, 2),
        "decode_attn_gbs_events": round(achieved, 2),
        "decode_attn_us": round(dec_b2b * 1e6, 3),
        "decode_attn_us_windows": spread(dec_spread, 1e6),
        "append_step_gbs": round(b_app / app_b2b / 1e9, 2),
        "append_step_us": round(app_b2b * 1e6, 3),
        "fp8_workspace_gbs": round(b_ws / ws_b2b / 1e9, 2),
        "fp8_workspace_us": round(ws_b2b * 1e6, 3),
        "fp8_rows_us": round(rows_s * 1e6, 3),
        "fp8_rows_gbs": round(b_rows / rows_s / 1e9, 2),
        "extend_attn_us": round(ext_s * 1e6, 2),
        "extend_attn_tflops": round(ext_tf, 2),
        "extend_roofline": {"bound": "mfma", "achieved": round(ext_tf, 2), "peak": PEAK_F16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ext_tf / PEAK_F16_TFLOPS, 4),
                            "kernel": "nvfp4_fp8_extend_attn (extend_kernel)", "flops_per_call": int(ext_flops),
                            "query_tokens": t_ext, "key_pairs": int(pairs)},
        "extend_attn_f8_us": round(ext8_s * 1e6, 2),
        "extend_attn_f8_tflops": round(ext8_tf, 2),
        "extend_f8_roofline": {"bound": "mfma", "achieved": round(ext8_tf, 2), "peak": PEAK_F8_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(ext8_tf / PEAK_F8_TFLOPS, 4),
                               "frac_of_f16_peak": round(ext8_tf / PEAK_F16_TFLOPS, 4),
                               "kernel": "nvfp4_fp8_extend_attn_f8 (extend_f8_kernel)",
                               "flops_per_call": int(ext_flops)},
        "quantize_append_bulk_gbs": round(bulk_gbs, 2),
        "quantize_append_bulk_us": round(bulk_us, 2),
        "quantize_append_bulk_gbs_single_call": round(sum(append_bytes) / (sum(append_ms) / 1e3) / 1e9, 2),
        "bytes_per_step": int(b_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": read_traffic(DECODE_SOURCES, wl.name),
                     "kernel": "nvfp4_paged_decode_attn", "algorithmic_bytes_per_call": int(b_dec)},
    }


def bench_uniform(args, wl, dev):
    """Equal-length batches (the tiny, 70B-class, 128K and 2M-token workloads)."""
    import numpy as np
    import torch

    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic import synth
    from synthetic.workloads import build_layer, first_chunk

    L = args.layers or wl.layers
    B, Hq, H, ctx = wl.batch, wl.q_heads, wl.kv_heads, wl.ctx
    pages_per_seq = (ctx + 15) // 16
    layer_bytes = B * pages_per_seq * H * 2304
    L_x = min(L, 2) if layer_bytes >= BIG_LAYER_BYTES else L  # layers of the comparison formats
    stream = torch.cuda.current_stream()
    print(f"[bench] workload {wl.name}: B={B} Hq={Hq} H={H} ctx={ctx} layers={L}", file=sys.stderr, flush=True)

    # ---- build L layer caches (bulk quantize-append of ctx-1 tokens per sequence, timed)
    warm_kernels(wl, dev)
    layers, tables, newk, newv, slots_new, qs, bts = [], [], [], [], [], [], []
    append_ms, append_bytes = [], []
    for l in range(L):
        fl = build_layer(wl, [ctx - 1] * B, [ctx] * B, l, dev, timed=True)
        append_ms += fl.append_ms
        append_bytes += fl.append_bytes
        layers.append(fl.layer)
        tables.append(fl.block_table_dev)
        bt_np = fl.block_table
        bts.append(bt_np)
        newk.append(synth.kv_values(B, H, wl.dist, wl.outlier_frac, 0, wl.in_dtype, dev, 3, l))
        newv.append(synth.kv_values(B, H, wl.dist, wl.outlier_frac, 1, wl.in_dtype, dev, 3, l))
        slots_new.append(torch.from_numpy(
            (bt_np[:, (ctx - 1) // 16].astype(np.int64) * 16 + (ctx - 1) % 16).astype(np.int32)).to(dev))
        qs.append(synth.queries(B, Hq, wl.in_dtype, dev, 4, l))
        print(f"[bench] layer {l} filled (g_k={fl.layer.k_global:.3e} g_v={fl.layer.v_global:.3e})",
              file=sys.stderr, flush=True)

    seq_lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    sm = 1 / math.sqrt(128)
    workspace = nk.decode_workspace(B, Hq, H, ctx, dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    in_b = newk[0].element_size()
    bytes_append_step = B * H * (2 * 128 * in_b + 144) + 4 * B
    bytes_decode = B * ctx * H * 144 + B * pages_per_seq * 4 + B * Hq * 128 * in_b + B * Hq * 128 * 4
    bytes_step = bytes_append_step + bytes_decode

    # the step as one library call: nvfp4_paged_decode_step appends the new
    # token inside the decode kernel, or launches the append kernel first, by shape
    kn_f = [newk[l].reshape(B, 1, H, 128) for l in range(L)]
    vn_f = [newv[l].reshape(B, 1, H, 128) for l in range(L)]
    q_f = [qs[l].reshape(B, 1, Hq, 128) for l in range(L)]
    out_f = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device=dev)

    def lib_step(i):
        l = i % L
        nk.paged_decode_step(layers[l], kn_f[l], vn_f[l], q_f[l], tables[l], seq_lens, ctx, sm, out=out_f,
                             workspace=workspace)

    def app_call(i):
        l = i % L
        nk.quantize_append(layers[l], newk[l], newv[l], slots_new[l])

    def dec_call(i):
        l = i % L
        nk.paged_decode_attn(layers[l], qs[l], tables[l], seq_lens, ctx, sm, out=out, workspace=workspace)

    def two_step(i):  # the same step as two explicit calls
        app_call(i)
        dec_call(i)

    for l in range(L):  # set-up: touch every layer once
        lib_step(l)
    torch.cuda.synchronize()

    # ---- warm-up, then the timed region: windows of exactly --steps step calls
    for i in range(args.warmup):
        lib_step(i)
    torch.cuda.synchronize()
    wall, ev = sync_windows(lib_step, args.steps, STEP_WINDOWS)
    per_step = float(np.median(wall))
    wall_two, _ = sync_windows(two_step, args.steps, 3)
    print("[bench] step timed", file=sys.stderr, flush=True)

    # ---- kernels back to back (the rooflines' per-launch durations)
    dec_spread = []
    dec_avg_s = back_to_back(stream, args.steps, dec_call, spread_out=dec_spread)
    step_s = back_to_back(stream, args.steps, lib_step)
    app_s = back_to_back(stream, args.steps, app_call)
    achieved = bytes_decode / dec_avg_s / 1e9
    b2b_layers = list(range(min(L, 2)))
    chunks = {}

    def chunk_set(fill):
        if fill not in chunks:
            chunks[fill] = [first_chunk(wl, [fill] * B, l, bts[l], dev) for l in b2b_layers]
        return chunks[fill]
    app_us, app_gbs, app_b = append_b2b(stream, args.steps, chunk_set(ctx - 1), [layers[l] for l in b2b_layers],
                                        nk.quantize_append, 144)
    print("[bench] decode and bulk append timed back to back", file=sys.stderr, flush=True)
    app_total_b = float(sum(append_bytes))
    app_total_s = float(sum(append_ms)) / 1e3

    result = {
        "value": round(bytes_step / per_step / 1e9, 2),
        "ms_per_step": round(per_step * 1e3, 5),
        "ms_per_step_windows": spread(wall, 1e3, 5),
        "ms_per_step_events_windows": spread(ev, 1e3, 5),
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": 128,
                   "context": ctx, "page_size": 16, "layers_rotated": L,
                   "step": "nvfp4_paged_decode_step: append 1 token/seq + decode attention, one layer"},
        "pct_of_peak": round(100 * bytes_step / per_step / 1e9 / PEAK_HBM_GBS, 2),
        "step_us_b2b": round(step_s * 1e6, 3),
        "step_append_then_decode": {"ms_per_step": round(float(np.median(wall_two)) * 1e3, 5),
                                    "value": round(bytes_step / float(np.median(wall_two)) / 1e9, 2)},
        "decode_attn_gbs_events": round(achieved, 2),
        "decode_attn_us": round(dec_avg_s * 1e6, 3),
        "decode_attn_us_windows": spread(dec_spread, 1e6),
        "append_step_us": round(app_s * 1e6, 3),
        "quantize_append_bulk_gbs": round(app_gbs, 2),
        "quantize_append_bulk_us": round(app_us, 2),
        "quantize_append_bulk_chunk_tokens": int(chunk_set(ctx - 1)[0][0].shape[0]),
        "append_roofline": {"bound": "hbm", "achieved": round(app_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(app_gbs / PEAK_HBM_GBS, 4),
                            "traffic": read_traffic(APPEND_SOURCES, wl.name, "append_hbm_bytes_per_call",
                                                    "append_source_sha256_16"),
                            "kernel": "nvfp4_kv_quantize_append (bulk, one chunk per call)",
                            "algorithmic_bytes_per_call": int(app_b)},
        "quantize_append_bulk_gbs_single_call": round(app_total_b / app_total_s / 1e9, 2),
        "quantize_append_bulk_tokens": int(B * (ctx - 1) * L),
        "bytes_per_step": int(bytes_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(DECODE_SOURCES, wl.name),
                     "kernel": "nvfp4_paged_decode_attn (decode_kernel)",
                     "algorithmic_bytes_per_call": int(bytes_decode)},
    }
    if args.no_extras:
        return result

    # ---- multi-token decode: T = 16 / G new tokens per sequence (the last T of
    # the context) fill the 16-row MFMA tile in the same pass over the cache
    T_m = 16 // (Hq // H)
    if T_m >= 2:
        q_m = [synth.queries(B * T_m, Hq, wl.in_dtype, dev, 6, l).reshape(B, T_m, Hq, 128) for l in range(L)]
        out_m = torch.empty((B, T_m, Hq, 128), dtype=torch.float32, device=dev)
        ws_m = torch.zeros(nk.decode_multi_workspace_bytes(B, T_m, Hq, H, ctx), dtype=torch.uint8, device=dev)

        def multi_call(i):
            l = i % L
            nk.paged_decode_attn_multi(layers[l], q_m[l], tables[l], seq_lens, ctx, sm, out=out_m, workspace=ws_m)
        multi_s = back_to_back(stream, args.steps, multi_call)
        b_multi = B * ctx * H * 144 + B * pages_per_seq * 4 + B * T_m * Hq * 128 * (in_b + 4)
        result["decode_multi_token"] = {"q_per_seq": T_m, "us": round(multi_s * 1e6, 3),
                                        "gbs": round(b_multi / multi_s / 1e9, 2),
                                        "query_tokens_per_s": round(B * T_m / multi_s, 1),
                                        "time_vs_one_token": round(multi_s / dec_avg_s, 4)}

    # ---- FP8 workspace dequant on the same cache: up to 8 sequences' full prefixes (extend path)
    n_ext = min(8, B)
    prefix = torch.full((n_ext,), ctx, dtype=torch.int32, device=dev)
    offs = torch.arange(0, (n_ext + 1) * ctx, ctx, dtype=torch.int32, device=dev)
    ws_k = torch.empty((n_ext * ctx, H, 128), dtype=torch.uint8, device=dev)
    ws_v = torch.empty_like(ws_k)
    tabs = [tables[l][:n_ext].contiguous() for l in range(L)]

    def ws_call(i):
        l = i % L
        nk.dequant_to_fp8_workspace(layers[l], tabs[l], prefix, offs, ctx, 6 * layers[l].k_global,
                                    6 * layers[l].v_global, ws_k, ws_v)
    ws_s = back_to_back(stream, max(4, args.steps // 2), ws_call)
    ws_bytes_alg = n_ext * ctx * H * (144 + 256) + n_ext * pages_per_seq * 4
    result["fp8_workspace_gbs"] = round(ws_bytes_alg / ws_s / 1e9, 2)
    result["fp8_workspace_us"] = round(ws_s * 1e6, 3)
    result["fp8_workspace_tokens"] = int(n_ext * ctx)
    del ws_k, ws_v

    # ---- MXFP4, the format the pages compare NVFP4 against (E8M0 scale per 32
    # values, 17/32 byte per value): the same tokens, slots and queries in
    # MXFP4 layers; bulk append and decode timed as above
    mx_layers, mx_app_ms, mx_app_b = [], [], []
    for l in range(L_x):
        fl = build_layer(wl, [ctx] * B, [ctx] * B, l, dev, timed=True, mx=True)
        mx_layers.append(fl.layer)
        mx_app_ms += fl.append_ms
        mx_app_b += fl.append_bytes
    print("[bench] MXFP4 layers filled", file=sys.stderr, flush=True)

    def mx_call(i):
        l = i % L_x
        nk.mx_paged_decode_attn(mx_layers[l], qs[l], tables[l], seq_lens, ctx, sm, out=out, workspace=workspace)
    for i in range(max(args.warmup, L_x)):
        mx_call(i)
    mx_s = back_to_back(stream, args.steps, mx_call)
    mx_app_us, mx_app_gbs, _ = append_b2b(stream, args.steps, chunk_set(ctx), [mx_layers[l] for l in b2b_layers],
                                          nk.mx_quantize_append, 136)
    bytes_mx = B * ctx * H * 136 + B * pages_per_seq * 4 + B * Hq * 128 * in_b + B * Hq * 128 * 4
    result["mxfp4"] = {"layers_rotated": L_x, "decode_us": round(mx_s * 1e6, 3),
                       "decode_gbs": round(bytes_mx / mx_s / 1e9, 2),
                       "decode_frac": round(bytes_mx / mx_s / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes_per_call": int(bytes_mx),
                       "decode_time_vs_nvfp4": round(mx_s / dec_avg_s, 4),
                       "quantize_append_bulk_gbs": round(mx_app_gbs, 2),
                       "quantize_append_bulk_us": round(mx_app_us, 2),
                       "quantize_append_bulk_gbs_single_call":
                           round(float(sum(mx_app_b)) / (float(sum(mx_app_ms)) / 1e3) / 1e9, 2)}
    del mx_layers
    # ---- Hadamard-rotated K (both formats): the same tokens stored with K
    # rotated by the append kernel; the decode rotates Q in its prologue and
    # takes Q as a hi + lo pair (twice the QK^T MFMAs)
    hadamard = {}
    for fmt, mx in (("nvfp4", False), ("mxfp4", True)):
        rot_layers, rot_ms, rot_b = [], [], []
        for l in range(L_x):
            fl = build_layer(wl, [ctx] * B, [ctx] * B, l, dev, timed=True, mx=mx, hadamard=True)
            rot_layers.append(fl.layer)
            rot_ms += fl.append_ms
            rot_b += fl.append_bytes
        dec = nk.mx_paged_decode_attn if mx else nk.paged_decode_attn

        def rot_call(i):
            l = i % L_x
            dec(rot_layers[l], qs[l], tables[l], seq_lens, ctx, sm, out=out, workspace=workspace, hadamard=True)
        for i in range(max(args.warmup, L_x)):
            rot_call(i)
        rot_s = back_to_back(stream, args.steps, rot_call)
        rot_app_us, rot_app_gbs, _ = append_b2b(stream, args.steps, chunk_set(ctx),
                                                [rot_layers[l] for l in b2b_layers],
                                                nk.mx_quantize_append if mx else nk.quantize_append,
                                                136 if mx else 144, hadamard=True)
        b_rot = bytes_mx if mx else bytes_decode
        plain_s = mx_s if mx else dec_avg_s
        hadamard[fmt] = {"layers_rotated": L_x, "decode_us": round(rot_s * 1e6, 3),
                         "decode_gbs": round(b_rot / rot_s / 1e9, 2),
                         "decode_time_vs_unrotated": round(rot_s / plain_s, 4),
                         "quantize_append_bulk_gbs": round(rot_app_gbs, 2),
                         "quantize_append_bulk_us": round(rot_app_us, 2),
                         "quantize_append_bulk_gbs_single_call":
                             round(float(sum(rot_b)) / (float(sum(rot_ms)) / 1e3) / 1e9, 2)}
        del rot_layers
    result["hadamard_k"] = hadamard
    print("[bench] Hadamard-rotated layers timed", file=sys.stderr, flush=True)
    result["sparse_mla"] = bench_mla(args, dev)
    return result


def bench_mla(args, dev):
    """Sparse MLA over the NVFP4 latent cache at a DeepSeek-V3.2-class decode
    shape (128 query tokens, one per sequence; latent rows of 512 + 64 values;
    top-2048 of each sequence's 32,768 cached tokens; 64-token pages in random
    order; 4 layer caches rotated, so the touched rows exceed the 256 MB
    Infinity Cache): bulk quantize-append, and the sparse decode at 128 and at
    16 heads per query token (the second: one tensor-parallel shard of 8)."""
    import torch

    import nvfp4_quantized_paged_kv_amd as nk
    from synthetic import synth
    from synthetic.workloads import MLA_CHUNK, MLA_OUTLIERS, MLA_SHAPE, build_mla_layer, mla_slots

    sh = MLA_SHAPE
    T, ctx, topk, page, L = sh["T"], sh["ctx"], sh["topk"], sh["page"], sh["layers"]
    n_slots = T * ctx
    stream = torch.cuda.current_stream()
    filled = [build_mla_layer(l, dev, timed=True) for l in range(L)]
    print("[bench] sparse-MLA layers filled", file=sys.stderr, flush=True)
    sm = 1 / math.sqrt(192)
    res = {"workload": f"sparse MLA decode: {T} query tokens, 576/512 latent rows, top-{topk} of {ctx}-token "
                       f"contexts, {page}-token pages, {L} rotated layers"}
    # bulk append: the first fill chunk re-appended into its own slots, back to back, alternating over two layers
    rows_b = [synth.mla_rows(MLA_CHUNK, MLA_OUTLIERS, torch.bfloat16, dev, 60, l, 0) for l in range(2)]
    tok = torch.arange(0, MLA_CHUNK, device=dev)
    slots_b = [mla_slots(filled[l].block_table, tok, ctx, page) for l in range(2)]
    app_s = back_to_back(stream, args.steps, lambda i: nk.mla_quantize_append(filled[i % 2].layer, rows_b[i % 2],
                                                                              slots_b[i % 2]))
    per_tok = 576 * 2 + 324 + 4
    app_gbs = MLA_CHUNK * per_tok / app_s / 1e9
    res["append_us"] = round(app_s * 1e6, 2)
    res["append_roofline"] = {"bound": "hbm", "achieved": round(app_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(app_gbs / PEAK_HBM_GBS, 4),
                              "algorithmic_bytes_per_call": int(MLA_CHUNK * per_tok), "tokens_per_call": MLA_CHUNK}
    app_ms = [m for f in filled for m in f.append_ms]
    res["append_gbs_single_call"] = round(n_slots * L * per_tok / (sum(app_ms) / 1e3) / 1e9, 2)
    for Hq in (128, 16):
        qs = [synth.mla_queries(T, Hq, torch.bfloat16, dev, 63, l) for l in range(L)]
        out = torch.empty((T, Hq, 512), dtype=torch.float32, device=dev)
        ws = torch.empty(max(nk.mla_sparse_decode_workspace_bytes(T, Hq, topk), 256), dtype=torch.uint8, device=dev)

        def call(i):
            l = i % L
            nk.mla_sparse_decode(filled[l].layer, qs[l], filled[l].indices, sm, out=out, workspace=ws)
        for i in range(max(args.warmup, L)):
            call(i)
        spread_s = []
        dec_s = back_to_back(stream, args.steps, call, spread_out=spread_s)
        flops = T * Hq * topk * 2 * (576 + 512)
        byts = T * topk * (324 + 4) + T * Hq * (576 * 2 + 512 * 4)
        tf = flops / dec_s / 1e12
        gbs = byts / dec_s / 1e9
        res[f"decode_heads{Hq}"] = {
            "us": round(dec_s * 1e6, 3), "us_windows": spread(spread_s, 1e6),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_F16_TFLOPS, 4), "flops_per_call": int(flops)},
            "hbm": {"achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_call": int(byts)},
            "workspace_bytes": int(ws.numel())}
    print("[bench] sparse-MLA decode timed", file=sys.stderr, flush=True)
    return res


def calibration_kernel():
    """A plain elementwise kernel of known traffic: y = x + 1 over 2^28 float32."""
    import torch

    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.add(x, 1.0, out=y)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    global SUSTAIN_S
    if args.sustain is not None:
        SUSTAIN_S = max(0.0, args.sustain)

    import torch

    import nvfp4_quantized_paged_kv_amd  # noqa: F401  (fails loudly if the HIP library is not built)
    from synthetic import synth

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    res = bench_mixed(args, wl, dev) if wl.lens else bench_uniform(args, wl, dev)
    in_dtype = "bf16" if wl.in_dtype == torch.bfloat16 else "f32"
    result = {"metric": METRIC, "value": res.pop("value"), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None,
              "dtype": f"nvfp4 cache; {in_dtype} in; f16 MFMA, fp32 accumulate",
              "data": "synthetic (seeded torch generators)",
              "sustain_s": SUSTAIN_S}
    result.update(res)
    if args.calibrate:
        calibration_kernel()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
