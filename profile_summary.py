"""Summarise rocprofv3 CSV output into the text summaries kept under profiles/.

usage:
  python profile_summary.py trace <dir> <title> <command>
      per-kernel dispatch durations (kernel trace), grouped by kernel and launch shape
  python profile_summary.py pmc <fetch_dir> <write_dir> <title> <command>
      FETCH_SIZE / WRITE_SIZE per dispatch, scaled by the plain elementwise add
      that `bench.py --calibrate` runs (2^28 float32 read and written), and the
      HBM bytes per call of the decode and bulk-append kernels, with the hash of
      the sources they were taken on (bench.py reports `traffic` only while it matches)
  python profile_summary.py counters <dir> <title> <command>
      every collected counter per dispatch (mean over dispatches of one kernel and shape)

The summary is printed on stdout.  Only kernels of libnvfp4kv (and the
calibration kernel) are listed.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "nvfp4_quantized_paged_kv_amd", "csrc")
DECODE_FILES = ["decode_attn.hip", "nvfp4_kv_internal.h", "nvfp4_device.h", "nvfp4_quant_device.h"]
APPEND_FILES = ["quant_append.hip", "nvfp4_kv_internal.h", "nvfp4_device.h", "nvfp4_quant_device.h"]


def src_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def rows(d, suffix):
    out = []
    for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def field(r, *names):
    for n in names:
        if n in r and r[n] != "":
            return r[n]
    return None


def short(name: str) -> str:
    """Readable kernel name: the decode instance flags spelled out."""
    m = re.search(r"(\w+_kernel)(<[^()]*>)?", name)
    if not m:
        return name.split("(")[0][:48]
    k, args = m.group(1), m.group(2)
    if not args:
        return k
    a = [x.strip() for x in args[1:-1].split(",")]
    if k == "decode_kernel" and len(a) == 6:
        b = [x == "true" for x in a]
        tags = ["f32 q" if b[0] else "bf16 q"]
        if not b[1]:
            tags.append("tile rsrc")
        for i, t in ((2, "multi"), (3, "+append"), (4, "mxfp4"), (5, "hadamard")):
            if b[i]:
                tags.append(t)
        return f"{k}<{','.join(tags)}>"
    tags = []
    if a and a[0] == "float":
        tags.append("f32 in")
    if a and a[-1] == "true":
        tags.append("hadamard K")
    rest = [x for x in a if x not in ("float", "true", "false", "unsigned short", "__bf16")]
    tags += rest
    return f"{k}<{','.join(tags)}>" if tags else k


def ours(name: str) -> bool:
    return "nvfp4kv" in name


def header(kind, title, cmd):
    print(f"# rocprofv3 {kind}: {title}")
    print("# MI355X (gfx950), one GPU; run from the repository root with TMPDIR=/tmp:")
    print(f"#   {cmd}")
    print("# summarised by: python profile_summary.py " + " ".join(sys.argv[1:2]) + " <output dirs> <title> <command>")


def trace(d, title, cmd):
    groups, order = {}, []
    for r in sorted(rows(d, "kernel_trace.csv"), key=lambda r: int(field(r, "Start_Timestamp"))):
        name = field(r, "Kernel_Name")
        if not ours(name):
            continue
        grid = (f"{field(r, 'Grid_Size_X', 'Grid_Size')}x{field(r, 'Grid_Size_Y') or 1}x"
                f"{field(r, 'Grid_Size_Z') or 1}/{field(r, 'Workgroup_Size_X', 'Workgroup_Size')}")
        us = (int(field(r, "End_Timestamp")) - int(field(r, "Start_Timestamp"))) / 1e3
        key = (short(name), grid)
        if key not in groups:
            groups[key] = []
            order.append(key)
        groups[key].append(us)
    header("kernel-trace summary", title, cmd)
    print("# durations in microseconds per dispatch, grouped by kernel and launch shape (grid threads x y z / "
          "workgroup); tiny shapes are the bench's one-call warm-up of each kernel")
    print(f"{'kernel':48s} {'grid/workgroup':24s} {'calls':>6s} {'median_us':>10s} {'avg_us':>10s} "
          f"{'min_us':>10s} {'max_us':>10s}")
    for key in order:
        v = groups[key]
        print(f"{key[0]:48s} {key[1]:24s} {len(v):6d} {statistics.median(v):10.2f} {statistics.mean(v):10.2f} "
              f"{min(v):10.2f} {max(v):10.2f}")


def counter_means(d, counter=None):
    """{(short name, grid, full name, counter): mean value per dispatch}, dispatch counts, order."""
    acc, order = {}, []
    for r in rows(d, "counter_collection.csv"):
        c = field(r, "Counter_Name")
        if counter is not None and c != counter:
            continue
        name = field(r, "Kernel_Name")
        key = (short(name), int(float(field(r, "Grid_Size"))), name, c)
        disp = field(r, "Dispatch_Id", "Correlation_Id")
        acc.setdefault(key, {})
        acc[key][disp] = acc[key].get(disp, 0.0) + float(field(r, "Counter_Value"))
        if key not in order:
            order.append(key)
    return ({k: statistics.mean(v.values()) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}, order)


def pmc(fd, wd, title, cmd):
    fetch, nf, order = counter_means(fd, "FETCH_SIZE")
    write, _, _ = counter_means(wd, "WRITE_SIZE")
    fetch = {k[:3]: v for k, v in fetch.items()}
    nf = {k[:3]: v for k, v in nf.items()}
    write = {k[:3]: v for k, v in write.items()}
    order = [k[:3] for k in order]
    cal = [k for k in fetch if "elementwise" in k[2] and "add" in k[2].lower() and "float" in k[2]]
    cal = max(cal, key=lambda k: k[1])
    kib = (1 << 28) * 4 / 1024
    fs, ws = kib / fetch[cal], kib / write[cal]
    header("HBM byte counters", title, cmd)
    print("# FETCH_SIZE / WRITE_SIZE: KiB per dispatch, mean over dispatches of the same kernel and grid size;")
    print("# each counter in its own profiled run (same command).")
    print(f"# calibration: the plain elementwise add of the same runs (2^28 float32 read, 2^28 written = "
          f"{kib:.0f} KiB each way)")
    print(f"#   reads FETCH_SIZE {fetch[cal]:.1f} KiB and WRITE_SIZE {write[cal]:.1f} KiB -> scales {fs:.3f} and "
          f"{ws:.3f}")
    print(f"fetch_scale: {fs:.4f}")
    print(f"write_scale: {ws:.4f}")
    dec = app = None
    for k in order:
        if k == cal or k not in write or not ours(k[2]):
            continue
        hb = (fetch[k] * fs + write[k] * ws) * 1024
        print(f"{k[0]} grid {k[1]}: dispatches {nf[k]}, FETCH_SIZE {fetch[k]:.1f} KiB, WRITE_SIZE {write[k]:.1f} KiB, "
              f"HBM bytes {hb:.0f}")
        if k[0] == "decode_kernel<bf16 q>" and (dec is None or k[1] > dec[0][1]):
            dec = (k, hb)
        if k[0] == "quantize_append_kernel" and (app is None or k[1] > app[0][1]):
            app = (k, hb)
    if dec is not None:
        print(f"# decode (decode_kernel<bf16 q>, grid {dec[0][1]}: one call over the whole batch)")
        print(f"hbm_bytes_per_call: {dec[1]:.0f}")
        print("# kernel_source_sha256_16: SHA-256 of " + ", ".join(DECODE_FILES) + ", concatenated")
        print(f"kernel_source_sha256_16: {src_hash(DECODE_FILES)}")
    if app is not None:
        print(f"# bulk quantize-append (quantize_append_kernel, grid {app[0][1]}: one fill chunk per call)")
        print(f"append_hbm_bytes_per_call: {app[1]:.0f}")
        print("# append_source_sha256_16: SHA-256 of " + ", ".join(APPEND_FILES) + ", concatenated")
        print(f"append_source_sha256_16: {src_hash(APPEND_FILES)}")


def counters(d, title, cmd):
    vals, n, order = counter_means(d)
    header("counter summary", title, cmd)
    print("# mean counter value per dispatch, over the dispatches of one kernel and grid size")
    for k in order:
        if not ours(k[2]):
            continue
        print(f"{k[0]} grid {k[1]}: {k[3]} = {vals[k]:.1f} (dispatches {n[k]})")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4])
    elif mode == "pmc":
        pmc(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif mode == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        sys.exit(__doc__)
