"""Build the gfx950 shared library ``libnvfp4kv.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled and floating-point contraction off (the quantizer's exact rounding
relies on products being rounded where the source writes them).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnvfp4kv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.cpp", "quant_append.hip", "decode_attn.hip", "decode_noalloc.hip", "dequant_ws.hip", "fp8_extend.hip",
           "mxfp4_append.hip", "mla_decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fvisibility=hidden",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around the
    # (rarely taken) softmax rescale in the decode loop
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
