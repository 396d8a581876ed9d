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
           "extend_f8.hip", "mxfp4_append.hip", "mla_decode.hip"]
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


# Host code (the C ABI's argument checks, launch set-up) under AddressSanitizer
# and UBSan; device code is compiled as always.  The sanitizer runtime is not
# linked: the process that loads this build preloads it.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB_PATH) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
