"""Host code under AddressSanitizer and UBSan, on the CPU.

The oracle (with all its pins) and the C ABI's host side (every argument
check and status path of test_abi.py) are built once more with clang's
address and undefined-behaviour sanitizers -- the library's device code is
compiled as always -- and the same tests run against those builds in a child
process that preloads the sanitizer runtime.  A sanitizer report fails the
child, and the child's failure fails the test.  The builds are cached under
_build/ by a hash of their sources.
"""
import glob
import hashlib
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD_DIR = os.path.join(ROOT, "_build")
LLVM = "/opt/rocm/lib/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
ORACLE_TESTS = ["tests/test_oracle_formats.py", "tests/test_oracle_pages.py", "tests/test_oracle_attention.py",
                "tests/test_oracle_extend.py", "tests/test_oracle_extend_fp8.py", "tests/test_oracle_mx.py", "tests/test_oracle_hadamard.py",
                "tests/test_oracle_mla.py"]
ABI_TESTS = ["tests/test_abi.py"]


def _runtime():
    found = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def _hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _cached(out: str, sources, make):
    """Build `out` with make(out) unless its recorded source hash is current."""
    stamp = out + ".sha"
    want = _hash(sources)
    if not (os.path.exists(out) and os.path.exists(stamp) and open(stamp).read() == want):
        make(out)
        with open(stamp, "w") as f:
            f.write(want)
    return out


@pytest.fixture(scope="module")
def sanitized_builds():
    rt = _runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("no clang sanitizer runtime in this toolchain")
    os.makedirs(BUILD_DIR, exist_ok=True)
    import oracle

    spec = importlib.util.spec_from_file_location(
        "_nvfp4kv_build", os.path.join(ROOT, "nvfp4_quantized_paged_kv_amd", "build.py"))
    hip_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hip_build)
    hip_sources = [os.path.join(hip_build.CSRC, s) for s in hip_build.SOURCES]
    hip_sources += sorted(glob.glob(os.path.join(hip_build.CSRC, "*.h")))
    hip_sources += [os.path.join(ROOT, "include", "nvfp4_kv.h")]
    lib = _cached(os.path.join(BUILD_DIR, "libnvfp4kv_san.so"), hip_sources,
                  lambda out: hip_build.build(sanitize=True, out=out))
    orc = _cached(os.path.join(BUILD_DIR, "libnvfp4_oracle_san.so"), [os.path.join(ROOT, "oracle", "nvfp4_oracle.c")],
                  lambda out: oracle.build_sanitized(out, CLANG))
    return rt, lib, orc


def _run_under_sanitizers(builds, tests):
    rt, lib, orc = builds
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",  # the interpreter keeps its objects to the end
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "NVFP4KV_LIBRARY": lib,
        "NVFP4_ORACLE_LIBRARY": orc,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = res.stdout + res.stderr
    reports = [ln for ln in out.splitlines() if "runtime error:" in ln or "ERROR: AddressSanitizer" in ln]
    assert res.returncode == 0 and not reports, "\n".join(reports) + "\n" + out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(sanitized_builds):
    out = _run_under_sanitizers(sanitized_builds, ORACLE_TESTS)
    assert " passed" in out


def test_abi_checks_under_asan_and_ubsan(sanitized_builds):
    out = _run_under_sanitizers(sanitized_builds, ABI_TESTS)
    assert " passed" in out
