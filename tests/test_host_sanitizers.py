"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is compiled as for libddtree.so, with the sanitizers applied to the host pass only
(`-Xarch_host`; the gfx950 device code is unchanged and never runs here), and linked into a shared
library that tests/sanitize_host_abi.c drives: each entry point's argument checks, the workspace
and split queries over shapes at the limits of their integer types, and overlap checks of buffers
at the top of the address space.  No call passes validation, so no GPU is needed.  A sanitizer
report (a heap or stack overrun, a signed overflow, a shift out of range, ...) fails the test with
the report.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mla_tree_verify_absorb_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize_host_abi.c")
CLANG = "/opt/rocm/llvm/bin/clang"
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _have_toolchain():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(CLANG)


@pytest.mark.skipif(not _have_toolchain(), reason="hipcc / clang not available")
def test_host_code_is_sanitizer_clean(tmp_path):
    host_flags = [f for flag in SANITIZE for f in ("-Xarch_host", flag)]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-I", os.path.join(ROOT, "include"), *B.DEVICE_FLAGS, *host_flags,
               "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as pool:
        objs = list(pool.map(compile_one, B.SOURCES))
    lib = str(tmp_path / "libddtree_sanitized.so")
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "sanitize_host_abi")
    r = subprocess.run([CLANG, "-std=c99", "-O1", "-g", *SANITIZE, "-I", os.path.join(ROOT, "include"), DRIVER,
                        lib, f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all statuses as expected" in r.stdout
