"""Build libddtree.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m mla_tree_verify_absorb_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libddtree.so")
SOURCES = ["ddtree_api.hip", "build_mask.hip", "accept.hip", "verify_attn_f32.hip", "verify_attn_bf16.hip",
           "compact_kv.hip", "build_tree.hip", "rope_tree.hip"]
# Achievable-rate probes (bench context only), a library of their own.
RATES_LIB_PATH = os.path.join(PKG_DIR, "libddtree_rates.so")
RATES_SOURCES = ["rates.hip"]
# Per-file device flags (none at present).
FILE_FLAGS = {}
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code (the compiler
# would otherwise form them from scalar float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def source_files():
    """Every file the libraries are built from: the HIP sources, their headers and the public headers."""
    hdrs = sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
    return ([os.path.join(CSRC, f) for f in SOURCES + RATES_SOURCES] + [os.path.join(CSRC, f) for f in hdrs] +
            [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
             if f.endswith(".h")])


def source_digest() -> str:
    """sha256 (first 16 hex digits) of the library's sources and compile flags.  The build stamps it into
    the library (ddtree_build_digest); loading compares it with the sources present, so a library built
    from other sources is never used by mistake."""
    h = hashlib.sha256()
    h.update(" ".join([ARCH, *DEVICE_FLAGS]).encode())
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)


def _build_one(sources, lib_path, digest, verbose):
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    for src in sources:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        _run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
              "-I", os.path.join(ROOT, "include"), f'-DDDTREE_SOURCE_DIGEST="{digest}"', *DEVICE_FLAGS,
              *FILE_FLAGS.get(src, []),
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib_path + ".tmp"], verbose)
    os.replace(lib_path + ".tmp", lib_path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared libraries (the verify library and the rate probes);
    returns the verify library's path."""
    digest = source_digest()
    _build_one(RATES_SOURCES, RATES_LIB_PATH, digest, verbose)
    _build_one(SOURCES, LIB_PATH, digest, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
