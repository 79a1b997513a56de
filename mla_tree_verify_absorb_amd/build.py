"""Build libddtree.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m mla_tree_verify_absorb_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

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
# Per-file device flags (none at present).
FILE_FLAGS = {}
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code (the compiler
# would otherwise form them from scalar float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


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


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library; returns its path."""
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        _run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
              "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *FILE_FLAGS.get(src, []),
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB_PATH + ".tmp"], verbose)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
