"""CPU: the library is never used stale.  The build stamps a digest of its sources into libddtree.so; the
binding compares it with the sources beside it, refuses a mismatch, and the test session rebuilds."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "mla_tree_verify_absorb_amd"

PROBE = """
import sys
sys.path.insert(0, {root!r})
from {pkg} import _lib
print("current", _lib.is_current())
try:
    _lib.lib()
    print("loaded")
except RuntimeError as e:
    print("refused:", e)
"""


def run_probe(root):
    out = subprocess.run([sys.executable, "-c", PROBE.format(root=str(root), pkg=PKG)], capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    return out.stdout


def test_touched_source_is_refused_until_rebuilt(tmp_path):
    from mla_tree_verify_absorb_amd import _lib
    assert _lib.is_current()                      # the session fixture built or checked it
    shutil.copytree(os.path.join(ROOT, PKG), tmp_path / PKG, ignore=shutil.ignore_patterns("_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    assert "current True" in run_probe(tmp_path) and "loaded" in run_probe(tmp_path)
    with open(tmp_path / PKG / "csrc" / "accept.hip", "a") as f:
        f.write("\n// an edit after the build\n")
    out = run_probe(tmp_path)
    assert "current False" in out and "refused:" in out and "built from other sources" in out
