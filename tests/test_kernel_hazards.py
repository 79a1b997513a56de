"""Compile-time check of the attention kernel's MFMA operand hazards (CPU only).

The kernel issues its MFMAs through inline asm, so the compiler's hazard recognizer does not
know they are MFMAs.  The wait states an MFMA needs after a VALU instruction writes one of
its source VGPRs therefore rest on the instruction schedule: the P operand is produced by
VALU code, and the register allocator may insert copies of it.  This test compiles the
kernel to gfx950 assembly and requires at least 4 other instructions between any VALU write
of a VGPR and an MFMA that reads it (the ISA asks for 2 wait states here).  The wait states
the asm itself provides (after the last S^T MFMA, before the first O^T MFMA, after the tile
loop) are written into the asm statements and need no check.

The O^T accumulators stay in AGPRs across the whole tile loop: the third test requires that the
compiler moves no accumulator through VGPRs (v_accvgpr_read / v_accvgpr_write) between the first
and the last MFMA of the kernel, since an AGPR written that way just before an asm MFMA that
accumulates into it would need wait states the compiler does not know to insert.

The tile copies (direct-to-LDS loads) also live in inline asm, each writing M0 right before
its load.  The second test requires that nothing else in the kernel reads or writes M0, so
that a compiler-generated M0 value can never be live across one of those statements.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mla_tree_verify_absorb_amd", "csrc", "verify_attn_bf16.hip")
MIN_BETWEEN = 4


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernel_lines(asm, name):
    out, inside = [], False
    for raw in asm.splitlines():
        line = raw.strip()
        if re.match(rf"^_Z\S*{name}\S*:", line):
            inside = True
            continue
        if inside:
            if line.startswith("s_endpgm"):
                break
            if line and not line.startswith((";", ".")):
                out.append(line)
    return out


_ASM = {}


def _kernel_asm(tmp_path_factory):
    if "lines" not in _ASM:
        asm_path = tmp_path_factory.mktemp("asm") / "verify_attn_bf16.s"
        subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", SRC,
                        "-o", str(asm_path)], check=True, capture_output=True)
        _ASM["lines"] = _kernel_lines(asm_path.read_text(), "verify_attn_bf16_kernel")
    return _ASM["lines"]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_m0_is_written_only_by_the_tile_copies(tmp_path_factory):
    lines = _kernel_asm(tmp_path_factory)
    uses = [(i, l) for i, l in enumerate(lines) if re.search(r"\bm0\b", l)]
    assert uses, "kernel not found in the assembly"
    for i, line in uses:
        # s_mov_b32 m0, <scalar register>; v_xad_u32 / v_add_u32 (the lane address); global_load_lds_dwordx4
        assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi|ttmp\d+)$", line), line
        assert lines[i + 1].startswith(("v_xad_u32", "v_add_u32")), lines[i + 1]
        assert lines[i + 2].startswith("global_load_lds_dwordx4"), lines[i + 2]
    assert len(uses) == sum(l.startswith("global_load_lds_dwordx4") for l in lines)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_no_accumulator_moves_inside_the_mfma_region(tmp_path_factory):
    lines = _kernel_asm(tmp_path_factory)
    mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
    assert len(mf) >= 68, "kernel not found in the assembly"
    moves = [l for l in lines[mf[0]:mf[-1]] if l.startswith(("v_accvgpr_read", "v_accvgpr_write", "v_accvgpr_mov"))]
    assert not moves, f"{len(moves)} accumulator moves between MFMAs, e.g. {moves[:3]}"


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_no_valu_write_close_before_an_mfma_source(tmp_path_factory):
    lines = _kernel_asm(tmp_path_factory)
    assert sum(l.startswith("v_mfma") for l in lines) >= 68, "kernel not found in the assembly"
    close = []
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        srcs = set()
        for op in line.split(None, 1)[1].split(",")[1:]:
            srcs |= _vgprs(op.strip())
        for back in range(1, MIN_BETWEEN + 1):
            j = i - back
            if j < 0:
                break
            prev = lines[j]
            if prev.startswith("v_") and not prev.startswith(("v_mfma", "v_accvgpr")) and " " in prev:
                dst = prev.split(None, 1)[1].split(",")[0].strip()
                if _vgprs(dst) & srcs:
                    close.append((back - 1, prev, line))
    assert not close, f"VALU writes too close before MFMA source reads: {close[:5]}"
