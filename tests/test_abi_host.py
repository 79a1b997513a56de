"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects invalid calls on the host before any HIP call is made."""
import ctypes
import os
import re

import pytest

import mla_tree_verify_absorb_amd as dd
from mla_tree_verify_absorb_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddtree.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = dd.DDTREE_OK, dd.DDTREE_ERR_INVALID_ARG, dd.DDTREE_ERR_UNSUPPORTED, \
    dd.DDTREE_ERR_WORKSPACE
F32, BF16 = dd.DDTREE_F32, dd.DDTREE_BF16
A = 0x10000      # fake, 16-byte aligned "device" addresses: never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtree_\w+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("ddtree_build_mask", "ddtree_verify_attn", "ddtree_greedy_accept"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = dd.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding's signature table covers all of them
    assert set(declared_functions()) == set(_lib._SIGNATURES)


def test_rates_library_exports_its_header():
    """The achievable-rate probes (bench context, not the verify path) live in their own library."""
    from mla_tree_verify_absorb_amd import rates
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ddtree_rates.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ddtree_rates_\w+)\s*\(", text)))
    assert names and set(names) == set(rates.SIGNATURES)
    lib = rates.lib()
    assert all(hasattr(lib, n) for n in names)
    assert lib.ddtree_rates_mfma_loop_flops(512, 10) == 512 * 4 * 10 * 4 * 32768
    assert lib.ddtree_rates_mfma_loop(0, 10, A, None) == -1                 # rejected on the host
    assert lib.ddtree_rates_stream_read(A, 100, 8, A, None) == -1           # not a multiple of 16


def test_status_strings():
    assert dd.ddtree_status_string(OK) == "DDTREE_OK"
    assert dd.ddtree_status_string(INVALID) == "DDTREE_ERR_INVALID_ARG"
    assert dd.ddtree_status_string(UNSUPPORTED) == "DDTREE_ERR_UNSUPPORTED"
    assert dd.ddtree_status_string(WORKSPACE) == "DDTREE_ERR_WORKSPACE"
    assert dd.ddtree_status_string(dd.DDTREE_ERR_HIP) == "DDTREE_ERR_HIP"
    assert dd.ddtree_status_string(12345) == "DDTREE_UNKNOWN_STATUS"


# ---------------------------------------------------------------- build_mask

def bm(parents=A, B=2, N=8, offs=A + 4096, mask=A + 8192, depth=A + 12288, pos=A + 16384, ok=A + 20480):
    return dd.lib().ddtree_build_mask(parents, B, N, offs, mask, depth, pos, ok, None)


def test_build_mask_rejects_bad_shapes_and_pointers():
    assert bm(N=0) == INVALID
    assert bm(B=-1) == INVALID
    assert bm(N=257) == UNSUPPORTED
    assert bm(B=0) == OK                      # nothing to do, nothing enqueued
    assert bm(parents=None) == INVALID
    assert bm(mask=None) == INVALID
    assert bm(depth=None) == INVALID
    assert bm(ok=None) == INVALID
    assert bm(mask=A + 16) == INVALID          # mask overlaps parents
    assert bm(depth=A + 8192 + 32) == INVALID  # depth overlaps mask
    assert bm(pos=A + 4096) == INVALID         # positions overlap prefix_offsets


# ---------------------------------------------------------------- verify_attn

def attn(dtype=BF16, B=1, N=8, H=64, Dl=512, Dr=64, q=A, qr=A + (1 << 24), ckv=A + (2 << 24), ld_ckv=576,
         krope=A + (2 << 24) + 1024, ld_krope=576, offs=A + (3 << 24), max_len=64, ckv_t=A + (4 << 24),
         ld_ckv_t=576, krope_t=A + (4 << 24) + 1024, ld_krope_t=576, mask=A + (5 << 24), scale=0.07,
         splits=1, o=A + (6 << 24), lse=A + (7 << 24), ws=None, ws_bytes=0):
    return dd.lib().ddtree_verify_attn(dtype, B, N, H, Dl, Dr, q, qr, ckv, ld_ckv, krope, ld_krope, offs, max_len,
                                       ckv_t, ld_ckv_t, krope_t, ld_krope_t, mask, scale, splits, o, lse, ws,
                                       ws_bytes, None)


def test_verify_attn_shape_support():
    assert attn(dtype=7) == UNSUPPORTED
    # bf16 at (512, 64) runs on the MFMA kernel, other dims on the generic kernel up to 512 each
    assert attn(Dl=1024, ld_ckv=1088, ld_ckv_t=1088) == UNSUPPORTED
    assert attn(Dr=520, ld_krope=1040, ld_krope_t=1040) == UNSUPPORTED
    assert attn(Dl=256, Dr=32, q=A + 1) == INVALID     # generic bf16 path: 2-byte alignment
    assert attn(Dl=256, Dr=32, ckv=A + (2 << 24) + 1) == INVALID
    assert attn(dtype=F32, Dl=1024) == UNSUPPORTED
    assert attn(N=257) == UNSUPPORTED
    assert attn(N=0) == INVALID
    assert attn(H=0) == INVALID
    assert attn(B=-2) == INVALID
    assert attn(B=0) == OK


def test_verify_attn_rejects_bad_pointers_strides_and_scale():
    assert attn(q=None) == INVALID
    assert attn(mask=None) == INVALID
    assert attn(o=None) == INVALID
    assert attn(ckv=None) == INVALID                  # a nonempty prefix needs a cache
    assert attn(ld_ckv=500) == INVALID                # row stride shorter than a row
    assert attn(ld_krope=60) == INVALID
    assert attn(ld_ckv=580) == INVALID                # bf16 rows must be 16-byte multiples
    assert attn(ld_ckv=(1 << 24) + 8) == UNSUPPORTED   # bf16 tile row offsets are 32-bit
    assert attn(ld_krope_t=(1 << 24) + 8) == UNSUPPORTED
    assert attn(ckv=A + (2 << 24) + 2) == INVALID     # misaligned bf16 base
    assert attn(scale=float("nan")) == INVALID
    assert attn(scale=float("inf")) == INVALID


def test_verify_attn_rejects_aliasing():
    assert attn(o=A + 64) == INVALID                  # o overlaps q_lat
    assert attn(lse=A + (6 << 24) + 4096) == INVALID  # lse overlaps o
    assert attn(o=A + (5 << 24)) == INVALID           # o overlaps mask
    # the first max_prefix_len (64) rows of the prefix cache: ckv rows end 73600 bytes past ckv, the
    # rotary rows (1024 bytes in, 128 bytes each) 73728
    assert attn(o=A + (2 << 24) + 4096) == INVALID            # o inside the latent rows
    assert attn(lse=A + (2 << 24) + 73650) == INVALID         # lse inside the last rotary row only
    assert attn(splits=4, ws=A + (2 << 24) + 32, ws_bytes=4 * 8 * 64 * 1032) == INVALID   # workspace


def test_workspace_contract():
    lib = dd.lib()
    # splits = 1 needs no workspace; S > 1 needs S * rows records of 2 Dl + 8 bytes (fp16 values, two floats)
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 8, 64, 512, 64, 4096, 1) == 0
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 8, 64, 512, 64, 4096, 4) == 4 * 8 * 64 * 1032
    assert lib.ddtree_verify_attn_workspace_size(F32, 1, 8, 4, 64, 32, 4096, 4) == 0   # fp32 path never splits
    assert attn(splits=4) == WORKSPACE
    assert attn(splits=4, ws=A + (8 << 24), ws_bytes=4 * 8 * 64 * 1032 - 4) == WORKSPACE
    assert attn(splits=4, ws=A + (8 << 24) + 8, ws_bytes=4 * 8 * 64 * 1032) == INVALID   # misaligned
    assert attn(splits=-1) == INVALID


def band_ws(R, W, Dl=512):
    """Band workspace for R row blocks per band and a bound of W windows: (window, slot, head/tail) partial
    slots of 128 row records (Dl fp16 values and two floats), then W records of 4 ints."""
    return 2 * W * R * 128 * (2 * Dl + 8) + 16 * W


BAND_WS = band_ws(32, 8)      # 32 row blocks per band, 8 windows: 67.6 MB


def test_auto_schedule():
    lib = dd.lib()
    # row blocks (128 rows each) in whole bands of 32, or a divisor of 32 of them: the band schedule (0)
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 64, 64, 512, 64, 4096) == 0       # 32 row blocks
    assert lib.ddtree_verify_attn_auto_splits(BF16, 4, 128, 64, 512, 64, 131072) == 0    # 64 per request
    assert lib.ddtree_verify_attn_auto_splits(BF16, 16, 64, 64, 512, 64, 32768) == 0
    assert lib.ddtree_verify_attn_auto_splits(BF16, 3, 32, 128, 512, 64, 10) == 0
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 0) == BAND_WS
    assert lib.ddtree_verify_attn_workspace_size(BF16, 16, 64, 64, 512, 64, 32768, 0) == BAND_WS
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 8, 64, 512, 64, 4096) == 0        # 4 row blocks
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 8, 64, 512, 64, 32) == 0
    assert lib.ddtree_verify_attn_auto_splits(BF16, 4, 128, 8, 512, 64, 131072) == 0     # 8 row blocks
    assert lib.ddtree_verify_attn_auto_splits(BF16, 2, 1, 8, 512, 64, 100) == 0          # one partial row block
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 16, 16, 512, 64, 4096) == 0       # 2 row blocks
    # one row block per band: 2 requests x 5 columns, under 8 columns a window: one window
    assert lib.ddtree_verify_attn_workspace_size(BF16, 2, 1, 8, 512, 64, 100, 0) == band_ws(1, 1)
    # otherwise uniform splits: enough workgroups to cover 256 CUs, at least 4 tiles per split
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 24, 64, 512, 64, 4096) == 22      # 12 row blocks: 256 / 12
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 40, 64, 512, 64, 4096) == 13      # 20 row blocks
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 40, 64, 512, 64, 4096, 0) == 13 * 40 * 64 * 1032
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 24, 64, 512, 64, 32) == 1         # 2 tiles: no split
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 3, 128, 512, 64, 4096) == 32      # 3 row blocks: 86, capped at 129 / 4
    assert lib.ddtree_verify_attn_auto_splits(BF16, 9, 40, 64, 512, 64, 4096) == 2       # 180 row blocks
    assert lib.ddtree_verify_attn_auto_splits(F32, 1, 8, 4, 64, 32, 4096) == 1
    # bf16 away from the MFMA dims takes the generic kernel: no split, no workspace
    assert lib.ddtree_verify_attn_auto_splits(BF16, 1, 64, 64, 256, 32, 4096) == 1
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 256, 32, 4096, 0) == 0
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 256, 32, 4096, 8) == 0
    assert lib.ddtree_verify_attn_workspace_size(F32, 1, 64, 64, 64, 32, 4096, 0) == 0
    # an explicit split count always takes the uniform schedule
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 1) == 0
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 8) == 8 * 64 * 64 * 1032
    # the band schedule needs its workspace like any split
    assert attn(N=64, splits=0) == WORKSPACE
    assert attn(N=64, splits=0, ws=A + (8 << 24), ws_bytes=band_ws(32, 1) - 4) == WORKSPACE   # max_len 64: 1 window


def test_band_workspace_is_sized_from_the_call():
    lib = dd.lib()
    ws = lambda B, N, H, L: lib.ddtree_verify_attn_workspace_size(BF16, B, N, H, 512, 64, L, 0)
    # the K2 workloads: 32 row blocks per band, 8 windows (the most for R = 32)
    assert ws(1, 64, 64, 4096) == ws(16, 64, 64, 32768) == ws(4, 128, 64, 131072) == band_ws(32, 8)
    # small requests: 130 columns / 8 = 16 windows (R = 1 or 4), far below the K2 size
    assert ws(1, 16, 8, 4096) == band_ws(1, 16) == 4227328
    assert ws(1, 64, 8, 4096) == band_ws(4, 16)
    # the bound follows max_prefix_len: a 64-node, 64-head request with no prefix has 2 columns, one window
    assert ws(1, 64, 64, 0) == band_ws(32, 1)
    assert ws(1, 64, 64, 250) == band_ws(32, 1)        # 8 + 2 columns
    assert ws(1, 64, 64, 800) == band_ws(32, 3)        # 25 + 2 columns
    # a workspace of the size returned is accepted by the host checks (and one byte less is not)
    assert attn(N=64, splits=0, max_len=800, ws=A + (8 << 24), ws_bytes=band_ws(32, 3) - 1) == WORKSPACE


def attn_noalloc(**kw):
    """The no-allocation variant with attn()'s fake pointers (no workspace arguments)."""
    a = dict(dtype=BF16, B=1, N=8, H=64, Dl=512, Dr=64, q=A, qr=A + (1 << 24), ckv=A + (2 << 24), ld_ckv=576,
             krope=A + (2 << 24) + 1024, ld_krope=576, offs=A + (3 << 24), max_len=64, ckv_t=A + (4 << 24),
             ld_ckv_t=576, krope_t=A + (4 << 24) + 1024, ld_krope_t=576, mask=A + (5 << 24), scale=0.07,
             splits=1, o=A + (6 << 24), lse=A + (7 << 24))
    a.update(kw)
    return dd.lib().ddtree_verify_attn_noalloc(*a.values(), None)


def test_noalloc_rejects_what_its_scratch_cannot_hold():
    """Checked before anything touches the device: a shape whose workspace exceeds the 72 MiB scratch is
    refused with DDTREE_ERR_WORKSPACE, and invalid arguments keep ddtree_verify_attn's errors."""
    lib = dd.lib()
    assert dd.DDTREE_NOALLOC_SCRATCH_BYTES == 72 << 20
    # the band schedule's largest workspace (32 row blocks per band, 8 windows) fits
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 0) == BAND_WS
    assert BAND_WS <= dd.DDTREE_NOALLOC_SCRATCH_BYTES
    # 64 nodes x 64 heads: 17 uniform splits fit, 18 do not
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 17) <= dd.DDTREE_NOALLOC_SCRATCH_BYTES
    assert lib.ddtree_verify_attn_workspace_size(BF16, 1, 64, 64, 512, 64, 4096, 18) > dd.DDTREE_NOALLOC_SCRATCH_BYTES
    assert attn_noalloc(N=64, splits=18, max_len=4096) == WORKSPACE
    assert attn_noalloc(N=64, splits=64, max_len=4096) == WORKSPACE
    assert attn_noalloc(B=0) == OK
    assert attn_noalloc(N=0) == INVALID
    assert attn_noalloc(q=None) == INVALID                                 # splits=1: no scratch needed
    assert attn_noalloc(o=A + 64) == INVALID


# ---------------------------------------------------------------- greedy_accept

def acc(logits=A, ld=512, tokens=A + (1 << 24), parents=A + (1 << 24) + 4096, B=1, N=8, V=512,
        tstar=A + (2 << 24), alen=A + (2 << 24) + 4096, nodes=A + (2 << 24) + 8192, commit=A + (2 << 24) + 12288):
    return dd.lib().ddtree_greedy_accept(logits, ld, tokens, parents, B, N, V, tstar, alen, nodes, commit, None)


def test_greedy_accept_validation():
    assert acc(V=0) == INVALID
    assert acc(ld=100) == INVALID                      # ld < V
    assert acc(N=0) == INVALID
    assert acc(N=300) == UNSUPPORTED
    assert acc(B=0) == OK
    assert acc(logits=None) == INVALID
    assert acc(commit=None) == INVALID
    assert acc(tstar=A + 100) == INVALID               # overlaps logits
    assert acc(nodes=A + (2 << 24) + 4) == INVALID     # overlaps target_argmax


def test_binding_refuses_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_LIB_PATH", "/nonexistent/libddtree.so")
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


# ---------------------------------------------------------------- compact_kv

def compact(dtype=BF16, B=2, N=16, Dl=512, Dr=64, ct=A + (1 << 24), ld_ct=576, rt=A + (1 << 24) + 1024, ld_rt=576,
            alen=A, nodes=A + 4096, dest=A + 8192, c=A + (2 << 24), ld_c=576, r=A + (2 << 24) + 1024, ld_r=576):
    return dd.lib().ddtree_compact_kv(dtype, B, N, Dl, Dr, ct, ld_ct, rt, ld_rt, alen, nodes, dest, c, ld_c, r, ld_r,
                                      None)


def test_compact_kv_validation():
    assert compact(dtype=5) == UNSUPPORTED
    assert compact(N=257) == UNSUPPORTED
    assert compact(N=0) == INVALID
    assert compact(B=-1) == INVALID
    assert compact(Dl=0) == INVALID
    assert compact(Dr=-1) == INVALID
    assert compact(B=0) == OK                          # nothing enqueued
    assert compact(ct=None) == INVALID
    assert compact(c=None) == INVALID
    assert compact(alen=None) == INVALID
    assert compact(nodes=None) == INVALID
    assert compact(dest=None) == INVALID
    assert compact(rt=None) == INVALID                 # a rotary part needs its rows
    assert compact(ld_ct=500) == INVALID               # stride shorter than a row
    assert compact(ld_r=60) == INVALID
    assert compact(ct=A + (1 << 24) + 1) == INVALID     # not aligned to the bf16 element
    assert compact(dtype=F32, c=A + (2 << 24) + 2) == INVALID
    assert compact(nodes=A + (1 << 24) + 64) == INVALID   # tree rows overlap the path arrays


# ---------------------------------------------------------------- build_tree

def btree(B=2, N=64, D=8, K=4, root=A, ct=A + 4096, cl=A + 8192, par=A + 16384, tok=A + 20480, dep=A + 24576,
          sc=A + 28672):
    return dd.lib().ddtree_build_tree(B, N, D, K, root, ct, cl, par, tok, dep, sc, None)


def test_build_tree_validation():
    assert btree(N=0) == INVALID
    assert btree(D=0) == INVALID
    assert btree(K=0) == INVALID
    assert btree(B=-1) == INVALID
    assert btree(N=257) == UNSUPPORTED
    assert btree(D=65) == UNSUPPORTED
    assert btree(K=65) == UNSUPPORTED
    assert btree(B=0, N=7, D=2, K=2) == OK             # 1 + 2 + 4 = 7 nodes fit
    assert btree(B=0, N=8, D=2, K=2) == UNSUPPORTED    # ... 8 do not
    assert btree(B=0, N=9, D=8, K=1) == OK             # a chain of 8 draft depths
    assert btree(B=0, N=10, D=8, K=1) == UNSUPPORTED
    assert btree(B=0) == OK
    assert btree(root=None) == INVALID
    assert btree(cl=None) == INVALID
    assert btree(par=None) == INVALID
    assert btree(tok=None) == INVALID
    assert btree(par=A + 8192 + 64) == INVALID          # parents overlap cand_logp
    assert btree(dep=A + 16384 + 4) == INVALID          # depth overlaps parents


# ---------------------------------------------------------------- rope_tree

def rope(dtype=BF16, B=2, N=16, H=64, Dr=64, q=A, k=A + (1 << 24), ld=576, pos=A + (2 << 24), inv=A + (3 << 24)):
    return dd.lib().ddtree_rope_tree(dtype, B, N, H, Dr, q, k, ld, pos, inv, None)


def test_rope_tree_validation():
    assert rope(dtype=9) == UNSUPPORTED
    assert rope(Dr=63) == INVALID              # odd width
    assert rope(Dr=0) == INVALID
    assert rope(Dr=1024) == UNSUPPORTED
    assert rope(N=257) == UNSUPPORTED
    assert rope(H=0) == INVALID
    assert rope(B=0) == OK
    assert rope(q=None, k=None) == OK          # nothing to rotate
    assert rope(pos=None) == INVALID
    assert rope(inv=None) == INVALID
    assert rope(ld=32) == INVALID              # key rows shorter than Dr
    assert rope(q=A + 1) == INVALID            # not element aligned
    assert rope(pos=A + 64) == INVALID         # positions overlap the rotated queries
    assert rope(k=A + 4096) == INVALID         # keys overlap the queries


def test_bench_traffic_hash_ignores_comments_only(tmp_path):
    """The HBM-traffic figure in the bench line is keyed to the kernel's code: comment-only edits keep the key,
    any code edit changes it."""
    import bench
    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) {  // trailing\n  /* block\n comment */ return x + 1;\n}\n")
    h0 = bench.source_hash(str(src))
    src.write_text("// another header\n\nint f(int x) {\n  return x + 1;  // changed comment\n}\n")
    assert bench.source_hash(str(src)) == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash(str(src)) != h0


def test_bench_traffic_summary_from_counter_files(tmp_path):
    """The HBM-traffic file is built from rocprofv3 --pmc outputs: per-dispatch KiB averaged over the attention
    kernel's dispatches, scaled by the copy's bytes over the copy's reading of the same counter."""
    import bench
    header = '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n'
    dirs = []
    for name, rows in (("f", [("k", bench.ATTN_KERNEL, 100.0), ("k", bench.ATTN_KERNEL, 300.0), ("o", "other", 5.0)]),
                       ("w", [("k", bench.ATTN_KERNEL, 50.0)]),
                       ("cf", [("c", "__amd_rocclr_copyBuffer", 512.0)]),
                       ("cw", [("c", "__amd_rocclr_copyBuffer", 1024.0)])):
        d = tmp_path / name / "host"
        d.mkdir(parents=True)
        (d / "x_counter_collection.csv").write_text(
            header + "".join(f'1,"{k}","C",{v}\n' for _, k, v in rows))
        dirs.append(str(tmp_path / name))
    out = bench.summarize_traffic(dirs, copy_mib=1, out_path=str(tmp_path / "t.json"))
    # copy of 1 MiB = 1024 KiB: fetch scale 1024 / 512 = 2, write scale 1; (200 * 2 + 50) KiB
    assert out["copy_calibration"]["fetch_scale"] == 2.0 and out["copy_calibration"]["write_scale"] == 1.0
    assert out["hbm_bytes_per_launch"] == (200 * 2 + 50) * 1024
    assert out["source_sha256_16"] == bench.source_hash(bench.ATTN_SOURCE)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with status 2 and a message, before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
