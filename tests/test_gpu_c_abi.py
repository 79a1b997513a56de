"""GPU: a plain C program (tests/c_abi_step.c: hipMalloc, a hipStream_t, no Python or torch) runs one verify
step through libddtree.so: build_mask, verify_attn with a caller workspace and without one (noalloc),
greedy_accept and compact_kv.  Its outputs, written as raw files, are checked here against the oracle: mask,
depth, positions, accept results and the compacted cache bit for bit, attention to the bf16 bar, and the two
attention calls bitwise equal to each other.  The program is built by __graft_entry__.build()."""
import os
import subprocess

import numpy as np
import pytest

from gpu_util import BF16_NORM_TOL
from oracle import build_mask_ref, compact_kv_ref, greedy_accept_ref, verify_attn_ref
from synth import make_workload

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "_build", "c_abi_step")


def test_c_caller_runs_a_verify_step(tmp_path):
    if not os.path.exists(BIN):   # build() warns when gcc is unavailable and builds the library regardless
        pytest.skip(f"{BIN} was not built (no C compiler when __graft_entry__.build() ran)")
    # ragged prefixes with an empty one; 40 nodes x 16 heads = 5 row blocks per request
    w = make_workload(B=3, N=40, H=16, Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0),
                      prefix=("list", [300, 0, 77]), tree=("bounded", 8, 4), V=3000, p_match=0.7, seed=91)
    B, N, H, Dl, Dr, V, T = w.B, w.N, w.H, w.Dl, w.Dr, w.V, w.T
    max_len = int(w.prefix_lens.max())
    cache_rows = T + B * N                       # the prefix, then room for each request's accepted rows
    ckv = np.zeros((cache_rows, Dl), np.uint16)
    krope = np.zeros((cache_rows, Dr), np.uint16)
    ckv[:T], krope[:T] = w.kv[:, :Dl], w.kv[:, Dl:]
    ckv_tree = np.ascontiguousarray(w.kv_tree[..., :Dl])
    krope_tree = np.ascontiguousarray(w.kv_tree[..., Dl:])
    dest_rows = (T + np.arange(B) * N).astype(np.int64)
    files = {"q_lat": w.q_lat, "q_rope": w.q_rope, "ckv": ckv, "krope": krope, "offsets": w.prefix_offsets,
             "ckv_tree": ckv_tree, "krope_tree": krope_tree, "parents": w.parents, "logits": w.logits,
             "tokens": w.tokens, "dest_rows": dest_rows}
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(str(tmp_path / f"{name}.bin"))
    (tmp_path / "meta.txt").write_text(f"{B} {N} {H} {Dl} {Dr} {V} {max_len} {cache_rows} {w.scale!r}\n")

    res = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stderr
    from mla_tree_verify_absorb_amd.build import source_digest
    from __graft_entry__ import c_driver_source_hash
    assert f"source {c_driver_source_hash()}" in res.stdout, "stale C caller: run __graft_entry__.build()"
    assert f"digest {source_digest()}" in res.stdout            # the library built from these sources

    def out(name, dtype, shape):
        return np.fromfile(str(tmp_path / f"out_{name}.bin"), dtype=dtype).reshape(shape)

    W = (N + 31) // 32
    m_ref, d_ref, p_ref, ok_ref = build_mask_ref(w.parents, w.prefix_lens)
    assert np.array_equal(out("mask", np.uint32, (B, N, W)), m_ref)
    assert np.array_equal(out("depth", np.int32, (B, N)), d_ref)
    assert np.array_equal(out("pos", np.int64, (B, N)), p_ref)
    assert np.array_equal(out("ok", np.int32, (B,)), ok_ref)

    o, lse = out("o", np.float32, (B, N, H, Dl)), out("lse", np.float32, (B, N, H))
    assert np.array_equal(out("o_noalloc", np.float32, (B, N, H, Dl)).view(np.uint32), o.view(np.uint32))
    assert np.array_equal(out("lse_noalloc", np.float32, (B, N, H)).view(np.uint32), lse.view(np.uint32))
    kvf, ktf = w.f32("kv"), w.f32("kv_tree")
    o_ref, lse_ref = verify_attn_ref(w.f32("q_lat"), w.f32("q_rope"), kvf[:, :Dl], kvf[:, Dl:], w.prefix_offsets,
                                     ktf[..., :Dl], ktf[..., Dl:], m_ref, w.scale)
    # the bf16 bar of the small cases (normwise on o and lse); the absolute lse bound of the long-context
    # workloads does not apply: with a few hundred keys a row's single-term bf16 exp-sum averages its rounding
    # over fewer terms
    eo = np.abs(o - o_ref).max() / np.abs(o_ref).max()
    el = np.abs(lse - lse_ref).max() / np.abs(lse_ref).max()
    print(f"C caller: normwise o err {eo:.2e}, lse err {el:.2e} "
          f"(absolute {np.abs(lse - lse_ref).max():.2e} nats)")
    assert eo <= BF16_NORM_TOL and el <= BF16_NORM_TOL, (eo, el)

    targ_ref, alen_ref, nodes_ref, commit_ref = greedy_accept_ref(w.logits, w.tokens, w.parents)
    assert np.array_equal(out("target_argmax", np.int32, (B, N)), targ_ref)
    assert np.array_equal(out("accept_len", np.int32, (B,)), alen_ref)
    assert np.array_equal(out("accept_nodes", np.int32, (B, N)), nodes_ref)
    assert np.array_equal(out("commit_tokens", np.int32, (B, N)), commit_ref)
    assert alen_ref.max() >= 1                                   # some drafts were accepted and moved

    ckv_exp, krope_exp = compact_kv_ref(ckv_tree, krope_tree, alen_ref, nodes_ref, ckv.copy(), krope.copy(),
                                        dest_rows)
    assert np.array_equal(out("ckv", np.uint16, (cache_rows, Dl)), ckv_exp)
    assert np.array_equal(out("krope", np.uint16, (cache_rows, Dr)), krope_exp)
