"""GPU: ddtree_verify_attn_noalloc (the library's own per-GPU scratch in place of a caller workspace) gives
the same o and lse as ddtree_verify_attn with a workspace, bit for bit, on calls in a row with shrinking
inputs (the scratch keeps the previous call's contents), and both match the oracle to the bf16 bar."""
import numpy as np
import pytest
import torch

import mla_tree_verify_absorb_amd as dd
from gpu_util import DevWorkload, check_mask, compare_attn, oracle_attn
from synth import make_workload

pytestmark = pytest.mark.gpu

K2 = dict(Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0))


def run_both(w, num_splits=0, oracle=True):
    dw = DevWorkload(w)
    mask, m_ref = check_mask(dw)
    o_ws, lse_ws = dw.attn(mask, num_splits=num_splits)
    need = dd.ddtree_verify_attn_workspace_size(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len, num_splits)
    assert 0 < need <= dd.DDTREE_NOALLOC_SCRATCH_BYTES                  # the case uses the scratch
    o = torch.full_like(o_ws, float("nan"))
    lse = torch.full_like(lse_ws, float("nan"))
    dd.ddtree_verify_attn_noalloc(dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, dw.max_len, dw.ckv_tree,
                                  dw.krope_tree, mask, w.scale, o=o, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    if not oracle:   # the workspace call's parity at this shape is covered by the parity tests
        return need, float("nan"), float("nan")
    o_ref, lse_ref = oracle_attn(w, m_ref)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref)
    return need, eo, el


def test_noalloc_equals_workspace_call_on_shrinking_calls():
    # 0: one 64-node request at 64 heads over 4096 tokens: the band schedule's largest workspace
    #    (32 row blocks per band, 8 windows, 67.6 MB), every row merged from 8 pieces
    w0 = make_workload(B=1, N=64, H=64, prefix=("fixed", 4096), tree=("bounded", 8, 4), seed=50, **K2)
    n0, _, _ = run_both(w0, oracle=False)
    # 1: two requests, 4 row blocks each (16 heads x 32 nodes), ragged prefixes: band schedule over 5
    #    windows, bands cut by window edges, so partials and the merge go through the scratch
    w1 = make_workload(B=2, N=32, H=16, prefix=("list", [1000, 300]), tree=("bounded", 8, 4), seed=51, **K2)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, 2, 32, 16, 512, 64, 1000) == 0
    n1, e1o, e1l = run_both(w1)
    assert n1 < n0
    # 2: a smaller call right after: one request, one row block (8 heads x 16 nodes), 500 tokens
    w2 = make_workload(B=1, N=16, H=8, prefix=("fixed", 500), tree=("bounded", 8, 4), seed=52, **K2)
    n2, e2o, e2l = run_both(w2)
    assert n2 < n1
    # 3: uniform splits through the scratch (an explicit split count), smaller again
    w3 = make_workload(B=1, N=8, H=16, prefix=("fixed", 700), tree=("chain",), seed=53, **K2)
    n3, e3o, e3l = run_both(w3, num_splits=3)
    print(f"no-alloc: scratch use {n0}, {n1}, {n2}, {n3} bytes; normwise o/lse errors {e1o:.2e}/{e1l:.2e}, "
          f"{e2o:.2e}/{e2l:.2e}, {e3o:.2e}/{e3l:.2e}")


def test_noalloc_refuses_a_call_its_scratch_cannot_hold():
    # 18 uniform splits of 4096 rows need 76.1 MB
    w = make_workload(B=1, N=64, H=64, prefix=("fixed", 4096), tree=("bounded", 8, 4), seed=54, **K2)
    dw = DevWorkload(w)
    mask, _ = check_mask(dw)
    o = torch.empty((1, 64, 64, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="DDTREE_ERR_WORKSPACE"):
        dd.ddtree_verify_attn_noalloc(dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, dw.max_len, dw.ckv_tree,
                                      dw.krope_tree, mask, w.scale, o=o, lse=lse, num_splits=18)
