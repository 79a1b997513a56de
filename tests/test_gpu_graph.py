"""The hot path captured in a HIP graph: mask, tree-verify attention (band schedule and its
merge), greedy accept.  The library allocates nothing, issues no memset and never
synchronises, so one verify step can be captured once and replayed.  Every replay, with the
program's own eager work and synchronisations in between, must reproduce the eager results
bit for bit (the kernels use no atomics whose order could vary)."""
import numpy as np
import pytest
import torch

import mla_tree_verify_absorb_amd as dd
from gpu_util import DevWorkload
from synth import make_workload

pytestmark = pytest.mark.gpu

K2 = dict(H=64, Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0))


@pytest.mark.parametrize("heads", [64, 8])
def test_verify_step_graph_replays_match_eager(heads):
    """64 heads: bands of 32 row blocks over 8 windows; 8 heads: bands of 4 row blocks over 19
    windows, the band of the 3000-token request cut at several edges."""
    params = dict(K2)
    params.update(B=4, N=64, H=heads, prefix=("list", [500, 3000, 0, 1200]), tree=("bounded", 8, 4), V=4096,
                  p_match=0.8)
    w = make_workload(seed=41, **params)
    dw = DevWorkload(w)
    B, N, H = w.B, w.N, w.H
    dev = "cuda"
    W = (N + 31) // 32
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, B, N, H, w.Dl, w.Dr, dw.max_len) == 0
    need = dd.ddtree_verify_attn_workspace_size(dd.DDTREE_BF16, B, N, H, w.Dl, w.Dr, dw.max_len, 0)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    bufs = dict(mask=torch.empty((B, N, W), dtype=torch.int32, device=dev),
                depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                positions=torch.empty((B, N), dtype=torch.int64, device=dev),
                tree_ok=torch.empty((B,), dtype=torch.int32, device=dev),
                o=torch.empty((B, N, H, w.Dl), dtype=torch.float32, device=dev),
                lse=torch.empty((B, N, H), dtype=torch.float32, device=dev),
                ta=torch.empty((B, N), dtype=torch.int32, device=dev),
                al=torch.empty((B,), dtype=torch.int32, device=dev),
                an=torch.empty((B, N), dtype=torch.int32, device=dev),
                ct=torch.empty((B, N), dtype=torch.int32, device=dev))

    def step():
        dd.ddtree_build_mask(dw.parents, dw.offsets, mask=bufs["mask"], depth=bufs["depth"],
                             positions=bufs["positions"], tree_ok=bufs["tree_ok"])
        dd.ddtree_verify_attn(dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, dw.max_len, dw.ckv_tree,
                              dw.krope_tree, bufs["mask"], w.scale, num_splits=0, o=bufs["o"], lse=bufs["lse"],
                              workspace=ws)
        dd.ddtree_greedy_accept(dw.logits, dw.tokens, dw.parents, target_argmax=bufs["ta"], accept_len=bufs["al"],
                                accept_nodes=bufs["an"], commit_tokens=bufs["ct"])

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in bufs.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        for v in bufs.values():                  # eager work between replays: clobber every output
            v.fill_(-7)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            assert torch.equal(v, eager[k]), f"replay {replay}: {k} differs from the eager step"
    print(f"3 replays bitwise equal to eager; accept_len {eager['al'].tolist()}")
