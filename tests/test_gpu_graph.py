"""GPU: the verify step (mask, attention, greedy accept) captured once in a HIP graph and replayed.

Every entry point only enqueues kernels on the caller's stream (no allocation, no memset inside), so a serving
loop can capture a step and replay it; the no-allocation attention entry point covers callers that cannot hand
over a workspace either.  The graph holds every output buffer.  Between replays the test changes the inputs in
place with eager work and synchronizes, then checks each replay bit for bit against eager calls on the same
inputs, and checks that the replay followed the change."""
import numpy as np
import pytest
import torch

import mla_tree_verify_absorb_amd as dd
from gpu_util import DevWorkload
from synth import make_workload

pytestmark = pytest.mark.gpu

K2 = dict(Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0))


@pytest.mark.parametrize("noalloc", [True, False])
def test_verify_step_replays_in_a_hip_graph(noalloc):
    # 64 nodes x 64 heads: bands of 32 row blocks cut by window edges (partial records and their merge)
    w = make_workload(B=2, N=64, H=64, prefix=("list", [3000, 700]), tree=("bounded", 8, 4), seed=81, **K2)
    dw = DevWorkload(w)
    dev = dw.q_lat.device
    B, N, H, V = w.B, w.N, w.H, 4096
    gen = torch.Generator().manual_seed(82)
    logits = torch.randn((B, N, V), generator=gen).to(dev)
    # drafts that follow the parent's argmax on 80% of the nodes, so that paths of several nodes get accepted
    parents_l = dw.parents.long().clamp(min=0)
    follow = logits.argmax(-1).gather(1, parents_l).int()
    other = torch.randint(0, V, (B, N), generator=gen, dtype=torch.int32).to(dev)
    tokens = torch.where(torch.rand((B, N), generator=gen).to(dev) < 0.8, follow, other).contiguous()

    W = (N + 31) // 32
    mask = torch.empty((B, N, W), dtype=torch.int32, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    pos = torch.empty((B, N), dtype=torch.int64, device=dev)
    ok = torch.empty((B,), dtype=torch.int32, device=dev)
    o = torch.empty((B, N, H, w.Dl), dtype=torch.float32, device=dev)
    lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    need = dd.ddtree_verify_attn_workspace_size(dd.DDTREE_BF16, B, N, H, w.Dl, w.Dr, dw.max_len, 0)
    assert need > 0
    ws = None if noalloc else torch.empty((need,), dtype=torch.uint8, device=dev)
    targ = torch.empty((B, N), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    commit = torch.empty((B, N), dtype=torch.int32, device=dev)
    outputs = (mask, depth, pos, ok, o, lse, targ, alen, nodes, commit)

    def step():
        dd.ddtree_build_mask(dw.parents, dw.offsets, mask=mask, depth=depth, positions=pos, tree_ok=ok)
        args = (dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, dw.max_len, dw.ckv_tree, dw.krope_tree, mask,
                w.scale)
        if noalloc:
            dd.ddtree_verify_attn_noalloc(*args, o=o, lse=lse)
        else:
            dd.ddtree_verify_attn(*args, o=o, lse=lse, workspace=ws)
        dd.ddtree_greedy_accept(logits, tokens, dw.parents, target_argmax=targ, accept_len=alen, accept_nodes=nodes,
                                commit_tokens=commit)

    # warm-up on a side stream (the first no-allocation call looks up the scratch address), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    prev = None
    for rep in range(4):
        if rep == 1:
            dw.q_lat.mul_(0.5)                              # exact in bf16: every score halves
        elif rep == 2:
            logits.copy_(torch.roll(logits, 1, dims=2))     # every row's argmax moves by one
        elif rep == 3:
            dw.ckv_tree.mul_(2.0)                           # the tree rows' latent keys and values change
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs]
        step()
        torch.cuda.synchronize()
        eager = [t.clone() for t in outputs]
        for i, (a, b) in enumerate(zip(got, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"
        assert int(ok.min()) == 1 and bool(torch.isfinite(o).all())
        if rep == 0:
            first_alen = got[7].tolist()
            assert max(first_alen) >= 1                     # the accept path is exercised
        if prev is not None:
            changed = {1: [4, 5], 2: [6], 3: [4]}[rep]      # o/lse; target argmax; o
            for i in changed:
                assert not torch.equal(got[i], prev[i]), f"replay {rep}: output {i} did not follow its input"
        prev = got
    print(f"graph replays (noalloc={noalloc}): accept lengths {first_alen}, then {alen.tolist()} after the logits moved")
