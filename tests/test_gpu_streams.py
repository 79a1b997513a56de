"""GPU: the library keeps no state between calls (the no-allocation entry point aside), so calls from several
host threads, each on its own HIP stream with its own outputs and workspace, may overlap.  Two threads run the
verify step (mask, attention, greedy accept) on different workloads many times over at the same time -- one
through the band schedule with cut bands and its merge, one through uniform KV splits and their merge -- and
every result equals the serial call's bit for bit."""
import threading

import numpy as np
import pytest
import torch

import mla_tree_verify_absorb_amd as dd
from gpu_util import DevWorkload
from synth import make_workload

pytestmark = pytest.mark.gpu

K2 = dict(Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0))
ITERS = 25


class Step:
    """One workload's verify step with every output and the workspace allocated up front."""

    def __init__(self, w):
        self.w, self.dw = w, DevWorkload(w)
        dev = self.dw.q_lat.device
        B, N, H = w.B, w.N, w.H
        self.mask = torch.empty((B, N, (N + 31) // 32), dtype=torch.int32, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.pos = torch.empty((B, N), dtype=torch.int64, device=dev)
        self.ok = torch.empty((B,), dtype=torch.int32, device=dev)
        self.o = torch.empty((B, N, H, w.Dl), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
        need = dd.ddtree_verify_attn_workspace_size(dd.DDTREE_BF16, B, N, H, w.Dl, w.Dr, self.dw.max_len, 0)
        assert need > 0                       # both workloads merge partials through the workspace
        self.ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        self.targ = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.alen = torch.empty((B,), dtype=torch.int32, device=dev)
        self.nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.commit = torch.empty((B, N), dtype=torch.int32, device=dev)

    def run(self):
        dw, w = self.dw, self.w
        dd.ddtree_build_mask(dw.parents, dw.offsets, mask=self.mask, depth=self.depth, positions=self.pos,
                             tree_ok=self.ok)
        dd.ddtree_verify_attn(dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, dw.max_len, dw.ckv_tree,
                              dw.krope_tree, self.mask, w.scale, o=self.o, lse=self.lse, workspace=self.ws)
        dd.ddtree_greedy_accept(dw.logits, dw.tokens, dw.parents, target_argmax=self.targ, accept_len=self.alen,
                                accept_nodes=self.nodes, commit_tokens=self.commit)

    def outputs(self):
        return [t.clone() for t in (self.mask, self.depth, self.pos, self.ok, self.o, self.lse, self.targ,
                                    self.alen, self.nodes, self.commit)]


def test_overlapping_calls_from_two_threads_on_their_own_streams():
    # band schedule: 64 nodes x 64 heads over ragged prefixes, bands cut by window edges
    wa = make_workload(B=2, N=64, H=64, prefix=("list", [3000, 700]), tree=("bounded", 8, 4), V=5000,
                       p_match=0.7, seed=61, **K2)
    # uniform KV splits: 40 nodes x 16 heads (5 row blocks a request), an empty prefix among them
    wb = make_workload(B=3, N=40, H=16, prefix=("list", [300, 0, 77]), tree=("bounded", 8, 4), V=3000,
                       p_match=0.7, seed=62, **K2)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, 2, 64, 64, 512, 64, 3000) == 0
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, 3, 40, 16, 512, 64, 300) > 1
    steps = [Step(wa), Step(wb)]
    torch.cuda.synchronize()

    serial = []
    for st in steps:
        st.run()
        torch.cuda.synchronize()
        serial.append(st.outputs())
        assert int(st.alen.max()) >= 1     # the accept path is exercised

    for st in steps:                        # poison every output before the concurrent runs
        for t in (st.mask, st.depth, st.pos, st.ok, st.o, st.lse, st.targ, st.alen, st.nodes, st.commit):
            t.fill_(-7)
    torch.cuda.synchronize()

    start = threading.Barrier(len(steps))
    errors = []

    def worker(st):
        try:
            stream = torch.cuda.Stream()    # default priority
            start.wait()
            with torch.cuda.stream(stream):
                for _ in range(ITERS):
                    st.run()
            stream.synchronize()
        except Exception as exc:            # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(st,)) for st in steps]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()

    for k, st in enumerate(steps):
        for i, (got, want) in enumerate(zip(st.outputs(), serial[k])):
            assert torch.equal(got, want), f"workload {k}: output {i} differs from the serial call"
    print(f"two threads x {ITERS} overlapping verify steps: every output equal to the serial calls")
