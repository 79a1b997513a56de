"""Helpers shared by the GPU tests: move a synthetic workload to the device in the
library's layouts, run the oracle on the same values, and compare."""
from __future__ import annotations

import numpy as np
import torch

import mla_tree_verify_absorb_amd as dd
from oracle import build_mask_ref, greedy_accept_ref, verify_attn_ref
from synth import Workload

DEV = "cuda:0"
FP32_ABS_TOL = 1e-5        # fp32 inputs: max abs error on o and lse
BF16_NORM_TOL = 2e-3       # bf16 inputs: max|err| / max|ref| on o and lse
# bf16 inputs, K2 workloads: max |lse - lse_ref| in nats.  Below the 2.4e-4 that leaving out (or doubling)
# one 32-key tile of a 131072-key row would cause (ln(1 - 32/131072)), so such a mistake fails here even
# though it passes the normwise bound.
BF16_LSE_ABS_TOL = 1.5e-4


def t_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


class DevWorkload:
    """Device copies of a workload: fused [T, Dl+Dr] cache, views for c and r."""

    def __init__(self, w: Workload):
        self.w = w
        self.parents = torch.from_numpy(w.parents).to(DEV)
        self.offsets = torch.from_numpy(w.prefix_offsets).to(DEV)
        self.q_lat = t_dev(w.q_lat, w.dtype)
        self.q_rope = t_dev(w.q_rope, w.dtype)
        self.kv = t_dev(w.kv, w.dtype)
        self.kv_tree = t_dev(w.kv_tree, w.dtype)
        self.ckv, self.krope = self.kv[:, :w.Dl], self.kv[:, w.Dl:]
        self.ckv_tree, self.krope_tree = self.kv_tree[..., :w.Dl], self.kv_tree[..., w.Dl:]
        self.logits = None if w.logits is None else torch.from_numpy(w.logits).to(DEV)
        self.tokens = None if w.tokens is None else torch.from_numpy(w.tokens).to(DEV)
        self.max_len = int(w.prefix_lens.max()) if w.B else 0

    def build_mask(self):
        return dd.ddtree_build_mask(self.parents, self.offsets)

    def attn(self, mask, num_splits=0):
        return dd.ddtree_verify_attn(self.q_lat, self.q_rope, self.ckv, self.krope, self.offsets, self.max_len,
                                     self.ckv_tree, self.krope_tree, mask, self.w.scale, num_splits=num_splits)


def oracle_attn(w: Workload, mask_u32: np.ndarray, nodes=None):
    f = w.f32
    kv = f("kv")
    kt = f("kv_tree")
    return verify_attn_ref(f("q_lat"), f("q_rope"), kv[:, :w.Dl], kv[:, w.Dl:], w.prefix_offsets,
                           kt[..., :w.Dl], kt[..., w.Dl:], mask_u32, w.scale, nodes=nodes)


def mask_np(mask_t: torch.Tensor) -> np.ndarray:
    return mask_t.cpu().numpy().view(np.uint32)


def lse_abs_err(lse, lse_ref, nodes=None):
    """max |lse - lse_ref| (nats) over all rows, or the sampled nodes' rows."""
    lse = lse.cpu().numpy().astype(np.float64)
    if nodes is not None:
        bi = tuple(np.array([b for b, _ in nodes])), tuple(np.array([i for _, i in nodes]))
        lse, lse_ref = lse[bi], lse_ref[bi]
    return float(np.abs(lse - lse_ref).max())


def compare_attn(w: Workload, o, lse, o_ref, lse_ref, nodes=None):
    """Returns (o_err, lse_err) in the config's metric and asserts the tolerance."""
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    if nodes is not None:
        bi = tuple(np.array([b for b, _ in nodes])), tuple(np.array([i for _, i in nodes]))
        o, lse, o_ref, lse_ref = o[bi], lse[bi], o_ref[bi], lse_ref[bi]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    if w.dtype == "f32":
        eo = float(np.abs(o - o_ref).max())
        el = float(np.abs(lse - lse_ref).max())
        assert eo <= FP32_ABS_TOL and el <= FP32_ABS_TOL, (eo, el)
    else:
        eo = float(np.abs(o - o_ref).max() / np.abs(o_ref).max())
        el = float(np.abs(lse - lse_ref).max() / np.abs(lse_ref).max())
        assert eo <= BF16_NORM_TOL and el <= BF16_NORM_TOL, (eo, el)
    return eo, el


def check_mask(dw: DevWorkload):
    mask, depth, pos, ok = dw.build_mask()
    torch.cuda.synchronize()
    m_ref, d_ref, p_ref, ok_ref = build_mask_ref(dw.w.parents, dw.w.prefix_lens)
    assert np.array_equal(mask_np(mask), m_ref)
    assert np.array_equal(depth.cpu().numpy(), d_ref)
    assert np.array_equal(pos.cpu().numpy(), p_ref)
    assert np.array_equal(ok.cpu().numpy(), ok_ref)
    return mask, m_ref


def check_accept(dw: DevWorkload):
    tstar, alen, nodes, commit = dd.ddtree_greedy_accept(dw.logits, dw.tokens, dw.parents)
    torch.cuda.synchronize()
    ref = greedy_accept_ref(dw.w.logits, dw.w.tokens, dw.w.parents)
    for got, exp in zip((tstar, alen, nodes, commit), ref):
        assert np.array_equal(got.cpu().numpy(), exp)
    return ref
