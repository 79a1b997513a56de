"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test fixes the oracle to a closed form, a special case that reduces to a
library routine (torch's scaled_dot_product_attention / logsumexp in float64
on the CPU), an algebraically different formulation (the unabsorbed MLA form,
the dense -inf mask form, the per-path causal form, the split/merge identity)
or brute force on tiny inputs.  A dropped term, a wrong sign or index or a
transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (build_mask_ref, build_tree_ref, compact_kv_ref, greedy_accept_ref, rope_inv_freq, rope_neox_ref,
                    target_argmax_ref, verify_attn_ref)
from synth import bounded_tree, chain_tree, make_config, make_draft_candidates, make_workload, uniform_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers that are independent of the oracle's code
# ----------------------------------------------------------------------------

def closure_visibility(parent_row):
    """Ancestor-or-self relation as a dense bool matrix, by boolean matrix powers."""
    n = len(parent_row)
    A = np.zeros((n, n), dtype=bool)
    for i in range(1, n):
        A[i, parent_row[i]] = True
    R = np.eye(n, dtype=bool)
    step = A.copy()
    for _ in range(n):
        R |= step
        step = (step.astype(np.int64) @ A.astype(np.int64)) > 0
    return R


def pack_words(vis):
    """Dense bool [N, N] -> uint32 words [N, W], bit k%32 of word k//32."""
    n = vis.shape[0]
    w = (n + 31) // 32
    padded = np.zeros((n, 32 * w), dtype=bool)
    padded[:, :n] = vis
    by = np.packbits(padded, axis=1, bitorder="little")
    return by.view(np.uint32).reshape(n, w) if by.shape[1] % 4 == 0 else None


def sdpa(q, k, v, mask, scale):
    """torch scaled_dot_product_attention in float64. q [H,nq,d], k/v [nk,*], mask bool [nq,nk]."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).unsqueeze(0).expand(qt.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).unsqueeze(0).expand(qt.shape[0], -1, -1)
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out.numpy()


def torch_lse(scores, mask):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float64))
    if mask is not None:
        s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


def f64_case(w):
    q = w.f32("q_lat").astype(np.float64)
    qr = w.f32("q_rope").astype(np.float64)
    kv = w.f32("kv").astype(np.float64)
    kt = w.f32("kv_tree").astype(np.float64)
    return q, qr, kv[:, :w.Dl], kv[:, w.Dl:], kt[..., :w.Dl], kt[..., w.Dl:]


def run_oracle(w):
    mask, depth, pos, ok = build_mask_ref(w.parents, w.prefix_lens)
    q, qr, c, r, ct, rt = f64_case(w)
    o, lse = verify_attn_ref(q, qr, c, r, w.prefix_offsets, ct, rt, mask, w.scale)
    return mask, depth, o, lse


def small(seed, B=2, N=12, H=3, Dl=16, Dr=8, L=(5, 9), tree=("uniform",), std=1.0):
    return make_workload(B=B, N=N, H=H, Dl=Dl, Dr=Dr, dtype="f32", std=std, scale=0.37,
                         prefix=("list", list(L)), tree=tree, seed=seed)


# ----------------------------------------------------------------------------
# visibility mask, depth, positions
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n", [1, 2, 7, 32, 33, 64, 100])
def test_mask_equals_transitive_closure(seed, n):
    rng = np.random.default_rng(seed)
    trees = [chain_tree(n), uniform_tree(rng, n), np.array([-1] + [0] * (n - 1), np.int32)]
    if n > 1:
        trees.append(bounded_tree(rng, n, 12, 4))
    parents = np.stack(trees)
    lens = rng.integers(0, 1000, size=len(trees))
    mask, depth, pos, ok = build_mask_ref(parents, lens)
    assert ok.tolist() == [1] * len(trees)
    assert mask.shape == (len(trees), n, (n + 31) // 32)
    for b in range(len(trees)):
        vis = closure_visibility(parents[b])
        packed = pack_words(vis)
        assert np.array_equal(mask[b], packed)
        # ancestor-or-self set size is depth + 1
        assert np.array_equal(vis.sum(axis=1) - 1, depth[b])
        assert np.array_equal(pos[b], lens[b] + depth[b].astype(np.int64))


def test_depth_special_trees():
    mask, depth, pos, ok = build_mask_ref(np.stack([chain_tree(9), np.array([-1] + [0] * 8, np.int32)]))
    assert depth[0].tolist() == list(range(9))
    assert depth[1].tolist() == [0] + [1] * 8
    assert pos.tolist() == depth.tolist()      # no prefix lengths: position = depth
    # star: every node sees the root and itself only
    assert all(int(mask[1, i, 0]) == (1 | (1 << i)) for i in range(9))


def test_mask_bit_layout_crosses_words():
    n = 40
    mask, depth, _, _ = build_mask_ref(chain_tree(n)[None])
    assert int(mask[0, 39, 0]) == 0xFFFFFFFF and int(mask[0, 39, 1]) == 0xFF
    assert int(mask[0, 32, 1]) == 1 and int(mask[0, 31, 1]) == 0


@pytest.mark.parametrize("bad", [
    [0, 0, 1],        # root parent not -1
    [-1, 1, 0],       # self parent
    [-1, 0, 3, 0],    # forward parent
    [-1, -1, 0],      # second root
    [-1, 0, -5],      # negative parent
])
def test_invalid_tree_flagged(bad):
    parents = np.stack([np.array(bad, np.int32), chain_tree(len(bad))])
    mask, depth, pos, ok = build_mask_ref(parents, np.array([3, 4]))
    assert ok.tolist() == [0, 1]
    assert not mask[0].any() and (depth[0] == -1).all() and (pos[0] == -1).all()
    assert depth[1].tolist() == list(range(len(bad)))


# ----------------------------------------------------------------------------
# attention: absorbed MLA form against the unabsorbed form (torch SDPA)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_absorbed_equals_unabsorbed(seed):
    """o_lat mapped through W_UV equals explicit attention with K = [W_UK c ; r], V = W_UV c."""
    H, Dl, Dr, Dn, Dv = 3, 16, 8, 6, 5
    w = small(seed, H=H, Dl=Dl, Dr=Dr, tree=("bounded", 4, 3))
    rng = np.random.default_rng(100 + seed)
    W_UK = rng.standard_normal((H, Dn, Dl))       # k_nope = W_UK c
    W_UV = rng.standard_normal((H, Dv, Dl))       # v = W_UV c
    _, qr, c, r, ct, rt = f64_case(w)
    q_nope = rng.standard_normal((w.B, w.N, H, Dn))
    q_lat = np.einsum("bnhd,hdl->bnhl", q_nope, W_UK)   # absorbed query: W_UK^T q_nope
    mask, _, _, _ = build_mask_ref(w.parents, w.prefix_lens)
    o_lat, lse = verify_attn_ref(q_lat, qr, c, r, w.prefix_offsets, ct, rt, mask, w.scale)
    for b in range(w.B):
        s0, s1 = int(w.prefix_offsets[b]), int(w.prefix_offsets[b + 1])
        L = s1 - s0
        vis = closure_visibility(w.parents[b])
        allowed = np.concatenate([np.ones((w.N, L), bool), vis], axis=1)       # [N, L+N]
        C = np.concatenate([c[s0:s1], ct[b]])
        R = np.concatenate([r[s0:s1], rt[b]])
        for h in range(H):
            K = np.concatenate([C @ W_UK[h].T, R], axis=1)                     # [L+N, Dn+Dr]
            Vv = C @ W_UV[h].T                                                  # [L+N, Dv]
            Q = np.concatenate([q_nope[b, :, h], qr[b, :, h]], axis=1)          # [N, Dn+Dr]
            ref = sdpa(Q[None], K, Vv, allowed, w.scale)[0]
            got = o_lat[b, :, h] @ W_UV[h].T
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
            ref_lse = torch_lse(w.scale * (Q @ K.T), allowed)
            np.testing.assert_allclose(lse[b, :, h], ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_general_tree_matches_sdpa_latent(seed):
    """Library cross-check in the latent space with an explicit boolean mask."""
    w = small(seed, B=3, N=20, L=(0, 3, 17), tree=("uniform",))
    mask, depth, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    for b in range(w.B):
        s0, s1 = int(w.prefix_offsets[b]), int(w.prefix_offsets[b + 1])
        allowed = np.concatenate([np.ones((w.N, s1 - s0), bool), closure_visibility(w.parents[b])], axis=1)
        K = np.concatenate([np.concatenate([c[s0:s1], ct[b]]), np.concatenate([r[s0:s1], rt[b]])], axis=1)
        V = np.concatenate([c[s0:s1], ct[b]])
        Q = np.concatenate([q[b], qr[b]], axis=2).transpose(1, 0, 2)            # [H, N, Dl+Dr]
        ref = sdpa(Q, K, V, allowed, w.scale).transpose(1, 0, 2)
        np.testing.assert_allclose(o[b], ref, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# special trees that reduce to textbook attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L", [0, 1, 8, 50])
def test_chain_equals_causal(L):
    """A single chain verifies exactly like causal attention over prefix ++ chain."""
    w = make_workload(B=1, N=9, H=4, Dl=32, Dr=16, dtype="f32", std=1.0, scale=0.21,
                      prefix=("fixed", L), tree=("chain",), seed=L)
    _, _, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    K = np.concatenate([np.concatenate([c, ct[0]]), np.concatenate([r, rt[0]])], axis=1)
    V = np.concatenate([c, ct[0]])
    Q = np.concatenate([q[0], qr[0]], axis=2).transpose(1, 0, 2)
    # causal with the queries at the last N positions (bottom-right aligned)
    n, T = w.N, L + w.N
    allowed = np.arange(T)[None, :] <= (L + np.arange(n))[:, None]
    ref = sdpa(Q, K, V, allowed, w.scale).transpose(1, 0, 2)
    np.testing.assert_allclose(o[0], ref, rtol=1e-11, atol=1e-12)
    # full square causal through torch's own causal flag: last N rows of a causal pass
    keys_as_queries = np.zeros((w.H, T, Q.shape[2]))
    keys_as_queries[:, L:] = Q
    qt = torch.from_numpy(keys_as_queries)
    kt = torch.from_numpy(K).unsqueeze(0).expand(w.H, -1, -1)
    vt = torch.from_numpy(V).unsqueeze(0).expand(w.H, -1, -1)
    full = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale).numpy()
    np.testing.assert_allclose(o[0], full[:, L:].transpose(1, 0, 2), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("L", [0, 5, 300])
def test_single_node_equals_decode(L):
    """N = 1: the root alone is plain decode attention over L + 1 keys."""
    w = make_workload(B=1, N=1, H=5, Dl=24, Dr=8, dtype="f32", std=1.0, scale=0.3,
                      prefix=("fixed", L), tree=("chain",), seed=7 + L)
    _, _, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    K = np.concatenate([np.concatenate([c, ct[0]]), np.concatenate([r, rt[0]])], axis=1)
    V = np.concatenate([c, ct[0]])
    Q = np.concatenate([q[0, 0], qr[0, 0]], axis=1)[:, None, :]               # [H, 1, d]
    ref = sdpa(Q, K, V, None, w.scale)[:, 0]
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], torch_lse(w.scale * (Q[:, 0] @ K.T), None), rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_each_node_equals_causal_over_its_path(seed):
    """Node i's output is the last row of causal attention over prefix ++ path(root -> i)."""
    w = small(seed, B=1, N=16, L=(11,), tree=("bounded", 5, 3))
    _, depth, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    for i in range(w.N):
        path = [i]
        while w.parents[0, path[-1]] != -1:
            path.append(int(w.parents[0, path[-1]]))
        path = path[::-1]
        K = np.concatenate([np.concatenate([c, ct[0, path]]), np.concatenate([r, rt[0, path]])], axis=1)
        V = np.concatenate([c, ct[0, path]])
        Q = np.concatenate([q[0, i], qr[0, i]], axis=1)[:, None, :]
        ref = sdpa(Q, K, V, None, w.scale)[:, 0]
        np.testing.assert_allclose(o[0, i], ref, rtol=1e-11, atol=1e-12)
        assert len(path) == depth[0, i] + 1


def test_dense_minus_inf_mask_form():
    """Scores over all L+N keys with -inf on invisible tree keys give the same result."""
    w = small(3, B=2, N=24, L=(7, 13), tree=("uniform",))
    mask, _, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    for b in range(w.B):
        s0, s1 = int(w.prefix_offsets[b]), int(w.prefix_offsets[b + 1])
        C = np.concatenate([c[s0:s1], ct[b]])
        R = np.concatenate([r[s0:s1], rt[b]])
        vis = closure_visibility(w.parents[b])
        for h in range(w.H):
            S = w.scale * (q[b, :, h] @ C.T + qr[b, :, h] @ R.T)
            S[:, s1 - s0:][~vis] = -np.inf
            P = torch.softmax(torch.from_numpy(S), dim=1).numpy()
            np.testing.assert_allclose(o[b, :, h], P @ C, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, h], torch.logsumexp(torch.from_numpy(S), 1).numpy(), rtol=1e-12)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_zero_query_closed_form():
    """q = 0: uniform weights, lse = ln(L + depth + 1), o = mean of the visible latent rows."""
    w = small(5, B=2, N=10, L=(4, 0), tree=("uniform",))
    mask, depth, _, _ = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    o, lse = verify_attn_ref(np.zeros_like(q), np.zeros_like(qr), c, r, w.prefix_offsets, ct, rt, mask, w.scale)
    for b in range(w.B):
        s0, s1 = int(w.prefix_offsets[b]), int(w.prefix_offsets[b + 1])
        vis = closure_visibility(w.parents[b])
        for i in range(w.N):
            n_keys = (s1 - s0) + depth[b, i] + 1
            np.testing.assert_allclose(lse[b, i], math.log(n_keys), rtol=0, atol=1e-14)
            rows = np.concatenate([c[s0:s1], ct[b, vis[i]]])
            np.testing.assert_allclose(o[b, i], np.broadcast_to(rows.mean(axis=0), o[b, i].shape), atol=1e-14)


def test_constant_value_rows_give_that_row():
    w = small(6, B=1, N=9, L=(20,))
    mask, _, _, _ = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    v = np.linspace(-2, 3, w.Dl)
    c2 = np.broadcast_to(v, c.shape).copy()
    ct2 = np.broadcast_to(v, ct.shape).copy()
    # scores then depend on r only; the output must still be v exactly (up to rounding)
    o, _ = verify_attn_ref(q, qr, c2, r, w.prefix_offsets, ct2, rt, mask, w.scale)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=1e-13)


def test_dominant_key_selects_its_row():
    """One key with a score far above the rest: o is that key's latent row, lse its score."""
    w = small(7, B=1, N=6, L=(15,), tree=("chain",))
    mask, _, _, _ = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    r = r * 0.0
    rt = rt * 0.0
    qr = np.ones_like(qr)
    j = 9
    r[j] = 1000.0 / (w.scale * w.Dr)              # rope score of key j = 1000
    o, lse = verify_attn_ref(np.zeros_like(q), qr, c, r, w.prefix_offsets, ct, rt, mask, w.scale)
    np.testing.assert_allclose(o, np.broadcast_to(c[j], o.shape), atol=1e-12)
    np.testing.assert_allclose(lse, 1000.0, atol=1e-9)


def test_prefix_row_order_is_irrelevant():
    w = small(8, B=1, N=7, L=(30,))
    mask, _, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    perm = np.random.default_rng(0).permutation(30)
    o2, lse2 = verify_attn_ref(q, qr, c[perm], r[perm], w.prefix_offsets, ct, rt, mask, w.scale)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


@pytest.mark.parametrize("cut", [0, 1, 13, 29, 30])
def test_split_merge_identity(cut):
    """Partials over a partition of the keys merge by the log-sum-exp weights to the whole."""
    w = small(9, B=1, N=11, L=(30,), tree=("uniform",))
    mask, _, o, lse = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    no_tree = np.zeros_like(mask)
    # part 1: prefix rows [0, cut) and no tree nodes; part 2: rows [cut, L) and the tree
    o2, l2 = verify_attn_ref(q, qr, c[cut:], r[cut:], np.array([0, 30 - cut]), ct, rt, mask, w.scale)
    if cut == 0:                  # part 1 is empty: part 2 is the whole key set
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
        return
    o1, l1 = verify_attn_ref(q, qr, c[:cut], r[:cut], np.array([0, cut]), ct, rt, no_tree, w.scale)
    lm = np.logaddexp(l1, l2)
    om = np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2
    np.testing.assert_allclose(lm, lse, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(om, o, rtol=1e-11, atol=1e-13)


def test_scale_zero_is_uniform():
    w = small(10, B=1, N=5, L=(6,))
    mask, depth, _, _ = run_oracle(w)
    q, qr, c, r, ct, rt = f64_case(w)
    o0, l0 = verify_attn_ref(q, qr, c, r, w.prefix_offsets, ct, rt, mask, 0.0)
    oz, lz = verify_attn_ref(0 * q, 0 * qr, c, r, w.prefix_offsets, ct, rt, mask, w.scale)
    np.testing.assert_allclose(o0, oz, atol=1e-14)
    np.testing.assert_allclose(l0, lz, atol=1e-14)


# ----------------------------------------------------------------------------
# greedy accept
# ----------------------------------------------------------------------------

def accept_by_propagation(tstar, tokens, parents):
    """O(N) form: valid[i] = valid[parent] and token matches; deepest valid node, smallest index."""
    B, N = tokens.shape
    out = []
    for b in range(B):
        valid = np.zeros(N, bool)
        d = np.zeros(N, int)
        valid[0] = True
        for i in range(1, N):
            p = parents[b, i]
            d[i] = d[p] + 1
            valid[i] = valid[p] and tokens[b, i] == tstar[b, p]
        cand = np.nonzero(valid)[0]
        term = int(cand[np.argmax(d[cand])])          # first maximum -> smallest index
        path = [term]
        while parents[b, path[-1]] != -1:
            path.append(int(parents[b, path[-1]]))
        out.append((d[term], path[::-1]))
    return out


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("p_match", [0.0, 0.5, 0.9, 1.0])
def test_accept_brute_force_equals_propagation(seed, p_match):
    w = make_workload(B=3, N=24, H=1, Dl=1, Dr=1, dtype="f32", std=1.0, scale=1.0, prefix=("fixed", 0),
                      tree=("uniform",) if seed % 2 else ("bounded", 6, 3), V=50, p_match=p_match, seed=seed)
    tstar, alen, nodes, commit = greedy_accept_ref(w.logits, w.tokens, w.parents)
    for b, (d, path) in enumerate(accept_by_propagation(tstar, w.tokens, w.parents)):
        assert alen[b] == d
        assert nodes[b, :d + 1].tolist() == path and (nodes[b, d + 1:] == -1).all()
        assert commit[b, :d].tolist() == [int(w.tokens[b, k]) for k in path[1:]]
        assert commit[b, d] == tstar[b, path[-1]] and (commit[b, d + 1:] == -1).all()


def test_planted_winner_is_the_argmax():
    w = make_config(2)
    assert np.array_equal(target_argmax_ref(w.logits), w.winners)


def test_chain_fully_matched_commits_block():
    w = make_config(1)
    tstar, alen, nodes, commit = greedy_accept_ref(w.logits, w.tokens, w.parents)
    assert alen.tolist() == [7]
    assert nodes[0].tolist() == list(range(8))
    assert commit[0].tolist() == [int(t) for t in w.tokens[0, 1:]] + [int(tstar[0, 7])]


def test_pages_chain8_golden():
    """Block size 8 with a drafter that always proposes the target's choice: 8 tokens per
    verify step, 24 tokens in 3 steps (golden values printed on the pages)."""
    with open(os.path.join(GOLDEN, "pages_chain8_block.json")) as f:
        g = json.load(f)
    committed = 0
    steps = 0
    for step in range(g["verify_steps"]):
        w = make_workload(B=1, N=g["block_size"], H=1, Dl=1, Dr=1, dtype="f32", std=1.0, scale=1.0,
                          prefix=("fixed", 0), tree=("chain",), V=g["vocab"], p_match=1.0, seed=1000 + step)
        _, alen, _, commit = greedy_accept_ref(w.logits, w.tokens, w.parents)
        committed += int((commit[0] >= 0).sum())
        steps += 1
        assert alen[0] + 1 == g["tokens_per_verify_step"]
    assert committed == g["tokens_generated"] and steps == g["verify_steps"]


def test_accept_single_node_is_greedy_decode():
    logits = np.array([[[0.1, 3.0, -1.0, 2.9]]], np.float32)
    tstar, alen, nodes, commit = greedy_accept_ref(logits, np.array([[2]]), np.array([[-1]]))
    assert alen.tolist() == [0] and nodes.tolist() == [[0]] and commit.tolist() == [[1]]


def test_accept_all_mismatched():
    w = make_workload(B=2, N=10, H=1, Dl=1, Dr=1, dtype="f32", std=1.0, scale=1.0, prefix=("fixed", 0),
                      tree=("uniform",), V=40, p_match=0.0, seed=3)
    tstar, alen, nodes, commit = greedy_accept_ref(w.logits, w.tokens, w.parents)
    assert alen.tolist() == [0, 0]
    assert (nodes[:, 0] == 0).all() and (nodes[:, 1:] == -1).all()
    assert commit[:, 0].tolist() == tstar[:, 0].tolist() and (commit[:, 1:] == -1).all()


def test_argmax_ties_pick_lowest_index():
    logits = np.zeros((1, 3, 6), np.float32)
    logits[0, 0, [2, 4]] = 5.0
    logits[0, 1, :] = -np.inf
    logits[0, 2, [5, 1, 3]] = [1.0, 1.0, 1.0]
    assert target_argmax_ref(logits).tolist() == [[2, 0, 1]]


def test_duplicate_matching_siblings_longest_then_smallest():
    #        0
    #      / | \
    #     1  2  3          tokens of 1, 2, 3 all equal argmax(0) = 7
    #     |  |  |
    #     4  5  6          4 and 6 match their parents; 5 does not
    #        |
    #        7             (child of 5, matches, but 5 is rejected)
    parents = np.array([[-1, 0, 0, 0, 1, 2, 3, 5]], np.int32)
    V = 10
    logits = np.zeros((1, 8, V), np.float32)
    am = [7, 2, 3, 4, 9, 6, 8, 1]
    for i, a in enumerate(am):
        logits[0, i, a] = 1.0
    tokens = np.array([[0, 7, 7, 7, 2, 0, 4, 6]], np.int32)
    tstar, alen, nodes, commit = greedy_accept_ref(logits, tokens, parents)
    assert tstar[0].tolist() == am
    assert alen.tolist() == [2]
    assert nodes[0].tolist() == [0, 1, 4, -1, -1, -1, -1, -1]    # 0-1-4 and 0-3-6 tie: smallest terminal
    assert commit[0].tolist() == [7, 2, 9, -1, -1, -1, -1, -1]


def test_longer_branch_beats_earlier_sibling():
    # 0 -> 1 (match, leaf); 0 -> 2 (match) -> 3 (match): the longer path through 2 wins
    parents = np.array([[-1, 0, 0, 2]], np.int32)
    logits = np.zeros((1, 4, 5), np.float32)
    for i, a in enumerate([3, 0, 1, 2]):
        logits[0, i, a] = 1.0
    tokens = np.array([[4, 3, 3, 1]], np.int32)
    _, alen, nodes, commit = greedy_accept_ref(logits, tokens, parents)
    assert alen.tolist() == [2]
    assert nodes[0].tolist() == [0, 2, 3, -1]
    assert commit[0].tolist() == [3, 1, 2, -1]


# ----------------------------------------------------------------------------
# KV-cache compaction after acceptance
# ----------------------------------------------------------------------------

def accepted_workload(seed, B=3, N=20, L=(7, 0, 12), p_match=0.8, tree=("bounded", 6, 3)):
    w = make_workload(B=B, N=N, H=2, Dl=8, Dr=4, dtype="f32", std=1.0, scale=0.4, prefix=("list", list(L)),
                      tree=tree, V=40, p_match=p_match, seed=seed)
    _, alen, nodes, _ = greedy_accept_ref(w.logits, w.tokens, w.parents)
    return w, alen, nodes


def cache_with_room(w, extra):
    """Per-request cache regions [L_b + extra rows]; returns (c, r, dest_rows) with the prefix copied in."""
    kv = w.f32("kv").astype(np.float64)
    starts, rows = [], 0
    for b in range(w.B):
        starts.append(rows)
        rows += int(w.prefix_lens[b]) + extra
    c = np.full((rows, w.Dl), np.nan)
    r = np.full((rows, w.Dr), np.nan)
    for b in range(w.B):
        s0, L = int(w.prefix_offsets[b]), int(w.prefix_lens[b])
        c[starts[b]:starts[b] + L] = kv[s0:s0 + L, :w.Dl]
        r[starts[b]:starts[b] + L] = kv[s0:s0 + L, w.Dl:]
    dest = np.array([starts[b] + int(w.prefix_lens[b]) for b in range(w.B)], np.int64)
    return c, r, dest


@pytest.mark.parametrize("seed", range(4))
def test_compaction_rows_sit_at_their_positions(seed):
    """Cache position L_b + k holds the accepted node whose build_mask position is L_b + k (depth k)."""
    w, alen, nodes = accepted_workload(seed)
    _, _, pos, _ = build_mask_ref(w.parents, w.prefix_lens)
    kt = w.f32("kv_tree").astype(np.float64)
    c, r, dest = cache_with_room(w, w.N)
    compact_kv_ref(kt[..., :w.Dl], kt[..., w.Dl:], alen, nodes, c, r, dest)
    for b in range(w.B):
        by_pos = {int(pos[b, i]): i for i in range(w.N) if i in set(nodes[b, :alen[b] + 1].tolist())}
        for k in range(alen[b] + 1):
            i = by_pos[int(w.prefix_lens[b]) + k]
            np.testing.assert_array_equal(c[dest[b] + k], kt[b, i, :w.Dl])
            np.testing.assert_array_equal(r[dest[b] + k], kt[b, i, w.Dl:])
        assert np.isnan(c[dest[b] + alen[b] + 1:dest[b] + w.N]).all()      # nothing past the path
        s0 = dest[b] - int(w.prefix_lens[b])
        kv = w.f32("kv").astype(np.float64)
        o0 = int(w.prefix_offsets[b])
        np.testing.assert_array_equal(c[s0:dest[b]], kv[o0:o0 + int(w.prefix_lens[b]), :w.Dl])   # prefix untouched


@pytest.mark.parametrize("seed", range(4))
def test_compacted_cache_reproduces_verify_attention(seed):
    """For every accepted node i at depth k, plain causal attention of i's query over the compacted cache
    rows up to position L_b + k equals the tree-verify attention of node i (the cache carries the path)."""
    w, alen, nodes = accepted_workload(seed)
    _, _, o, lse = run_oracle(w)
    q, qr, _, _, ct, rt = f64_case(w)
    c, r, dest = cache_with_room(w, w.N)
    compact_kv_ref(ct, rt, alen, nodes, c, r, dest)
    for b in range(w.B):
        start = dest[b] - int(w.prefix_lens[b])
        for k in range(alen[b] + 1):
            i = int(nodes[b, k])
            end = dest[b] + k + 1
            K = np.concatenate([c[start:end], r[start:end]], axis=1)
            Q = np.concatenate([q[b, i], qr[b, i]], axis=1)[:, None, :]
            ref = sdpa(Q, K, c[start:end], None, w.scale)[:, 0]
            np.testing.assert_allclose(o[b, i], ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], torch_lse(w.scale * (Q[:, 0] @ K.T), None), rtol=1e-12)


def test_compaction_in_place_equals_separate_buffers():
    """Tree rows stored in the cache right after each prefix (in place) give the same cache as separate
    tree buffers; the path 0 -> 2 -> 3 -> 4 makes row 2 both a source (depth 1) and a destination (depth 2)."""
    N, Dl, Dr = 6, 5, 3
    parents = np.array([[-1, 0, 0, 2, 3, 0]], np.int32)
    alen = np.array([3], np.int32)
    nodes = np.array([[0, 2, 3, 4, -1, -1]], np.int32)
    rng = np.random.default_rng(0)
    L = 4
    c = rng.standard_normal((L + N, Dl))
    r = rng.standard_normal((L + N, Dr))
    tree_c, tree_r = c[L:].copy()[None], r[L:].copy()[None]
    c_sep, r_sep = c.copy(), r.copy()
    compact_kv_ref(tree_c, tree_r, alen, nodes, c_sep, r_sep, np.array([L]))
    c_in, r_in = c.copy(), r.copy()
    compact_kv_ref(c_in[L:][None], r_in[L:][None], alen, nodes, c_in, r_in, np.array([L]))   # views of the cache
    np.testing.assert_array_equal(c_in[:L + 4], c_sep[:L + 4])
    np.testing.assert_array_equal(r_in[:L + 4], r_sep[:L + 4])
    np.testing.assert_array_equal(c_sep[L:L + 4], tree_c[0, [0, 2, 3, 4]])
    assert parents[0, 2] == 0 and parents[0, 3] == 2 and parents[0, 4] == 3


def test_compaction_edge_cases():
    """accept_len 0 moves only the root; a negative dest row leaves the request alone; invalid node
    entries are skipped; a fully accepted chain stored in place leaves the cache unchanged."""
    N, Dl, Dr = 4, 3, 2
    rng = np.random.default_rng(1)
    tree_c, tree_r = rng.standard_normal((3, N, Dl)), rng.standard_normal((3, N, Dr))
    c, r = np.zeros((12, Dl)), np.zeros((12, Dr))
    compact_kv_ref(tree_c, tree_r, np.array([0, 2, 3]), np.array([[0, -1, -1, -1], [0, 9, 1, -1], [0, 1, 2, 3]]),
                   c, r, np.array([1, 6, -1]))
    np.testing.assert_array_equal(c[1], tree_c[0, 0])
    np.testing.assert_array_equal(c[6], tree_c[1, 0])
    np.testing.assert_array_equal(c[8], tree_c[1, 1])
    np.testing.assert_array_equal(r[8], tree_r[1, 1])
    assert not c[[0, 2, 3, 4, 5, 7, 9, 10, 11]].any()
    c2 = rng.standard_normal((3 + N, Dl))
    r2 = rng.standard_normal((3 + N, Dr))
    before_c, before_r = c2.copy(), r2.copy()
    compact_kv_ref(c2[3:][None], r2[3:][None], np.array([N - 1]), np.arange(N, dtype=np.int32)[None], c2, r2,
                   np.array([3]))
    np.testing.assert_array_equal(c2, before_c)
    np.testing.assert_array_equal(r2, before_r)


# ----------------------------------------------------------------------------
# best-first draft-tree builder
# ----------------------------------------------------------------------------

def all_candidate_nodes(cand_tokens, cand_logp):
    """Every node of the candidate tree of one request, by enumeration: (key, path of ranks, tokens, score),
    with the float32 score summed root to leaf."""
    D, K = cand_tokens.shape
    out = []

    def rec(ranks, score, parent_key):
        d = len(ranks)
        if d == D:
            return
        for j in range(K):
            sc = np.float32(score + cand_logp[d, j])
            path = ranks + [j]
            out.append((sc, path))
            rec(path, sc, None)

    rec([], np.float32(0.0), None)
    return out


def topk_by_definition(cand_tokens, cand_logp, N):
    """Root plus the N-1 best candidate nodes under the key (score desc, depth, parent node, rank).  The
    parent node index is the parent's own position in that order, so rank the nodes level by level."""
    nodes = all_candidate_nodes(cand_tokens, cand_logp)
    chosen = {(): 0}                   # rank path -> node index
    order = []
    remaining = list(nodes)
    while len(order) < N - 1:
        # the best node whose parent is already chosen (the only ones the key can rank next)
        best = None
        for sc, path in remaining:
            par = tuple(path[:-1])
            if par not in chosen:
                continue
            key = (-sc, len(path), chosen[par], path[-1])
            if best is None or key < best[0]:
                best = (key, sc, path)
        key, sc, path = best
        chosen[tuple(path)] = len(order) + 1
        order.append((chosen[tuple(path[:-1])], int(cand_tokens[len(path) - 1, path[-1]]), len(path), sc))
        remaining = [(x, p) for x, p in remaining if p != path]
    return order


@pytest.mark.parametrize("seed,D,K,N", [(0, 3, 3, 12), (1, 4, 2, 20), (2, 2, 5, 25), (3, 5, 3, 40), (4, 3, 4, 2)])
def test_tree_builder_equals_ranked_enumeration(seed, D, K, N):
    """The heap build equals ranking every candidate node of the (tiny) candidate tree by the key."""
    c = make_draft_candidates(B=2, D=D, K=K, V=60, seed=seed)
    parents, tokens, depth, scores = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, N)
    for b in range(2):
        ref = topk_by_definition(c.cand_tokens[b], c.cand_logp[b], N)
        got = [(int(parents[b, n]), int(tokens[b, n]), int(depth[b, n]), scores[b, n]) for n in range(1, N)]
        assert got == ref
        assert tokens[b, 0] == c.root_tokens[b] and parents[b, 0] == -1 and depth[b, 0] == 0


def test_tree_builder_ties_follow_the_key():
    """Log-probabilities on a coarse grid make many equal scores; the order is still the key's."""
    c = make_draft_candidates(B=3, D=4, K=3, V=40, seed=9, tie_step=0.5)
    parents, tokens, depth, scores = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, 30)
    assert len(set(np.round(scores[0], 6))) < 30                # ties do occur
    for b in range(3):
        ref = topk_by_definition(c.cand_tokens[b], c.cand_logp[b], 30)
        assert [(int(parents[b, n]), int(tokens[b, n]), int(depth[b, n]), scores[b, n]) for n in range(1, 30)] == ref


def test_tree_builder_single_proposal_is_a_chain():
    c = make_draft_candidates(B=2, D=8, K=1, V=100, seed=3)
    parents, tokens, depth, scores = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, 9)
    for b in range(2):
        assert parents[b].tolist() == chain_tree(9).tolist()
        assert tokens[b, 1:].tolist() == c.cand_tokens[b, :, 0].tolist()
        assert depth[b].tolist() == list(range(9))
        np.testing.assert_allclose(scores[b, 1:], np.cumsum(c.cand_logp[b, :, 0], dtype=np.float64), rtol=1e-6)


def test_tree_builder_oracle_drafter_block_of_8():
    """An "oracle drafter" (golden token at rank 0 with probability 0.9, distractors far below) over the
    block's block_size - 1 draft depths (node 0 is the last committed token) makes the golden continuation
    nodes 1..7, a chain; the greedy accept of a target that agrees with it takes all of them and commits
    block_size = 8 tokens per verify step, the pages' figure (golden fixture)."""
    golden_doc = json.load(open(os.path.join(GOLDEN, "pages_chain8_block.json")))
    block = int(golden_doc["block_size"])
    D = block - 1
    V = int(golden_doc["vocab"])
    c = make_draft_candidates(B=2, D=D, K=4, V=V, seed=5, golden_p=0.9)
    N = 24
    parents, tokens, depth, _ = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, N)
    for b in range(2):
        assert parents[b, 1:D + 1].tolist() == list(range(D))
        assert tokens[b, 1:D + 1].tolist() == c.golden[b].tolist()
    # target logits whose argmax at node i is the golden token of depth(i) + 1 (and something else below)
    logits = np.zeros((2, N, V), np.float32)
    for b in range(2):
        for i in range(N):
            logits[b, i, c.golden[b, depth[b, i]] if depth[b, i] < D else 0] = 5.0
    _, alen, nodes, commit = greedy_accept_ref(logits, tokens, parents)
    assert alen.tolist() == [D, D]
    assert nodes[0, :D + 1].tolist() == list(range(D + 1))
    assert ((commit >= 0).sum(axis=1) == golden_doc["tokens_per_verify_step"]).all()


@pytest.mark.parametrize("seed", range(3))
def test_tree_builder_structure(seed):
    c = make_draft_candidates(B=4, D=6, K=4, V=500, seed=seed)
    parents, tokens, depth, scores = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, 64)
    for b in range(4):
        assert tree_is_valid_np(parents[b])
        for n in range(1, 64):
            p = parents[b, n]
            assert depth[b, n] == depth[b, p] + 1
            assert tokens[b, n] in set(c.cand_tokens[b, depth[b, n] - 1].tolist())
            assert scores[b, n] <= scores[b, p]
        kids = {}
        for n in range(1, 64):
            kids.setdefault(int(parents[b, n]), []).append(int(tokens[b, n]))
        assert all(len(v) == len(set(v)) for v in kids.values())        # siblings carry distinct tokens
        _, dep, _, ok = build_mask_ref(parents[b:b + 1], None)
        assert ok[0] == 1 and (dep[0] == depth[b]).all()


def level_order_scores(cand_logp):
    """float32 scores of every node of a request's candidate tree, level by level (a node's score is
    its parent's plus the proposal's log-probability), with the depth of each."""
    D, K = cand_logp.shape
    level = np.zeros(1, np.float32)
    scores, depths = [], []
    for d in range(D):
        level = (level[:, None] + cand_logp[d][None, :]).reshape(-1)      # float32 additions
        scores.append(level)
        depths.append(np.full(level.shape, d + 1))
    return np.concatenate(scores), np.concatenate(depths)


@pytest.mark.parametrize("seed,D,K,N", [(0, 8, 3, 256), (1, 7, 4, 128), (2, 4, 8, 200), (3, 3, 16, 256),
                                        (4, 12, 2, 128)])
def test_tree_builder_takes_the_best_of_the_whole_candidate_tree(seed, D, K, N):
    """With log-probabilities <= 0, the N-1 taken nodes are the N-1 best (score descending, then depth) of
    the whole candidate tree, enumerated level by level and sorted; so the taken scores and depths, in
    order, equal that sorted list's head.  Sizes up to 256 nodes, depth 12, 16 proposals."""
    c = make_draft_candidates(B=2, D=D, K=K, V=4000, seed=seed)
    _, _, depth, scores = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, N)
    for b in range(2):
        all_s, all_d = level_order_scores(c.cand_logp[b])
        order = np.lexsort((all_d, -all_s.astype(np.float64)))[:N - 1]
        np.testing.assert_array_equal(scores[b, 1:], all_s[order])
        np.testing.assert_array_equal(depth[b, 1:], all_d[order])


def tree_is_valid_np(p):
    return p[0] == -1 and all(0 <= p[i] < i for i in range(1, len(p)))


def test_tree_builder_rejects_too_small_candidate_trees():
    c = make_draft_candidates(B=1, D=2, K=2, V=10, seed=0)
    build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, 7)        # 1 + 2 + 4 nodes exist
    with pytest.raises(ValueError):
        build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, 8)


# ----------------------------------------------------------------------------
# NeoX rotary embedding at tree positions
# ----------------------------------------------------------------------------

def test_rope_hand_cases():
    """A 2-vector turns counterclockwise by the angle; NeoX pairs element i with i + Dr/2 (not 2i, 2i+1)."""
    for p in (0, 1, 7, 123456789012):
        out = rope_neox_ref(np.array([1.0, 0.0]), np.int64(p), np.array([1.0]))
        assert out.tolist() == [math.cos(float(p)), math.sin(float(p))]
    f = np.array([0.5, 0.25])
    out = rope_neox_ref(np.array([1.0, 0.0, 0.0, 0.0]), np.int64(3), f)
    assert out.tolist() == [math.cos(1.5), 0.0, math.sin(1.5), 0.0]
    out = rope_neox_ref(np.array([0.0, 0.0, 0.0, 1.0]), np.int64(3), f)
    assert out.tolist() == [0.0, -math.sin(0.75), 0.0, math.cos(0.75)]
    inv = rope_inv_freq(8, 10000.0)
    assert inv.tolist() == [1.0, 10000.0 ** -0.25, 10000.0 ** -0.5, 10000.0 ** -0.75]


def test_rope_identity_norms_composition_and_relative_position():
    rng = np.random.default_rng(0)
    Dr = 64
    inv = rope_inv_freq(Dr, 10000.0)
    x = rng.standard_normal((5, Dr))
    pos = np.array([0, 1, 17, 4096, 131072 + 11], np.int64)
    np.testing.assert_array_equal(rope_neox_ref(x, np.zeros(5, np.int64), inv), x)
    y = rope_neox_ref(x, pos, inv)
    h = Dr // 2
    np.testing.assert_allclose(y[:, :h] ** 2 + y[:, h:] ** 2, x[:, :h] ** 2 + x[:, h:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(rope_neox_ref(rope_neox_ref(x, pos, inv), 3 * pos, inv), rope_neox_ref(x, 4 * pos, inv),
                               rtol=1e-9, atol=1e-9)
    q, k = rng.standard_normal(Dr), rng.standard_normal(Dr)
    for pq, pk in [(5, 2), (131083, 131072), (100, 100)]:
        lhs = rope_neox_ref(q, np.int64(pq), inv) @ rope_neox_ref(k, np.int64(pk), inv)
        rhs = rope_neox_ref(q, np.int64(pq - pk), inv) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_rope_at_tree_positions_makes_verify_shift_invariant():
    """Rotating the prefix keys at 0..L-1 and the tree queries and keys at L + depth, then verifying, gives
    the same outputs when every position is shifted by a constant: only relative positions matter."""
    w = small(3, B=2, N=12, L=(5, 9), tree=("bounded", 4, 3))
    mask, depth, pos, _ = build_mask_ref(w.parents, w.prefix_lens)
    q, qr, c, r, ct, rt = f64_case(w)
    inv = rope_inv_freq(w.Dr, 10000.0)
    outs = []
    for shift in (0, 1000):
        rp = np.concatenate([rope_neox_ref(r[w.prefix_offsets[b]:w.prefix_offsets[b + 1]],
                                           np.arange(w.prefix_lens[b]) + shift, inv) for b in range(w.B)])
        qrr = rope_neox_ref(qr, (pos + shift)[:, :, None], inv)
        rtr = rope_neox_ref(rt, pos + shift, inv)
        outs.append(verify_attn_ref(q, qrr, c, rp, w.prefix_offsets, ct, rtr, mask, w.scale))
    np.testing.assert_allclose(outs[0][0], outs[1][0], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(outs[0][1], outs[1][1], rtol=1e-11)
