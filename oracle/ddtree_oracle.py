"""Plain CPU oracle for DDTree tree verification (test infrastructure only).

This module is the correctness reference for the GPU library.  It is test
infrastructure: only the test suite, the smoke check and the benchmark's CPU
baseline leg import it.  The product path never calls it, and it shares no
code with the HIP kernels or their host library.  Everything is computed in
float64 with NumPy, in the most direct form of each definition: no online
softmax, no tiling, no bitmask tricks beyond storing the mask.

Pages cited (titles of the source pages):
  [Validating] "The Moment of Proof: Validating a Native CUDA Speculative Decoding Engine"
  [Running]    "The Moment of Proof: Running the Native DDTree Speculative Decoding Engine"
  [Truth]      "The Moment of Truth: Validating a Custom CUDA Inference Engine for Kimi K2.6"
  [Build]      "The Build That Proved It: Compiling the Native DDTree Speculative Decoding Engine"

What the pages fix, and the readings taken where they are silent:
  * A draft tree is verified in one target forward under a custom attention
    mask; the accepted tokens are those on the longest path whose tokens match
    the target's greedy choices ([Validating] "Input Knowledge Required";
    [Running] "Input Knowledge Required"; [Build] "The Output Knowledge Created").
  * The tree is a parent array, node 0 the root (the last committed token),
    parent[i] < i.  A node sees the cached prefix plus its ancestors and
    itself (reading: ancestor-or-self, so that a single chain is causal).
  * Attention is MLA in absorbed form: scores use the latent query against
    the latent cache row c plus the rotary query against the rotary key r;
    the value is the latent row c itself ([Validating] "Input Knowledge
    Required": the absorb form folds the up-projections into attention).
  * Positions are cache length plus node depth, as int64 ([Build] "The
    Thinking Process Visible in Reasoning").
  * The log-sum-exp is the natural log of the sum of exp of the scaled scores.
  * Greedy accept: a node's draft token is accepted when it equals the
    target's argmax at its parent and its parent is accepted; the longest
    accepted root path wins, ties to the smallest terminal index; the
    commit is the path's draft tokens after the root plus the target's
    argmax at the terminal node (the bonus token).  argmax ties go to the
    lowest vocabulary index (NumPy's argmax).

Every function here is pinned by the CPU tests against closed forms, special
cases that reduce to library routines and brute-force alternatives.
"""
from __future__ import annotations

import numpy as np

__all__ = ["tree_is_valid", "build_mask_ref", "visible_nodes", "verify_attn_ref", "target_argmax_ref",
           "greedy_accept_ref"]


# ----------------------------------------------------------------------------
# Visibility mask, depth and positions
# ----------------------------------------------------------------------------

def tree_is_valid(parent_row: np.ndarray) -> bool:
    """Root first with parent -1, every other parent an earlier node."""
    n = len(parent_row)
    if n == 0 or int(parent_row[0]) != -1:
        return False
    return all(0 <= int(parent_row[i]) < i for i in range(1, n))


def build_mask_ref(parents: np.ndarray, prefix_lens: np.ndarray | None = None):
    """Ancestor-or-self visibility mask of every tree node, by pointer chasing.

    The mask is the custom attention mask of tree verification ([Validating]
    "Input Knowledge Required"; [Validating] "Output Knowledge Created":
    attention mask construction in the live decode loop).  Node depth is the
    number of parent steps to the root; position = cache length + depth,
    int64 ([Build] "The Thinking Process Visible in Reasoning").

    Returns (mask uint32 [B,N,W] with bit k of word k//32 set when node k is
    visible to node i, depth int32 [B,N], positions int64 [B,N],
    tree_ok int32 [B]).  An invalid tree gives mask 0, depth -1,
    position -1 and tree_ok 0 for that request.
    """
    parents = np.asarray(parents)
    B, N = parents.shape
    W = (N + 31) // 32
    if prefix_lens is None:
        prefix_lens = np.zeros(B, dtype=np.int64)
    mask = np.zeros((B, N, W), dtype=np.uint32)
    depth = np.full((B, N), -1, dtype=np.int32)
    positions = np.full((B, N), -1, dtype=np.int64)
    ok = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if not tree_is_valid(parents[b]):
            continue
        ok[b] = 1
        for i in range(N):
            k = i
            steps = 0
            while k != -1:
                mask[b, i, k // 32] |= np.uint32(1 << (k % 32))
                k = int(parents[b, k])
                steps += 1
            depth[b, i] = steps - 1
            positions[b, i] = int(prefix_lens[b]) + steps - 1
    return mask, depth, positions, ok


def visible_nodes(mask_row: np.ndarray, n: int) -> list:
    """Tree node indices whose bit is set in one node's mask words, ascending."""
    return [k for k in range(n) if (int(mask_row[k // 32]) >> (k % 32)) & 1]


# ----------------------------------------------------------------------------
# Tree-verify attention, absorbed MLA form
# ----------------------------------------------------------------------------

def verify_attn_ref(q_lat, q_rope, ckv, krope, prefix_offsets, ckv_tree, krope_tree, mask, scale, nodes=None):
    """Attention of every tree node over the shared prefix plus its visible tree nodes.

    For request b, node i and head h, the key set J is the cached prefix rows
    prefix_offsets[b] .. prefix_offsets[b+1]-1 followed by the tree nodes k
    visible to i (mask bit k).  With c_j the latent row and r_j the rotary key,
        s_j = scale * (q_lat[b,i,h] . c_j + q_rope[b,i,h] . r_j)
        o   = sum_j softmax(s)_j c_j            (the value is the latent row)
        lse = ln sum_j exp(s_j)
    ([Validating] "Input Knowledge Required" for the absorbed MLA form and the
    tree mask; [Running] "Input Knowledge Required": verify attention with
    visibility masking).  Softmax is taken directly: max, exp, sum, divide.

    Arguments are float arrays (converted to float64 here):
      q_lat [B,N,H,Dl], q_rope [B,N,H,Dr], ckv [T,Dl], krope [T,Dr],
      prefix_offsets int [B+1], ckv_tree [B,N,Dl], krope_tree [B,N,Dr],
      mask uint32 [B,N,W].
    nodes: optional list of (b, i) pairs to compute (others stay 0), for
    sampling large workloads; the arithmetic per node is unchanged.
    Returns o float64 [B,N,H,Dl], lse float64 [B,N,H].
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    B, N, H, Dl = q_lat.shape
    o = np.zeros((B, N, H, Dl), dtype=np.float64)
    lse = np.zeros((B, N, H), dtype=np.float64)
    wanted = None if nodes is None else {(int(b), int(i)) for b, i in nodes}
    for b in range(B):
        if wanted is not None and not any(wb == b for wb, _ in wanted):
            continue
        s0, s1 = int(prefix_offsets[b]), int(prefix_offsets[b + 1])
        C_prefix = np.asarray(ckv[s0:s1], dtype=np.float64)
        R_prefix = np.asarray(krope[s0:s1], dtype=np.float64)
        for i in range(N):
            if wanted is not None and (b, i) not in wanted:
                continue
            vis = visible_nodes(mask[b, i], N)
            C = np.concatenate([C_prefix, np.asarray(ckv_tree[b, vis], dtype=np.float64)], axis=0)
            R = np.concatenate([R_prefix, np.asarray(krope_tree[b, vis], dtype=np.float64)], axis=0)
            S = scale * (q_lat[b, i] @ C.T + q_rope[b, i] @ R.T)          # [H, |J|]
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            o[b, i] = (P @ C) / l
            lse[b, i] = m[:, 0] + np.log(l[:, 0])
    return o, lse


# ----------------------------------------------------------------------------
# Greedy tree accept
# ----------------------------------------------------------------------------

def target_argmax_ref(logits) -> np.ndarray:
    """The target's greedy choice per tree node: first index of the maximum logit."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int32)


def greedy_accept_ref(logits, tokens, parents):
    """Longest root path whose draft tokens match the target's greedy choices.

    ([Validating] "Input Knowledge Required": tokens along the longest
    matching path are accepted; [Running] "Input Knowledge Required": greedy
    token acceptance and path selection; [Build] "The Output Knowledge
    Created": the longest prefix matching the target's greedy choices.)

    Brute force: every node defines one root->node path; the path is
    accepted when each non-root node's draft token equals the argmax of its
    parent's logits.  The longest accepted path wins (ties: smallest
    terminal node).  Commit = draft tokens of the path after the root, then
    the terminal node's argmax.

    Returns (target_argmax int32 [B,N], accept_len int32 [B] (drafts
    accepted), accept_nodes int32 [B,N] (root first, -1 padded),
    commit_tokens int32 [B,N] (accept_len+1 entries, -1 padded)).
    """
    tokens = np.asarray(tokens)
    parents = np.asarray(parents)
    B, N = tokens.shape
    tstar = target_argmax_ref(logits)
    accept_len = np.zeros(B, dtype=np.int32)
    accept_nodes = np.full((B, N), -1, dtype=np.int32)
    commit = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        if not tree_is_valid(parents[b]):
            raise ValueError(f"request {b}: not a valid tree")
        best = None
        for t in range(N):
            path = [t]
            while int(parents[b, path[-1]]) != -1:
                path.append(int(parents[b, path[-1]]))
            path.reverse()                      # root ... t
            if all(int(tokens[b, path[k]]) == int(tstar[b, path[k - 1]]) for k in range(1, len(path))):
                if best is None or len(path) > len(best):
                    best = path
        accept_len[b] = len(best) - 1
        accept_nodes[b, :len(best)] = best
        committed = [int(tokens[b, k]) for k in best[1:]] + [int(tstar[b, best[-1]])]
        commit[b, :len(committed)] = committed
    return tstar, accept_len, accept_nodes, commit


# ----------------------------------------------------------------------------
# KV-cache compaction after acceptance
# ----------------------------------------------------------------------------

def compact_kv_ref(ckv_tree, krope_tree, accept_len, accept_nodes, ckv, krope, dest_rows):
    """Move the accepted path's latent rows into the cache, in place.

    ([Validating] "Output Knowledge Created": the engine keeps a KV cache with
    post-verify compaction; [Build] "The Output Knowledge Created": the
    compaction keeps the accepted tokens for the following steps.)

    Reading: the root (node 0, the last committed token) and the accepted
    drafts, in path order, become cache positions L_b .. L_b + accept_len of
    request b; dest_rows[b] is the cache row of position L_b.  The bonus token
    has no latent row yet (it is the next step's root).  Rows are moved one at
    a time in path order: position L_b + k receives node accept_nodes[b, k].
    Because a path's node indices grow with depth, this order is also correct
    when the tree rows live in the cache itself right after the prefix (row
    dest_rows[b] + i holding node i): a row is always read before it is
    overwritten.

    ckv_tree [B, N, Dl] and krope_tree [B, N, Dr] may be views of ckv / krope
    (that in-place layout); ckv [R, Dl] and krope [R, Dr] are updated.
    Entries of accept_nodes outside 0..N-1 are skipped; requests with a
    negative dest row are left alone.
    """
    B, N = np.asarray(accept_nodes).shape
    for b in range(B):
        d0 = int(dest_rows[b])
        if d0 < 0:
            continue
        for k in range(min(int(accept_len[b]), N - 1) + 1):
            s = int(accept_nodes[b, k])
            if not 0 <= s < N:
                continue
            ckv[d0 + k, :] = ckv_tree[b, s, :]
            krope[d0 + k, :] = krope_tree[b, s, :]
    return ckv, krope


# ----------------------------------------------------------------------------
# Best-first draft-tree builder
# ----------------------------------------------------------------------------

def build_tree_ref(root_tokens, cand_tokens, cand_logp, N):
    """Grow each request's draft tree best-first from per-depth drafter proposals.

    (The pages' engine builds the draft tree on the GPU best-first, replacing a
    per-request CPU heap: [Validating] opening and "Output Knowledge
    Created"; [Truth] opening.  They give no further detail; the reading
    below is the plainest one.)

    Reading: depth d (1..D) offers K proposals (token, log-probability).  Any
    node at depth d-1 may take any depth-d proposal as a child; a node's score
    is its parent's score plus the proposal's log-probability (float32, added
    root to leaf), the root scoring 0.  Starting from the root, each step
    looks at every child of every node taken so far that is not taken yet,
    and takes the best one under the key (score descending, then depth,
    parent index and proposal rank ascending), until N nodes exist.  Taken
    nodes are numbered in order, so every parent precedes its children.

    This is the definition written out: every step scans the whole frontier
    (no heap, no lazily grown frontier).  With log-probabilities <= 0 a child
    never outranks its parent, so the result is the root plus the N-1 best
    nodes of the whole candidate tree.

    Returns parents, tokens, depth (int32 [B, N]) and scores (float32 [B, N]).
    """
    root_tokens = np.asarray(root_tokens)
    cand_tokens = np.asarray(cand_tokens)
    cand_logp = np.asarray(cand_logp, dtype=np.float32)
    B, D, K = cand_tokens.shape
    parents = np.full((B, N), -1, np.int32)
    tokens = np.full((B, N), -1, np.int32)
    depth = np.zeros((B, N), np.int32)
    scores = np.zeros((B, N), np.float32)
    for b in range(B):
        tokens[b, 0] = root_tokens[b]
        taken = np.zeros((N, K), dtype=bool)     # taken[p, j]: child j of node p is a node already
        for n in range(1, N):
            # every child (p, j) of the n nodes taken so far: its score, depth, parent and rank
            p_idx = np.repeat(np.arange(n), K)
            j_idx = np.tile(np.arange(K), n)
            p_depth = depth[b, p_idx]
            open_ = (p_depth < D) & ~taken[p_idx, j_idx]
            if not open_.any():
                raise ValueError(f"request {b}: only {n} nodes can be built from {D} depths of {K} proposals")
            p_idx, j_idx, p_depth = p_idx[open_], j_idx[open_], p_depth[open_]
            child = scores[b, p_idx] + cand_logp[b, p_depth, j_idx]       # float32 additions
            # the key's best: highest score, then lowest depth, parent, rank (lexsort: last key first)
            best = np.lexsort((j_idx, p_idx, p_depth, -child.astype(np.float64)))[0]
            p, j = int(p_idx[best]), int(j_idx[best])
            taken[p, j] = True
            parents[b, n] = p
            tokens[b, n] = cand_tokens[b, depth[b, p], j]
            depth[b, n] = depth[b, p] + 1
            scores[b, n] = child[best]
    return parents, tokens, depth, scores


# ----------------------------------------------------------------------------
# NeoX rotary embedding at tree positions
# ----------------------------------------------------------------------------

def rope_inv_freq(Dr, base):
    """Plain rotary frequencies base^(-2i/Dr), i = 0 .. Dr/2 - 1, in float64."""
    return base ** (-np.arange(0, Dr, 2, dtype=np.float64) / Dr)


def rope_neox_ref(x, positions, inv_freq):
    """NeoX-style rotation of the last axis of x at the given positions, in float64.

    (The engine applies NeoX rotary embeddings and computes the angle in
    double precision: [Truth] "What the Output Tells Us"; positions are
    cache length plus node depth, int64: [Build] "The Thinking Process
    Visible in Reasoning".)

    NeoX pairs element i with element i + Dr/2.  With angle
    a_i = position * inv_freq[i]: out[i] = x[i] cos a_i - x[i + Dr/2] sin a_i and
    out[i + Dr/2] = x[i + Dr/2] cos a_i + x[i] sin a_i.

    x: [..., Dr]; positions: broadcastable to x.shape[:-1] (int64); returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[..., None] * np.asarray(inv_freq, dtype=np.float64)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
