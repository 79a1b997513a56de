"""Seeded synthetic workloads for DDTree tree verification.

This module only draws random inputs: draft trees (parent arrays), per-request
prefix lengths, absorbed latent queries, the latent KV cache (c_kv and the
rotary key part), the tree nodes' own latent rows, target logits and draft
tokens.  It performs none of the verification arithmetic (no masks, no scores,
no softmax, no argmax, no path search); both the CPU oracle and the GPU path
receive exactly the arrays made here.

Shapes follow the statement of the problem on the pages ("The Moment of Proof",
sections "Input Knowledge Required": a draft tree verified in one forward with
a custom mask, MLA with its compressed latent KV cache in absorbed form).

Layouts (row-major, C order):
  parents      int32 [B, N]            parent[b,0] = -1 (root), parent[b,i] < i
  prefix_lens  int64 [B]               cached prefix length L_b per request
  prefix_offsets int64 [B+1]           exclusive scan of prefix_lens
  q_lat        [B, N, H, Dl]           absorbed latent query per node and head
  q_rope       [B, N, H, Dr]           rotary query part (already rotated)
  kv           [T, Dl+Dr]              packed prefix cache rows: c_kv | k_rope
  kv_tree      [B, N, Dl+Dr]           the tree nodes' own latent rows
  logits       float32 [B, N, V]       target logits per node (optional)
  tokens       int32 [B, N]            draft token of each node (root: any)
Floating point arrays are float32, or uint16 bfloat16 bit patterns when the
workload dtype is "bf16" (round-to-nearest-even from the float32 draw).

Draw order (fixed, one numpy Generator per workload): tree, prefix lengths,
q_lat, q_rope, prefix c_kv, prefix k_rope, tree c_kv, tree k_rope, logits,
planted winners, planted winner values, root tokens, match coin flips,
mismatch tokens.

Logits: N(0,1), except that every row has one planted winner index whose
value is set to 8 + U(0,1).  Draft tokens copy the parent's planted winner
with the workload's match probability, else a uniform other token.  The
planted winner lets the generator make drafts that match the parent's
argmax with a chosen probability without computing any argmax; the argmax
itself is computed independently by each side (a normal draw above 8 has
probability ~6e-16, so the planted entry is the row's maximum in practice).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PLANT_BASE = 8.0


# ----------------------------------------------------------------------------
# bfloat16 bit handling (a storage conversion, not part of the method)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; returns uint16 bits.

    Inputs are finite draws; NaN payloads are not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """float32 view of a workload array regardless of its storage dtype."""
    return bf16_to_f32(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float32)


# ----------------------------------------------------------------------------
# Trees
# ----------------------------------------------------------------------------

def chain_tree(n: int) -> np.ndarray:
    """parent[i] = i - 1: a single draft path (block of n tokens)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def uniform_tree(rng: np.random.Generator, n: int) -> np.ndarray:
    """parent[i] uniform over the earlier nodes [0, i); node 0 is the root."""
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def bounded_tree(rng: np.random.Generator, n: int, max_depth: int, max_branch: int) -> np.ndarray:
    """parent[i] uniform over earlier nodes with depth < max_depth and < max_branch children."""
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    depth = np.zeros(n, dtype=np.int64)
    children = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        eligible = np.nonzero((depth[:i] < max_depth) & (children[:i] < max_branch))[0]
        if eligible.size == 0:
            raise ValueError("tree bounds leave no eligible parent")
        k = int(eligible[rng.integers(0, eligible.size)])
        p[i] = k
        depth[i] = depth[k] + 1
        children[k] += 1
    return p


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    B: int
    N: int
    H: int
    Dl: int
    Dr: int
    scale: float
    parents: np.ndarray
    prefix_lens: np.ndarray
    prefix_offsets: np.ndarray
    q_lat: np.ndarray
    q_rope: np.ndarray
    kv: np.ndarray
    kv_tree: np.ndarray
    logits: Optional[np.ndarray] = None
    tokens: Optional[np.ndarray] = None
    winners: Optional[np.ndarray] = None
    V: int = 0

    @property
    def T(self) -> int:
        return int(self.prefix_offsets[-1])

    # float32 views (exact for bf16 storage)
    def f32(self, name: str) -> np.ndarray:
        return to_f32(getattr(self, name), self.dtype)


# The five reference workloads.  Sizes and distributions follow the
# configurations this path is specified on; scale is the caller's softmax
# scale (1/sqrt of the unabsorbed q.k head width).
CONFIGS = {
    1: dict(name="tiny-chain", B=1, N=8, H=4, Dl=64, Dr=32, dtype="f32", std=1.0,
            scale=1.0 / math.sqrt(96.0), prefix=("fixed", 8), tree=("chain",), V=512, p_match=1.0),
    2: dict(name="small-random-trees", B=4, N=32, H=4, Dl=64, Dr=32, dtype="f32", std=1.0,
            scale=1.0 / math.sqrt(96.0), prefix=("fixed", 512), tree=("uniform",), V=512, p_match=0.7),
    3: dict(name="k2-single", B=1, N=64, H=64, Dl=512, Dr=64, dtype="bf16", std=0.5,
            scale=1.0 / math.sqrt(192.0), prefix=("fixed", 4096), tree=("bounded", 8, 4), V=0, p_match=0.0),
    4: dict(name="k2-batched-ragged", B=16, N=64, H=64, Dl=512, Dr=64, dtype="bf16", std=0.5,
            scale=1.0 / math.sqrt(192.0), prefix=("uniform", 1024, 32768), tree=("bounded", 8, 4), V=0,
            p_match=0.0),
    5: dict(name="k2-long-context-accept", B=4, N=128, H=64, Dl=512, Dr=64, dtype="bf16", std=0.5,
            scale=1.0 / math.sqrt(192.0), prefix=("fixed", 131072), tree=("bounded", 12, 4), V=163840,
            p_match=0.8),
}


def _draw_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_workload(*, B: int, N: int, H: int, Dl: int, Dr: int, dtype: str, std: float, scale: float,
                  prefix, tree, V: int = 0, p_match: float = 0.0, seed: int = 0,
                  name: str = "custom") -> Workload:
    """Draw one workload.

    prefix: ("fixed", L) | ("uniform", lo, hi) | ("list", [L_0, ..., L_{B-1}])
    tree:   ("chain",) | ("uniform",) | ("bounded", max_depth, max_branch) | ("given", parents[B,N])
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)

    # 1. trees
    kind = tree[0]
    if kind == "chain":
        parents = np.stack([chain_tree(N) for _ in range(B)]) if B else np.zeros((0, N), np.int32)
    elif kind == "uniform":
        parents = np.stack([uniform_tree(rng, N) for _ in range(B)]) if B else np.zeros((0, N), np.int32)
    elif kind == "bounded":
        parents = (np.stack([bounded_tree(rng, N, tree[1], tree[2]) for _ in range(B)])
                   if B else np.zeros((0, N), np.int32))
    elif kind == "given":
        parents = np.asarray(tree[1], dtype=np.int32).reshape(B, N).copy()
    else:
        raise ValueError(kind)
    parents = np.ascontiguousarray(parents, dtype=np.int32)

    # 2. prefix lengths
    pk = prefix[0]
    if pk == "fixed":
        lens = np.full(B, int(prefix[1]), dtype=np.int64)
    elif pk == "uniform":
        lens = rng.integers(int(prefix[1]), int(prefix[2]) + 1, size=B).astype(np.int64)
    elif pk == "list":
        lens = np.asarray(prefix[1], dtype=np.int64).reshape(B)
    else:
        raise ValueError(pk)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    T = int(offsets[-1])
    D = Dl + Dr

    # 3-8. latent queries and caches
    q_lat = _draw_normal(rng, (B, N, H, Dl), std)
    q_rope = _draw_normal(rng, (B, N, H, Dr), std)
    kv = np.empty((T, D), dtype=np.float32)
    kv[:, :Dl] = _draw_normal(rng, (T, Dl), std)
    kv[:, Dl:] = _draw_normal(rng, (T, Dr), std)
    kv_tree = np.empty((B, N, D), dtype=np.float32)
    kv_tree[:, :, :Dl] = _draw_normal(rng, (B, N, Dl), std)
    kv_tree[:, :, Dl:] = _draw_normal(rng, (B, N, Dr), std)

    if dtype == "bf16":
        q_lat, q_rope, kv, kv_tree = (bf16_bits(a) for a in (q_lat, q_rope, kv, kv_tree))

    logits = tokens = winners = None
    if V:
        # 9-11. logits with one planted winner per row
        logits = rng.standard_normal(size=(B, N, V), dtype=np.float32)
        winners = rng.integers(0, V, size=(B, N)).astype(np.int32)
        plant = (PLANT_BASE + rng.random(size=(B, N))).astype(np.float32)
        bi, ni = np.meshgrid(np.arange(B), np.arange(N), indexing="ij")
        logits[bi, ni, winners] = plant
        # 12-14. draft tokens
        root_tok = rng.integers(0, V, size=B).astype(np.int32)
        coins = rng.random(size=(B, N)) < p_match
        other = rng.integers(0, max(V - 1, 1), size=(B, N)).astype(np.int64)
        tokens = np.empty((B, N), dtype=np.int32)
        for b in range(B):
            tokens[b, 0] = root_tok[b]
            for i in range(1, N):
                w = int(winners[b, parents[b, i]])
                if coins[b, i]:
                    tokens[b, i] = w
                else:
                    r = int(other[b, i])
                    tokens[b, i] = r + (1 if r >= w else 0)
    return Workload(name=name, dtype=dtype, B=B, N=N, H=H, Dl=Dl, Dr=Dr, scale=float(scale),
                    parents=parents, prefix_lens=lens, prefix_offsets=offsets,
                    q_lat=q_lat, q_rope=q_rope, kv=kv, kv_tree=kv_tree,
                    logits=logits, tokens=tokens, winners=winners, V=int(V))


def make_config(k: int, seed: Optional[int] = None, heads: Optional[int] = None) -> Workload:
    """One of the five reference workloads; the default seed is the config number.  heads
    overrides the head count (e.g. 8: one GPU's share of 64 heads under 8-way head parallelism;
    the latent KV is shared by all heads, so each GPU holds all of it)."""
    c = dict(CONFIGS[k])
    H = c["H"] if heads is None else int(heads)
    name = c["name"] if heads is None else f"{c['name']}-h{H}"
    return make_workload(B=c["B"], N=c["N"], H=H, Dl=c["Dl"], Dr=c["Dr"], dtype=c["dtype"],
                         std=c["std"], scale=c["scale"], prefix=c["prefix"], tree=c["tree"],
                         V=c["V"], p_match=c["p_match"], seed=k if seed is None else seed,
                         name=name)


def restrict(w: Workload, b: int, n: int) -> Workload:
    """Request b only, first n nodes (still a valid tree): a bounded sample of a workload."""
    s0, s1 = int(w.prefix_offsets[b]), int(w.prefix_offsets[b + 1])
    L = s1 - s0
    return Workload(name=w.name + f"[b{b},n{n}]", dtype=w.dtype, B=1, N=n, H=w.H, Dl=w.Dl, Dr=w.Dr,
                    scale=w.scale, parents=w.parents[b:b + 1, :n].copy(),
                    prefix_lens=np.array([L], np.int64), prefix_offsets=np.array([0, L], np.int64),
                    q_lat=w.q_lat[b:b + 1, :n], q_rope=w.q_rope[b:b + 1, :n], kv=w.kv[s0:s1],
                    kv_tree=w.kv_tree[b:b + 1, :n],
                    logits=None if w.logits is None else w.logits[b:b + 1, :n],
                    tokens=None if w.tokens is None else w.tokens[b:b + 1, :n],
                    winners=None if w.winners is None else w.winners[b:b + 1, :n], V=w.V)


def make_accept_draws(*, B: int, N: int, V: int, seed: int = 0):
    """Unplanted accept inputs: logits N(0,1) float32 [B, N, V] with no planted winner (the top two of a
    row sit close together, as in a real vocabulary), match coin flips U(0,1) [B, N], and uniform draws
    in [0, V-1) [B, N] for mismatched tokens.  Turning these into draft tokens needs the parent's argmax,
    which this module never computes: the caller derives the tokens from its own argmax.
    Draw order: logits, coin flips, mismatch draws."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(size=(B, N, V), dtype=np.float32)
    coins = rng.random(size=(B, N))
    other = rng.integers(0, max(V - 1, 1), size=(B, N)).astype(np.int64)
    return logits, coins, other


# ----------------------------------------------------------------------------
# drafter candidates for the best-first tree builder
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class DraftCandidates:
    """Per-request, per-depth top-K drafter proposals (the tree builder's input).

    root_tokens  int32 [B]        the last committed token (tree node 0)
    cand_tokens  int32 [B, D, K]  candidate tokens for depth d+1, distinct within a depth
    cand_logp    float32 [B, D, K] their log-probabilities, <= 0, non-increasing along K
    golden       int32 [B, D] or None: the tokens placed at rank 0 ("oracle drafter")
    """
    root_tokens: np.ndarray
    cand_tokens: np.ndarray
    cand_logp: np.ndarray
    golden: Optional[np.ndarray] = None


def make_draft_candidates(*, B: int, D: int, K: int, V: int, seed: int = 0, alpha: float = 0.5,
                          golden_p: Optional[float] = None, tie_step: Optional[float] = None) -> DraftCandidates:
    """Seeded drafter proposals.

    Probabilities per depth: a Dirichlet(alpha) draw over K + 1 categories (the last one stands for the
    rest of the vocabulary), the K proposal probabilities sorted in decreasing order; tokens: K distinct
    draws from the vocabulary.  golden_p: the rank-0 probability is set to this value and the others
    rescaled below it, the pages' "oracle drafter" proposing the golden continuation with the highest
    probability and distractors elsewhere.  tie_step: log-probabilities rounded down to multiples of this
    step, which makes many equal scores (tie-breaking cases).
    Draw order: root tokens, then per request and depth: tokens, Dirichlet draw.
    """
    rng = np.random.default_rng(seed)
    root = rng.integers(0, V, size=B).astype(np.int32)
    toks = np.empty((B, D, K), np.int32)
    logp = np.empty((B, D, K), np.float32)
    for b in range(B):
        for d in range(D):
            toks[b, d] = rng.choice(V, size=K, replace=False)
            p = np.sort(rng.dirichlet(np.full(K + 1, alpha))[:K])[::-1]
            if golden_p is not None:
                rest = p[1:] / max(p[1:].sum(), 1e-30) * (1.0 - golden_p) * 0.5
                p = np.concatenate([[golden_p], np.minimum(rest, golden_p)])
            lp = np.log(np.maximum(p, 1e-30)).astype(np.float32)
            if tie_step is not None:
                lp = (np.floor(lp / tie_step) * tie_step).astype(np.float32)
            logp[b, d] = np.minimum(np.sort(lp)[::-1], 0.0)
    golden = toks[:, :, 0].copy() if golden_p is not None else None
    return DraftCandidates(root_tokens=root, cand_tokens=toks, cand_logp=logp, golden=golden)
