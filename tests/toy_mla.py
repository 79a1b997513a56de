"""A tiny random-weight MLA transformer driven through the library's calls: the DDTree
speculative loop against plain greedy decoding (test workload, not part of the library).

Dimensions follow the pages' tiny test model (hidden 256, 4 layers, 4 heads, kv_lora 64,
vocabulary 512; page "The Moment of Proof: Running the Native DDTree Speculative Decoding
Engine", section "The Message Itself").  Its feed-forward block is a dense SwiGLU (the
mixture of experts is left out: the invariant under test does not depend on it).  Weights
are seeded random draws; there are no trained weights.

Per layer, attention is MLA in absorbed form:
  latent kv  c = RMSNorm(h W_dkv[:, :64]),  rotary key r = h W_dkv[:, 64:]  (one per token)
  queries    q = h W_q per head, split into q_nope (32) and q_rope (32);
             q_lat = q_nope W_uk (32 -> 64, per head), the absorbed latent query
  RoPE       ddtree_rope_tree rotates q_rope and the tree nodes' r at their positions
  attention  ddtree_verify_attn over the cached prefix plus the tree under the mask
  output     o_lat (64, per head) -> W_uv (64 -> 32) -> concat heads -> W_o
The cache holds each committed token's [c | r] row; ddtree_compact_kv appends the accepted
path after every step.  Everything except the library calls is plain torch float32.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import mla_tree_verify_absorb_amd as dd


def toy_weights(seed=0, hidden=256, layers=4, heads=4, kv_lora=64, d_nope=32, d_rope=32, d_v=32, ffn=512,
                vocab=512):
    """The seeded float32 weights of the toy model, on the CPU (shared by the GPU model and its float64 twin)."""
    g = torch.Generator().manual_seed(seed)

    def w(*shape, scale=None):
        s = scale if scale is not None else 1.0 / math.sqrt(shape[-2] if len(shape) > 1 else shape[-1])
        return torch.randn(*shape, generator=g) * s

    embed = w(vocab, hidden, scale=1.0)
    per_layer = []
    for _ in range(layers):
        per_layer.append(dict(
            wq=w(hidden, heads * (d_nope + d_rope)), wdkv=w(hidden, kv_lora + d_rope),
            wuk=w(heads, d_nope, kv_lora), wuv=w(heads, kv_lora, d_v), wo=w(heads * d_v, hidden),
            wg=w(hidden, ffn), wu=w(hidden, ffn), wd=w(ffn, hidden)))
    lm_head = w(hidden, vocab)
    return dict(embed=embed, layers=per_layer, lm_head=lm_head)


def toy_inv_freq(d_rope=32, base=10000.0):
    """Rotary frequencies base^(-2i/d), float64."""
    return base ** (-np.arange(0, d_rope, 2, dtype=np.float64) / d_rope)


class ToyMLA:
    def __init__(self, seed=0, hidden=256, layers=4, heads=4, kv_lora=64, d_nope=32, d_rope=32, d_v=32, ffn=512,
                 vocab=512, capacity=512, device="cuda:0"):
        wts = toy_weights(seed, hidden, layers, heads, kv_lora, d_nope, d_rope, d_v, ffn, vocab)
        self.H, self.Dl, self.Dr, self.dn, self.dv, self.V = heads, kv_lora, d_rope, d_nope, d_v, vocab
        self.dev = device
        self.embed = wts["embed"].to(device)
        self.layers = [{k: v.to(device) for k, v in p.items()} for p in wts["layers"]]
        self.lm_head = wts["lm_head"].to(device)
        self.scale = 1.0 / math.sqrt(d_nope + d_rope)
        self.inv_freq = torch.from_numpy(toy_inv_freq(d_rope)).to(device)
        # one [capacity, Dl + Dr] latent cache per layer
        self.cache = [torch.zeros((capacity, kv_lora + d_rope), dtype=torch.float32, device=device)
                      for _ in range(layers)]
        self.L = 0

    @staticmethod
    def _rms(x, eps=1e-6):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps)

    def forward_tree(self, tokens, parents):
        """Logits [N, V] of a tree of N nodes after the cached prefix; also the nodes' latent rows per layer."""
        N = len(tokens)
        dev = self.dev
        parents_t = torch.tensor(np.asarray(parents, np.int32)[None], device=dev)
        offsets = torch.tensor([0, self.L], dtype=torch.int64, device=dev)
        mask, depth, pos, ok = dd.ddtree_build_mask(parents_t, offsets)
        x = self.embed[torch.tensor(np.asarray(tokens, np.int64), device=dev)]
        tree_rows = []
        for li, p in enumerate(self.layers):
            h = self._rms(x)
            q = (h @ p["wq"]).view(N, self.H, self.dn + self.Dr)
            q_nope, q_rope = q[..., :self.dn], q[..., self.dn:].contiguous()
            kv = h @ p["wdkv"]
            tree = torch.cat([self._rms(kv[:, :self.Dl]), kv[:, self.Dl:]], dim=1).contiguous()[None]   # [1, N, 96]
            q_lat = torch.einsum("nhd,hdl->nhl", q_nope, p["wuk"]).contiguous()
            q_rope = q_rope[None].contiguous()
            dd.ddtree_rope_tree(q_rope, tree[..., self.Dl:], pos, self.inv_freq)
            c = self.cache[li]
            o_lat, _ = dd.ddtree_verify_attn(q_lat[None], q_rope, c[:self.L, :self.Dl], c[:self.L, self.Dl:], offsets,
                                             self.L, tree[..., :self.Dl], tree[..., self.Dl:], mask, self.scale)
            o = torch.einsum("nhl,hlv->nhv", o_lat[0], p["wuv"]).reshape(N, self.H * self.dv)
            x = x + o @ p["wo"]
            h2 = self._rms(x)
            x = x + (torch.nn.functional.silu(h2 @ p["wg"]) * (h2 @ p["wu"])) @ p["wd"]
            tree_rows.append(tree)
        return self._rms(x) @ self.lm_head, tree_rows

    def commit(self, tree_rows, accept_len, accept_nodes):
        """Append the accepted path's rows to every layer's cache."""
        dest = torch.tensor([self.L], dtype=torch.int64, device=self.dev)
        for li, tree in enumerate(tree_rows):
            c = self.cache[li]
            dd.ddtree_compact_kv(tree[..., :self.Dl], tree[..., self.Dl:], accept_len, accept_nodes, dest,
                                 c[:, :self.Dl], c[:, self.Dl:])
        self.L += int(accept_len[0]) + 1


def prefill(model, prompt):
    """The prompt as a chain tree: every row goes to the cache; returns the first generated token."""
    n = len(prompt)
    logits, rows = model.forward_tree(prompt, [-1] + list(range(n - 1)))
    dev = model.dev
    model.commit(rows, torch.tensor([n - 1], dtype=torch.int32, device=dev),
                 torch.arange(n, dtype=torch.int32, device=dev)[None])
    return int(torch.argmax(logits[-1]))


def greedy_ar(model, prompt, n_tokens):
    """Plain greedy decoding, one target forward per token (a single-node tree each step)."""
    out = [prefill(model, prompt)]
    dev = model.dev
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    root_path = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    forwards = 1
    while len(out) < n_tokens:
        logits, rows = model.forward_tree([out[-1]], [-1])
        forwards += 1
        model.commit(rows, zero, root_path)
        out.append(int(torch.argmax(logits[0])))
    return out[:n_tokens], forwards


def ddtree_decode(model, prompt, n_tokens, proposals, N):
    """DDTree speculative decoding: per step, a best-first tree from the drafter's proposals, one target
    forward over it, greedy accept, cache compaction.  proposals(step, committed) -> (cand_tokens [D, K],
    cand_logp [D, K]).  Returns (tokens, target forwards, accepted drafts per step)."""
    out = [prefill(model, prompt)]
    dev = model.dev
    forwards, per_step = 1, []
    while len(out) < n_tokens:
        ct, cl = proposals(len(per_step), out)
        parents, tokens, _, _ = dd.ddtree_build_tree(torch.tensor([out[-1]], dtype=torch.int32, device=dev),
                                                     torch.from_numpy(ct[None]).to(dev),
                                                     torch.from_numpy(cl[None]).to(dev), N)
        tok = tokens[0].cpu().numpy()
        par = parents[0].cpu().numpy()
        logits, rows = model.forward_tree(tok, par)
        forwards += 1
        _, alen, anodes, commit = dd.ddtree_greedy_accept(logits[None].contiguous(), tokens, parents)
        model.commit(rows, alen, anodes)
        a = int(alen[0])
        out.extend(int(t) for t in commit[0, :a + 1].cpu().numpy())
        per_step.append(a)
    return out[:n_tokens], forwards, per_step


def oracle_drafter(golden, D, K, V, seed=0, p_golden=0.9):
    """Proposals whose rank-0 token at depth d is the golden continuation (when known), distractors below."""
    rng = np.random.default_rng(seed)

    def proposals(step, committed):
        ct = np.empty((D, K), np.int32)
        cl = np.empty((D, K), np.float32)
        base = len(committed)
        for d in range(D):
            g = golden[base + d] if base + d < len(golden) else int(rng.integers(0, V))
            others = [t for t in rng.choice(V, size=K + 1, replace=False).tolist() if t != g][:K - 1]
            ct[d] = [g] + others
            rest = np.sort(rng.random(K - 1))[::-1] * (1 - p_golden) / (K - 1)
            cl[d] = np.log(np.concatenate([[p_golden], rest])).astype(np.float32)
        return ct, cl
    return proposals


def random_drafter(D, K, V, seed=0):
    rng = np.random.default_rng(seed)

    def proposals(step, committed):
        ct = np.stack([rng.choice(V, size=K, replace=False) for _ in range(D)]).astype(np.int32)
        cl = np.log(np.sort(rng.dirichlet(np.ones(K + 1))[:K])[::-1]).astype(np.float32)[None].repeat(D, 0)
        return ct, cl
    return proposals
