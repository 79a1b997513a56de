"""The toy MLA model's float64 CPU twin: the golden for the DDTree loop (test workload).

Same seeded weights as the GPU model (`toy_mla.toy_weights`), widened to float64.  Every step of
the verify path comes from the oracle: the visibility mask and positions (`build_mask_ref`), NeoX
RoPE at tree positions (`rope_neox_ref`), tree-verify attention in absorbed form
(`verify_attn_ref`), the target argmax and greedy accept (`target_argmax_ref`,
`greedy_accept_ref`), cache compaction (`compact_kv_ref`) and the best-first tree builder
(`build_tree_ref`).  The layers around attention (projections, RMSNorm, SwiGLU) are plain NumPy
float64.  Greedy decoding of this twin gives the golden tokens that both GPU loops must reproduce,
the pages' invariant that autoregressive decoding and DDTree decoding both equal the golden from
the reference implementation (page "The Build That Proved It: Compiling the Native DDTree
Speculative Decoding Engine", section "The Output Knowledge Created"; page "The Moment of Proof:
Validating a Native CUDA Speculative Decoding Engine", section "How Decisions Were Made").
"""
from __future__ import annotations

import math

import numpy as np

from oracle import (build_mask_ref, build_tree_ref, compact_kv_ref, greedy_accept_ref, rope_neox_ref,
                    target_argmax_ref, verify_attn_ref)
from toy_mla import toy_inv_freq, toy_weights


class ToyMLARef:
    def __init__(self, seed=0, hidden=256, layers=4, heads=4, kv_lora=64, d_nope=32, d_rope=32, d_v=32, ffn=512,
                 vocab=512, capacity=512):
        wts = toy_weights(seed, hidden, layers, heads, kv_lora, d_nope, d_rope, d_v, ffn, vocab)
        f64 = lambda t: t.numpy().astype(np.float64)
        self.H, self.Dl, self.Dr, self.dn, self.dv, self.V = heads, kv_lora, d_rope, d_nope, d_v, vocab
        self.embed = f64(wts["embed"])
        self.layers = [{k: f64(v) for k, v in p.items()} for p in wts["layers"]]
        self.lm_head = f64(wts["lm_head"])
        self.scale = 1.0 / math.sqrt(d_nope + d_rope)
        self.inv_freq = toy_inv_freq(d_rope)
        self.cache = [np.zeros((capacity, kv_lora + d_rope)) for _ in range(layers)]
        self.L = 0

    @staticmethod
    def _rms(x, eps=1e-6):
        return x / np.sqrt((x * x).mean(-1, keepdims=True) + eps)

    def forward_tree(self, tokens, parents):
        """Logits [N, V] (float64) of a tree of N nodes after the cached prefix, and each layer's tree rows."""
        tokens = np.asarray(tokens, np.int64)
        N = len(tokens)
        parents = np.asarray(parents, np.int32)[None]
        mask, _, pos, ok = build_mask_ref(parents, np.array([self.L]))
        assert ok[0] == 1
        x = self.embed[tokens]
        tree_rows = []
        for li, p in enumerate(self.layers):
            h = self._rms(x)
            q = (h @ p["wq"]).reshape(N, self.H, self.dn + self.Dr)
            q_nope, q_rope = q[..., :self.dn], q[..., self.dn:]
            kv = h @ p["wdkv"]
            tree = np.concatenate([self._rms(kv[:, :self.Dl]), kv[:, self.Dl:]], axis=1)
            tree[:, self.Dl:] = rope_neox_ref(tree[:, self.Dl:], pos[0], self.inv_freq)
            q_rope = rope_neox_ref(q_rope, pos[0][:, None], self.inv_freq)
            q_lat = np.einsum("nhd,hdl->nhl", q_nope, p["wuk"])
            c = self.cache[li][:self.L]
            o_lat, _ = verify_attn_ref(q_lat[None], q_rope[None], c[:, :self.Dl], c[:, self.Dl:],
                                       np.array([0, self.L]), tree[None, :, :self.Dl], tree[None, :, self.Dl:],
                                       mask, self.scale)
            o = np.einsum("nhl,hlv->nhv", o_lat[0], p["wuv"]).reshape(N, self.H * self.dv)
            x = x + o @ p["wo"]
            h2 = self._rms(x)
            g = h2 @ p["wg"]
            x = x + ((g / (1.0 + np.exp(-g))) * (h2 @ p["wu"])) @ p["wd"]
            tree_rows.append(tree)
        return self._rms(x) @ self.lm_head, tree_rows

    def commit(self, tree_rows, accept_len, accept_nodes):
        """Append the accepted path's rows to every layer's cache (in path order)."""
        for li, tree in enumerate(tree_rows):
            c = self.cache[li]
            compact_kv_ref(tree[None, :, :self.Dl], tree[None, :, self.Dl:], np.asarray([accept_len]),
                           np.asarray(accept_nodes)[None], c[:, :self.Dl], c[:, self.Dl:], np.array([self.L]))
        self.L += int(accept_len) + 1


def ref_prefill(model, prompt):
    n = len(prompt)
    logits, rows = model.forward_tree(prompt, [-1] + list(range(n - 1)))
    model.commit(rows, n - 1, np.arange(n))
    return int(target_argmax_ref(logits[-1:])[0]), logits[-1]


def top2_margin(row):
    """Gap between the largest and second largest logit of a row."""
    s = np.sort(np.asarray(row, np.float64))
    return float(s[-1] - s[-2])


def ref_greedy_ar(model, prompt, n_tokens):
    """Golden greedy tokens, one forward per token; also the smallest top-2 logit gap over the decisions."""
    tok, last = ref_prefill(model, prompt)
    out, margin = [tok], top2_margin(last)
    while len(out) < n_tokens:
        logits, rows = model.forward_tree([out[-1]], [-1])
        model.commit(rows, 0, [0])
        out.append(int(target_argmax_ref(logits)[0]))
        margin = min(margin, top2_margin(logits[0]))
    return out[:n_tokens], margin


def ref_ddtree_decode(model, prompt, n_tokens, proposals, N):
    """The DDTree loop with every step from the oracle: best-first tree, one forward, greedy accept, compaction."""
    out = [ref_prefill(model, prompt)[0]]
    forwards, per_step = 1, []
    while len(out) < n_tokens:
        ct, cl = proposals(len(per_step), out)
        parents, tokens, _, _ = build_tree_ref(np.array([out[-1]], np.int32), ct[None], cl[None], N)
        logits, rows = model.forward_tree(tokens[0], parents[0])
        forwards += 1
        _, alen, anodes, commit = greedy_accept_ref(logits[None], tokens, parents)
        a = int(alen[0])
        model.commit(rows, a, anodes[0])
        out.extend(int(t) for t in commit[0, :a + 1])
        per_step.append(a)
    return out[:n_tokens], forwards, per_step
