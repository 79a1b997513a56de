"""CPU: the toy model's float64 twin, every verify step from the oracle, keeps the pages' invariant on
its own: DDTree decoding with a best-first tree and greedy accept commits exactly the greedy
autoregressive tokens (page "The Build That Proved It: Compiling the Native DDTree Speculative Decoding
Engine", section "The Output Knowledge Created").  A dropped ancestor in the mask, RoPE at a wrong
position, a wrong accept rule or a compaction out of path order breaks the equality, so this pins the
oracle's mask, RoPE, attention, accept, compaction and tree-builder functions together."""
import json
import os

import numpy as np
import pytest

from toy_mla import oracle_drafter, random_drafter
from toy_mla_ref import ToyMLARef, ref_ddtree_decode, ref_greedy_ar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_chain8_block.json")


def prompt_tokens(seed, n=12, V=512):
    return np.random.default_rng(seed).integers(0, V, size=n).tolist()


@pytest.mark.parametrize("seed", [0, 1])
def test_twin_ddtree_with_oracle_drafter_equals_its_greedy_ar(seed):
    g = json.load(open(GOLDEN))
    block, steps = int(g["block_size"]), int(g["verify_steps"])
    n_tokens = 1 + steps * block
    prompt = prompt_tokens(seed)
    ar, margin = ref_greedy_ar(ToyMLARef(seed=seed), prompt, n_tokens)
    dt, f_dt, per_step = ref_ddtree_decode(ToyMLARef(seed=seed), prompt, n_tokens,
                                           oracle_drafter(ar, D=block - 1, K=4, V=512, seed=seed), N=16)
    assert dt == ar
    assert per_step == [block - 1] * steps and f_dt == 1 + steps
    assert margin > 0.0


def test_twin_ddtree_with_random_drafter_equals_its_greedy_ar():
    prompt = prompt_tokens(2)
    ar, _ = ref_greedy_ar(ToyMLARef(seed=2), prompt, 12)
    dt, _, per_step = ref_ddtree_decode(ToyMLARef(seed=2), prompt, 12, random_drafter(D=5, K=3, V=512, seed=2), N=24)
    assert dt == ar


def test_twin_detects_a_dropped_root_row():
    """A mistake planted in the loop (the root's row, the last committed token, left out of the cache at
    every verify step) changes the tokens, so the equality above checks what compaction keeps.  (The
    order of the committed rows is not checked this way: cached rows are already rotated, and attention
    over the prefix does not depend on their order.)"""
    prompt = prompt_tokens(0)
    ar, _ = ref_greedy_ar(ToyMLARef(seed=0), prompt, 25)
    model = ToyMLARef(seed=0)
    orig = model.commit
    calls = []

    def commit_without_root(rows, a, nodes):
        calls.append(a)
        if len(calls) == 1:                    # the prefill commits the prompt as it is
            return orig(rows, a, nodes)
        nodes = np.asarray(nodes)
        if a > 0:                              # the accepted drafts only (rows of tree nodes 1 ..)
            orig([r[1:] for r in rows], a - 1, nodes[1:a + 1] - 1)
        model.L += 1                           # positions still advance by a + 1 in all
    model.commit = commit_without_root
    dt, _, _ = ref_ddtree_decode(model, prompt, 25, oracle_drafter(ar, D=7, K=4, V=512, seed=0), N=16)
    assert dt != ar
