"""End to end: the DDTree speculative loop on a tiny random-weight MLA model, every step through
the library (tree builder, mask and positions, RoPE, tree-verify attention, greedy accept, cache
compaction), produces exactly the greedy autoregressive tokens.

The pages' demonstration: with block size 8 and a drafter that proposes the target's greedy
continuation, 24 tokens take 3 verify steps instead of 24 forwards, and the output matches plain
greedy decoding token for token (page "The Build That Proved It: Compiling the Native DDTree
Speculative Decoding Engine", section "The Output Knowledge Created"; page "The Moment of Proof:
Running the Native DDTree Speculative Decoding Engine", section "The Message Itself").  The pages'
own model file is not available; the weights here are random, which the invariant does not depend on.
The golden tokens come from the model's float64 CPU twin, whose verify steps are all the oracle's
(`toy_mla_ref`): the pages' check is autoregressive == golden and DDTree == golden (page "The Build That
Proved It...", section "The Output Knowledge Created"), with the golden from the reference
implementation rather than from the engine under test.
"""
import json
import os

import numpy as np
import pytest
import torch

from toy_mla import ToyMLA, ddtree_decode, greedy_ar, oracle_drafter, random_drafter
from toy_mla_ref import ToyMLARef, ref_greedy_ar

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_chain8_block.json")


def prompt_tokens(seed, n=12, V=512):
    return np.random.default_rng(seed).integers(0, V, size=n).tolist()


def golden_tokens(seed, prompt, n_tokens):
    """Greedy tokens of the float64 twin (oracle verify steps) and their smallest top-2 logit gap."""
    return ref_greedy_ar(ToyMLARef(seed=seed), prompt, n_tokens)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_ddtree_with_oracle_drafter_equals_greedy_ar_equals_golden(seed):
    g = json.load(open(GOLDEN))
    block, steps = int(g["block_size"]), int(g["verify_steps"])
    n_tokens = 1 + steps * block                          # the prefill's token, then 3 full blocks
    prompt = prompt_tokens(seed)
    golden, margin = golden_tokens(seed, prompt, n_tokens)
    ar, f_ar = greedy_ar(ToyMLA(seed=seed), prompt, n_tokens)
    dt, f_dt, per_step = ddtree_decode(ToyMLA(seed=seed), prompt, n_tokens,
                                       oracle_drafter(golden, D=block - 1, K=4, V=512, seed=seed), N=16)
    print(f"seed {seed}: AR {f_ar} forwards, DDTree {f_dt} forwards, accepted drafts per step {per_step}, "
          f"golden's smallest top-2 logit gap {margin:.3e}")
    assert ar == golden
    assert dt == golden
    assert per_step == [block - 1] * steps                # every step commits block_size tokens
    assert f_ar == n_tokens and f_dt == 1 + steps


@pytest.mark.parametrize("seed", [2, 3])
def test_ddtree_with_random_drafter_equals_greedy_ar(seed):
    """A drafter that is mostly wrong: rejections and bonus tokens only, the output is still greedy-exact."""
    prompt = prompt_tokens(seed)
    golden, _ = golden_tokens(seed, prompt, 14)
    ar, _ = greedy_ar(ToyMLA(seed=seed), prompt, 14)
    dt, f_dt, per_step = ddtree_decode(ToyMLA(seed=seed), prompt, 14, random_drafter(D=5, K=3, V=512, seed=seed),
                                       N=24)
    print(f"seed {seed}: accepted drafts per step {per_step}")
    assert ar == golden and dt == golden
    assert f_dt == 1 + len(per_step) and sum(a + 1 for a in per_step) >= 13


def test_ddtree_with_partly_right_drafter_equals_greedy_ar():
    """Golden proposals with some depths corrupted: partial acceptance of varying length."""
    prompt = prompt_tokens(7)
    golden, _ = golden_tokens(7, prompt, 30)
    ar, _ = greedy_ar(ToyMLA(seed=7), prompt, 30)
    assert ar == golden
    base = oracle_drafter(ar, D=6, K=4, V=512, seed=7)
    rng = np.random.default_rng(7)

    def proposals(step, committed):
        ct, cl = base(step, committed)
        d = int(rng.integers(0, 6))
        ct[d, 0] = (ct[d, 0] + 1 + int(rng.integers(0, 500))) % 512 if ct[d, 0] not in ct[d, 1:] else ct[d, 0]
        return ct, cl

    dt, f_dt, per_step = ddtree_decode(ToyMLA(seed=7), prompt, 30, proposals, N=32)
    print(f"accepted drafts per step {per_step}")
    assert dt == ar
    assert len(set(per_step)) > 1
