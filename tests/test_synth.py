"""The seeded input generator: determinism, tree bounds, bf16 rounding, draft-token structure."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits, bf16_to_f32, bounded_tree, make_config, make_workload


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-30, 1e-3, 1, 1e3, 1e30)])
    # exact ties: mantissa ending in 0x8000 must round to even
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("seed", range(5))
def test_bounded_tree_respects_bounds(seed):
    rng = np.random.default_rng(seed)
    for n, d, br in ((64, 8, 4), (128, 12, 4), (40, 2, 20)):
        p = bounded_tree(rng, n, d, br)
        depth = np.zeros(n, int)
        for i in range(1, n):
            assert 0 <= p[i] < i
            depth[i] = depth[p[i]] + 1
        assert depth.max() <= d
        assert np.bincount(p[1:], minlength=n).max() <= br


def test_deterministic_and_seeded():
    a, b, c = make_config(2), make_config(2), make_config(2, seed=99)
    for name in ("parents", "q_lat", "kv", "kv_tree", "logits", "tokens"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.q_lat, c.q_lat)


def test_config_shapes_small():
    for k in (1, 2, 3):
        w = make_config(k)
        c = CONFIGS[k]
        assert w.q_lat.shape == (c["B"], c["N"], c["H"], c["Dl"])
        assert w.q_rope.shape == (c["B"], c["N"], c["H"], c["Dr"])
        assert w.kv.shape == (w.T, c["Dl"] + c["Dr"]) and w.kv_tree.shape == (c["B"], c["N"], c["Dl"] + c["Dr"])
        assert (w.q_lat.dtype == np.uint16) == (c["dtype"] == "bf16")
    w1 = make_config(1)
    assert w1.parents[0].tolist() == [-1, 0, 1, 2, 3, 4, 5, 6]


def test_draft_tokens_follow_match_probability():
    w = make_workload(B=64, N=64, H=1, Dl=1, Dr=1, dtype="f32", std=1.0, scale=1.0, prefix=("fixed", 0),
                      tree=("uniform",), V=100, p_match=0.7, seed=5)
    match = np.array([[w.tokens[b, i] == w.winners[b, w.parents[b, i]] for i in range(1, 64)] for b in range(64)])
    assert abs(match.mean() - 0.7) < 0.02
    assert ((w.tokens >= 0) & (w.tokens < 100)).all()


def test_ragged_prefix_offsets():
    w = make_workload(B=5, N=3, H=2, Dl=8, Dr=4, dtype="bf16", std=0.5, scale=0.1,
                      prefix=("uniform", 0, 40), tree=("chain",), seed=1)
    assert w.prefix_offsets[0] == 0 and np.array_equal(np.diff(w.prefix_offsets), w.prefix_lens)
    assert w.kv.shape[0] == w.prefix_lens.sum()
