"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer outputs (mask, depth, positions, tree_ok, target argmax, accepted path,
committed tokens) must match exactly.  float32 workloads: max abs error <= 1e-5
on o and lse.  bf16 workloads: max|err| / max|ref| <= 2e-3 on o and lse.
Full-size workloads run in the benchmark's launch configuration and are
compared on sampled tree nodes (all heads of each sampled node).
"""
import numpy as np
import pytest
import torch

import mla_tree_verify_absorb_amd as dd
from gpu_util import (BF16_LSE_ABS_TOL, DevWorkload, check_accept, check_mask, compare_attn, lse_abs_err, mask_np,
                      oracle_attn)
from synth import CONFIGS, make_accept_draws, make_config, make_draft_candidates, make_workload

pytestmark = pytest.mark.gpu

_CACHE = {}


def config(k):
    if k not in _CACHE:
        _CACHE.clear()                      # keep at most one large workload resident
        w = make_config(k)
        _CACHE[k] = (w, DevWorkload(w))
    return _CACHE[k]


# ---------------------------------------------------------------- visibility mask

@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_build_mask_configs(k):
    _, dw = config(k)
    check_mask(dw)


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 64, 200, 255, 256])
def test_build_mask_sizes(n):
    w = make_workload(B=3, N=n, H=1, Dl=8, Dr=0, dtype="f32", std=1.0, scale=1.0,
                      prefix=("list", [0, 5, 7]), tree=("uniform",), seed=n)
    check_mask(DevWorkload(w))


def test_build_mask_int64_positions():
    from oracle import build_mask_ref
    parents = np.stack([np.arange(-1, 9, dtype=np.int32)] * 3)
    lens = np.array([1 << 40, 0, (1 << 33) + 3], np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    mask, depth, pos, ok = dd.ddtree_build_mask(torch.from_numpy(parents).cuda(), torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), build_mask_ref(parents, lens)[2])


def test_build_mask_invalid_trees_and_no_offsets():
    parents = np.array([[-1, 0, 1, 2, 3], [0, 0, 1, 2, 3], [-1, 0, 4, 1, 2], [-1, -1, 0, 1, 2],
                        [-1, 0, 0, 1, 1]], np.int32)
    pt = torch.from_numpy(parents).cuda()
    mask, depth, pos, ok = dd.ddtree_build_mask(pt, None)
    torch.cuda.synchronize()
    from oracle import build_mask_ref
    m_ref, d_ref, p_ref, ok_ref = build_mask_ref(parents, None)
    assert ok.cpu().tolist() == [1, 0, 0, 0, 1] == ok_ref.tolist()
    assert np.array_equal(mask_np(mask), m_ref)
    assert np.array_equal(depth.cpu().numpy(), d_ref)
    assert np.array_equal(pos.cpu().numpy(), p_ref)


# ---------------------------------------------------------------- greedy accept

@pytest.mark.parametrize("k", [1, 2, 5])
def test_accept_configs(k):
    w, dw = config(k)
    tstar, alen, nodes, commit = check_accept(dw)
    if k == 1:
        assert alen.tolist() == [7] and (commit[0] >= 0).sum() == 8     # block of 8 fully committed


def test_accept_ties_infinities_and_duplicate_siblings():
    B, N, V = 3, 8, 37
    logits = np.random.default_rng(0).standard_normal((B, N, V)).astype(np.float32)
    logits[0, 0, [3, 20, 36]] = 9.0                 # tie -> 3
    logits[0, 1, :] = -np.inf                       # all -inf -> 0
    logits[0, 2, [0, 36]] = np.inf                  # +inf tie -> 0
    logits[1, :, :] = 1.0                           # every row a full tie -> 0
    parents = np.array([[-1, 0, 0, 1, 1, 2, 5, 6], [-1, 0, 1, 2, 3, 4, 5, 6], [-1, 0, 0, 0, 1, 2, 3, 5]], np.int32)
    from oracle import target_argmax_ref
    ts = target_argmax_ref(logits)
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            tokens[b, i] = ts[b, parents[b, i]]     # everything matches ...
    tokens[2, 4] = (ts[2, 1] + 1) % V               # ... except node 4 of request 2
    dw = DevWorkload(make_workload(B=B, N=N, H=1, Dl=8, Dr=0, dtype="f32", std=1.0, scale=1.0,
                                   prefix=("fixed", 0), tree=("given", parents), seed=0))
    dw.w.logits, dw.w.tokens = logits, tokens
    dw.logits, dw.tokens = torch.from_numpy(logits).cuda(), torch.from_numpy(tokens).cuda()
    check_accept(dw)


@pytest.mark.parametrize("V,pad", [(1, 0), (3, 0), (7, 1), (512, 0), (1000, 3), (4099, 5)])
def test_accept_vocab_sizes_and_strided_rows(V, pad):
    B, N = 2, 16
    w = make_workload(B=B, N=N, H=1, Dl=8, Dr=0, dtype="f32", std=1.0, scale=1.0, prefix=("fixed", 0),
                      tree=("uniform",), V=V, p_match=0.8, seed=V)
    dw = DevWorkload(w)
    if pad:
        big = torch.full((B, N, V + pad), -7.0, device="cuda")
        big[..., :V] = dw.logits
        dw.logits = big[..., :V]                    # row stride V + pad (unaligned: scalar path)
    check_accept(dw)


@pytest.mark.parametrize("k,p_match", [(5, 0.8), (2, 0.7)])
def test_accept_unplanted_normal_logits(k, p_match):
    """The configs' own logits: N(0,1) over the full vocabulary with no planted winner, so each row's top
    two values are close (at V = 163840 the gap is typically ~0.1).  Draft tokens copy the parent's argmax
    with the config's match probability, the argmax taken by the oracle here."""
    from oracle import target_argmax_ref
    c = CONFIGS[k]
    B, N, V = c["B"], c["N"], c["V"]
    w = make_workload(B=B, N=N, H=1, Dl=8, Dr=0, dtype="f32", std=1.0, scale=1.0, prefix=("fixed", 0),
                      tree=c["tree"], seed=k)
    logits, coins, other = make_accept_draws(B=B, N=N, V=V, seed=1000 + k)
    ts = target_argmax_ref(logits)
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            t = int(ts[b, w.parents[b, i]])
            tokens[b, i] = t if coins[b, i] < p_match else int(other[b, i]) + (1 if other[b, i] >= t else 0)
    srt = np.sort(logits, axis=-1)
    gap = float((srt[..., -1] - srt[..., -2]).min())
    dw = DevWorkload(w)
    dw.w.logits, dw.w.tokens = logits, tokens
    dw.logits, dw.tokens = torch.from_numpy(logits).cuda(), torch.from_numpy(tokens).cuda()
    _, alen, _, _ = check_accept(dw)
    print(f"config {k} shape, unplanted N(0,1) logits: smallest top-2 gap {gap:.2e}, accept_len {alen.tolist()}")


def test_accept_single_node():
    logits = torch.tensor([[[0.5, 2.0, 2.0, -1.0]]], device="cuda")
    ta, al, an, ct = dd.ddtree_greedy_accept(logits, torch.tensor([[3]], dtype=torch.int32, device="cuda"),
                                             torch.tensor([[-1]], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert ta.tolist() == [[1]] and al.tolist() == [0] and an.tolist() == [[0]] and ct.tolist() == [[1]]


# ---------------------------------------------------------------- attention, float32

@pytest.mark.parametrize("k", [1, 2])
def test_attn_fp32_configs(k):
    w, dw = config(k)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_attn(w, m_ref)
    compare_attn(w, o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("case", [
    dict(B=1, N=1, H=2, Dl=64, Dr=32, prefix=("fixed", 0), tree=("chain",)),
    dict(B=3, N=20, H=3, Dl=24, Dr=8, prefix=("list", [0, 1, 130]), tree=("uniform",)),
    dict(B=2, N=70, H=1, Dl=512, Dr=64, prefix=("list", [65, 3]), tree=("bounded", 6, 3)),
    dict(B=1, N=5, H=5, Dl=100, Dr=0, prefix=("fixed", 64), tree=("chain",)),
])
def test_attn_fp32_edges(case):
    w = make_workload(dtype="f32", std=1.0, scale=0.125, seed=11, **case)
    dw = DevWorkload(w)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    compare_attn(w, o, lse, *oracle_attn(w, m_ref))


# ---------------------------------------------------------------- attention, bf16 MFMA kernel

K2 = dict(H=64, Dl=512, Dr=64, dtype="bf16", std=0.5, scale=1.0 / np.sqrt(192.0))


@pytest.mark.parametrize("case", [
    dict(B=1, N=8, prefix=("fixed", 40), tree=("chain",), splits=1),
    dict(B=2, N=33, H=16, prefix=("list", [0, 70]), tree=("uniform",), splits=0),
    dict(B=3, N=64, H=8, prefix=("list", [31, 32, 33]), tree=("bounded", 8, 4), splits=2),
    dict(B=1, N=100, H=3, prefix=("fixed", 300), tree=("uniform",), splits=3),
    dict(B=1, N=256, H=1, prefix=("fixed", 17), tree=("uniform",), splits=1),
    dict(B=2, N=16, prefix=("list", [1000, 5]), tree=("bounded", 8, 4), splits=4),
    dict(B=1, N=1, prefix=("fixed", 0), tree=("chain",), splits=1),
    dict(B=1, N=40, prefix=("fixed", 2000), tree=("bounded", 12, 4), splits=7),
])
def test_attn_bf16_small(case):
    case = dict(case)
    splits = case.pop("splits")
    params = dict(K2)
    params.update(case)
    w = make_workload(seed=5, **params)
    dw = DevWorkload(w)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask, num_splits=splits)
    torch.cuda.synchronize()
    compare_attn(w, o, lse, *oracle_attn(w, m_ref))


def sampled_nodes(w, per_request=3, requests=2):
    bs = sorted({0, w.B - 1})[:requests]
    out = []
    for b in bs:
        for i in sorted({0, w.N // 2, w.N - 1})[:per_request]:
            out.append((b, i))
    return out


@pytest.mark.parametrize("k", [3, 4, 5])
def test_attn_bf16_full_configs(k):
    """Full-size K2 workloads in the benchmark's launch configuration, sampled nodes."""
    w, dw = config(k)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)                          # automatic split count, as benchmarked
    torch.cuda.synchronize()
    nodes = sampled_nodes(w)
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    ea = lse_abs_err(lse, lse_ref, nodes=nodes)
    print(f"config {k}: normwise o err {eo:.2e}, lse err {el:.2e} (absolute {ea:.2e} nats) on {len(nodes)} nodes")
    assert ea <= BF16_LSE_ABS_TOL, ea


def test_attn_bf16_single_request_every_row():
    """The single 64-node request over 4096 tokens, every one of its 4096 rows against the oracle: each row is
    merged from 8 fp16 partial records (one band of 32 row blocks over 8 windows, slot-major mapping)."""
    w, dw = config(3)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_attn(w, m_ref)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref)
    ea = lse_abs_err(lse, lse_ref)
    print(f"k2-single (B1 N64 H64 L4096), every row: normwise o err {eo:.2e}, lse err {el:.2e} "
          f"(absolute {ea:.2e} nats)")
    assert ea <= BF16_LSE_ABS_TOL, ea


def test_attn_bf16_ragged_batch_every_request():
    """The ragged batch: the root, a middle node and the last node of every one of its 16 requests (prefixes
    of 1K to 32K tokens, bands cut by window edges) against the oracle."""
    w, dw = config(4)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(w.B) for i in (0, w.N // 2, w.N - 1)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    ea = lse_abs_err(lse, lse_ref, nodes=nodes)
    print(f"k2-batched-ragged (B16 N64 H64), every request: normwise o err {eo:.2e}, lse err {el:.2e} "
          f"(absolute {ea:.2e} nats) "
          f"on {len(nodes)} nodes")
    assert ea <= BF16_LSE_ABS_TOL, ea


def test_attn_bf16_long_context_every_request():
    """The 131072-token batch: two nodes of every one of its 4 requests (each request's 64 row blocks form two
    bands, which the workgroup mapping places on their own pair of XCDs) against the oracle."""
    w, dw = config(5)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(w.B) for i in (w.N // 3, 2 * w.N // 3 + 1)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    ea = lse_abs_err(lse, lse_ref, nodes=nodes)
    print(f"k2-long-context (B4 N128 H64 L131072), every request: normwise o err {eo:.2e}, lse err {el:.2e} "
          f"(absolute {ea:.2e} nats) on {len(nodes)} nodes")
    assert ea <= BF16_LSE_ABS_TOL, ea


@pytest.mark.parametrize("k", [3, 4, 5])
def test_attn_bf16_tp8_share(k):
    """One GPU's share of the K2 workloads under 8-way head parallelism (8 of 64 heads, the latent
    KV replicated): 1 to 8 row blocks per request, a divisor of 32, take the band schedule with
    bands of that many row blocks."""
    w = make_config(k, heads=8)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = sampled_nodes(w)
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    ea = lse_abs_err(lse, lse_ref, nodes=nodes)
    print(f"config {k}, 8 heads: normwise o err {eo:.2e}, lse err {el:.2e} (absolute {ea:.2e} nats) "
          f"on {len(nodes)} nodes")
    assert ea <= BF16_LSE_ABS_TOL, ea


def test_attn_bf16_split_invariance_and_determinism():
    """Every split count matches the oracle; a repeated call is bitwise identical (no atomics).
    Different split counts round P to bf16 against different running maxima, so they agree
    with each other only to within the bf16 tolerance, not bitwise."""
    w, dw = config(3)
    mask, m_ref = check_mask(dw)
    nodes = sampled_nodes(w)
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    for s in (1, 2, 8, 13):
        o, lse = dw.attn(mask, num_splits=s)
        o2, lse2 = dw.attn(mask, num_splits=s)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)


@pytest.mark.parametrize("case", [
    # ragged prefixes (empty, sub-tile, tile edges, thousands): several bands cut by window edges
    dict(B=12, N=64, H=64, prefix=("list", [0, 1, 31, 32, 33, 1500, 700, 2900, 64, 5, 3100, 950]),
         tree=("bounded", 8, 4)),
    # one request with an empty prefix: 2 tile columns over 8 windows, six of them empty
    dict(B=1, N=64, H=64, prefix=("fixed", 0), tree=("bounded", 8, 4)),
    # one long request: its band is cut into 8 pieces
    dict(B=1, N=64, H=64, prefix=("fixed", 5000), tree=("uniform",)),
    # two bands per request (128 nodes x 64 heads = 64 row blocks)
    dict(B=3, N=128, H=64, prefix=("list", [2500, 40, 900]), tree=("bounded", 12, 4)),
    # more requests than one 64-lane scan chunk (32 nodes x 128 heads)
    dict(B=66, N=32, H=128, prefix=("uniform", 0, 96), tree=("uniform",)),
    # the node limit: 256 nodes x 64 heads = 4 bands per request, 8 mask words per row
    dict(B=2, N=256, H=64, prefix=("list", [3000, 100]), tree=("bounded", 16, 4)),
])
def test_attn_bf16_band_schedule(case):
    """The automatic band schedule (row blocks in groups of 32, KV columns cut into 8 equal
    windows): every output row, whole or merged from pieces, matches the oracle, and a
    repeated call is bitwise identical."""
    params = dict(K2)
    params.update(case)
    w = make_workload(seed=31, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    o2, lse2 = dw.attn(mask)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    nodes = None
    if w.B > 32:
        nodes = [(b, i) for b in (0, 31, 63, 64, w.B - 1) for i in (0, w.N // 2, w.N - 1)]
    elif w.N > 128:
        nodes = [(b, i) for b in range(w.B) for i in (0, 1, 63, 64, 127, 128, 200, w.N - 1)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    print(f"band schedule B={w.B} N={w.N} H={w.H}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("seed", [101, 102, 103])
def test_attn_bf16_band_schedule_random_shapes(seed):
    """Seeded random band-schedule shapes: request count, (nodes, heads) with whole bands of 32
    row blocks, and a length mix of empty, sub-tile and long prefixes; sampled nodes of every
    fifth request against the oracle."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 24))
    N, H = [(64, 64), (32, 128), (128, 64)][int(rng.integers(0, 3))]
    lens = [int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(40, 6000))])) for _ in range(B)]
    params = dict(K2)
    params.update(B=B, N=N, H=H, prefix=("list", lens), tree=("bounded", 10, 4))
    w = make_workload(seed=seed, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(0, B, 5) for i in sorted({0, N // 3, N - 1})]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    print(f"seed {seed}: B={B} N={N} H={H} lens={lens}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("case", [
    # 4 row blocks per request: bands of 4, 64 windows, ragged prefixes
    dict(B=12, N=64, H=8, prefix=("list", [0, 1, 31, 32, 33, 1500, 700, 2900, 64, 5, 3100, 950]),
         tree=("bounded", 8, 4)),
    # 1 row block: 256 windows over 158 columns, most of them empty; the band is cut at every
    # non-empty window's edge
    dict(B=1, N=16, H=8, prefix=("fixed", 5000), tree=("uniform",)),
    # 2 row blocks, the second one ragged (240 rows)
    dict(B=3, N=30, H=8, prefix=("list", [400, 0, 2000]), tree=("bounded", 6, 3)),
    # 16 row blocks per request, 16 windows
    dict(B=5, N=128, H=16, prefix=("list", [3000, 0, 700, 41, 1500]), tree=("bounded", 12, 4)),
    # more requests than one 64-lane scan chunk, 2 row blocks each
    dict(B=70, N=16, H=16, prefix=("uniform", 0, 300), tree=("uniform",)),
    # one node per request: 1 row block of 8 rows
    dict(B=2, N=1, H=8, prefix=("list", [100, 0]), tree=("chain",)),
])
def test_attn_bf16_small_bands(case):
    """Band schedule with fewer than 32 row blocks per request (a divisor of 32): bands of that
    many row blocks over 256 / R windows.  Every output row, whole or merged from pieces, matches
    the oracle; a repeated call is bitwise identical."""
    params = dict(K2)
    params.update(case)
    w = make_workload(seed=37, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    o2, lse2 = dw.attn(mask)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    nodes = None
    if w.B > 32:
        nodes = [(b, i) for b in (0, 31, 63, 64, w.B - 1) for i in (0, w.N // 2, w.N - 1)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    print(f"small bands B={w.B} N={w.N} H={w.H}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("seed", [111, 112, 114, 115, 117, 130])
def test_attn_bf16_small_bands_random_shapes(seed):
    """Seeded random shapes with 1 to 16 row blocks per request and a length mix of empty,
    sub-tile and long prefixes; sampled nodes of every fourth request against the oracle."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    N, H = [(16, 8), (64, 8), (128, 8), (30, 8), (64, 16), (128, 16), (32, 32)][int(rng.integers(0, 7))]
    lens = [int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(40, 6000))])) for _ in range(B)]
    params = dict(K2)
    params.update(B=B, N=N, H=H, prefix=("list", lens), tree=("bounded", 10, 4))
    w = make_workload(seed=seed, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(0, B, 4) for i in sorted({0, N // 3, N - 1})]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    print(f"seed {seed}: B={B} N={N} H={H}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("case", [
    dict(B=1, N=64, prefix=("list", [100])),                      # one window
    dict(B=3, N=64, prefix=("list", [300, 1000, 50])),            # 6 windows, cuts across band boundaries
    dict(B=2, N=128, prefix=("list", [2000, 700])),               # two bands per request, 8 windows
    dict(B=5, N=64, prefix=("list", [0, 33, 400, 4000, 9])),      # empty and short prefixes
])
def test_attn_bf16_slot_major_short_windows(case):
    """Bands of 32 row blocks (64 heads) cut into windows of at most 128 tile columns take the slot-major
    mapping (each XCD runs 4 row blocks of every window); sampled nodes of every request against the oracle,
    and a repeat call is bitwise equal."""
    params = dict(K2)
    params.update(H=64, tree=("bounded", 8, 4), **case)
    w = make_workload(seed=71 + case["B"], **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(w.B) for i in sorted({0, 1, w.N // 2, w.N - 1})]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    o2, lse2 = dw.attn(mask)                                       # repeat calls are bitwise equal
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    print(f"slot-major {case}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("case", [
    dict(B=1, N=64, H=64, prefix=("fixed", 4096), splits=0),          # band schedule: 8 records per row
    dict(B=2, N=32, H=16, prefix=("list", [1000, 300]), splits=0),    # small bands cut by window edges
    dict(B=1, N=24, H=64, prefix=("fixed", 2000), splits=3),          # uniform splits
])
@pytest.mark.parametrize("e", [60, -60])
def test_attn_bf16_partial_records_hold_any_range(case, e):
    """Latent cache (prefix and tree rows) times 2^e and latent queries times 2^-e leave every score bit for bit
    (power-of-two scalings are exact in bf16 and in each product), so o must come out 2^e times the unscaled o
    and lse unchanged.  At e = +-60 the outputs lie far outside fp16's range, so this pins the partial records'
    per-row power-of-two scale.  lse is bitwise equal; o within 1e-5 normwise: a record's log2 weight k (the
    row's reference plus its scale exponent, |k| up to about 64 + 14 + |reference| here) is a float rounded to
    half an ulp, 2^-18 between 64 and 128, which moves the record's weight by ln 2 * 2^-18 = 2.6e-6 relative."""
    params = dict(K2)
    shape = {k: v for k, v in case.items() if k != "splits"}
    splits = case["splits"]
    params.update(tree=("bounded", 8, 4), **shape)
    w = make_workload(seed=61, **params)
    dw = DevWorkload(w)
    mask, _, _, _ = dw.build_mask()
    o0, l0 = dw.attn(mask, num_splits=splits)
    dw.ckv.mul_(2.0 ** e)
    dw.ckv_tree.mul_(2.0 ** e)
    dw.q_lat.mul_(2.0 ** -e)
    o1, l1 = dw.attn(mask, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(l1, l0)
    ref = o0.double() * 2.0 ** e
    err = float((o1.double() - ref).norm() / ref.norm())
    assert bool(torch.isfinite(o1).all()) and err <= 1e-5, err
    print(f"records at 2^{e}, {case}: normwise o error against the exact scaling {err:.2e}")


@pytest.mark.parametrize("H,max_len", [(8, 0), (8, 100), (64, 0)])
def test_attn_bf16_band_understated_max_prefix_len(H, max_len):
    """The band schedule's window count is bounded on the host from max_prefix_len and on the
    device from the true lengths; a max_prefix_len below the true lengths (outside the documented
    contract) gives fewer windows, never a wrong result."""
    params = dict(K2)
    params.update(B=3, N=64, H=H, prefix=("list", [2500, 40, 4000]), tree=("bounded", 8, 4))
    w = make_workload(seed=38, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dd.ddtree_verify_attn(dw.q_lat, dw.q_rope, dw.ckv, dw.krope, dw.offsets, max_len, dw.ckv_tree,
                                   dw.krope_tree, mask, w.scale, num_splits=0)
    torch.cuda.synchronize()
    nodes = [(b, i) for b in range(w.B) for i in (0, 21, 42, 63)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    print(f"H={H}, max_prefix_len {max_len}: normwise o err {eo:.2e}, lse err {el:.2e}")


@pytest.mark.parametrize("case", [
    dict(B=2, N=8, H=4, Dl=64, Dr=32, prefix=("list", [8, 0]), tree=("chain",)),        # the tiny model's dims
    dict(B=3, N=33, H=8, Dl=256, Dr=32, prefix=("list", [100, 0, 700]), tree=("uniform",)),
    dict(B=1, N=5, H=3, Dl=500, Dr=12, prefix=("fixed", 40), tree=("bounded", 3, 2)),     # odd dims
])
def test_attn_bf16_generic_dims(case):
    """bf16 inputs at dims other than the MFMA kernel's (512, 64) run on the generic kernel, in
    float32 arithmetic on the same bf16 values the oracle reads: held to the fp32 bar."""
    w = make_workload(dtype="bf16", std=0.5, scale=0.11, seed=17, **case)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 1
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_attn(w, m_ref)
    compare_attn(w, o, lse, o_ref, lse_ref)
    eo = float(np.abs(o.cpu().numpy() - o_ref).max())
    el = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    assert eo <= 1e-5 and el <= 1e-5, (eo, el)


def test_attn_bf16_band_schedule_long_single_request():
    """One 131072-token request, 128 nodes: its two bands (64 row blocks) are cut across all 8
    windows, so every row is merged from pieces; sampled nodes against the oracle."""
    params = dict(K2)
    params.update(B=1, N=128, prefix=("fixed", 131072), tree=("bounded", 12, 4))
    w = make_workload(seed=33, **params)
    dw = DevWorkload(w)
    assert dd.ddtree_verify_attn_auto_splits(dd.DDTREE_BF16, w.B, w.N, w.H, w.Dl, w.Dr, dw.max_len) == 0
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask)
    torch.cuda.synchronize()
    nodes = [(0, i) for i in (0, 1, 63, 64, 127)]
    o_ref, lse_ref = oracle_attn(w, m_ref, nodes=nodes)
    eo, el = compare_attn(w, o, lse, o_ref, lse_ref, nodes=nodes)
    ea = lse_abs_err(lse, lse_ref, nodes=nodes)
    print(f"band schedule, one 131072-token request: normwise o err {eo:.2e}, lse err {el:.2e} "
          f"(absolute {ea:.2e} nats)")
    assert ea <= BF16_LSE_ABS_TOL, ea


@pytest.mark.parametrize("splits", [1, 3])
def test_attn_bf16_uniform_splits_on_band_shapes(splits):
    """An explicit split count takes the uniform schedule even where the band schedule would apply."""
    params = dict(K2)
    params.update(B=5, N=64, prefix=("list", [3000, 0, 700, 41, 1500]), tree=("bounded", 8, 4))
    w = make_workload(seed=34, **params)
    dw = DevWorkload(w)
    mask, m_ref = check_mask(dw)
    o, lse = dw.attn(mask, num_splits=splits)
    torch.cuda.synchronize()
    compare_attn(w, o, lse, *oracle_attn(w, m_ref))


def _bf16_bits(x):
    from synth import bf16_bits
    return bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("jump_key", [5, 900, 2047])
def test_attn_bf16_large_score_jump(jump_key):
    """A key whose score exceeds the first tile's maximum by far more than the kernel's
    headroom (2^100 in exp2 units) forces the workgroup's second pass."""
    params = dict(K2)
    params.update(B=1, N=12, prefix=("fixed", 2048), tree=("bounded", 6, 3))
    w = make_workload(seed=21, **params)
    # rotary query of every node/head and rotary key of one prefix row set to 8: that key's
    # score is 8 * 8 * 64 * scale ~ 296 (natural units), about 427 in log2 units
    w.q_rope[...] = _bf16_bits(np.full(w.q_rope.shape, 8.0))
    w.kv[jump_key, w.Dl:] = _bf16_bits(np.full(w.Dr, 8.0))
    dw = DevWorkload(w)
    mask, m_ref = check_mask(dw)
    for s in (1, 3):
        o, lse = dw.attn(mask, num_splits=s)
        torch.cuda.synchronize()
        compare_attn(w, o, lse, *oracle_attn(w, m_ref))


# ---------------------------------------------------------------- KV-cache compaction

SENTINEL = {"f32": np.float32(-12345.5), "bf16": np.uint16(0x7FC1)}


def host_rows(w, arr):
    """Raw host rows of a workload array (uint16 bf16 bits or float32), as stored on the device."""
    return np.ascontiguousarray(arr)


def cache_regions(w, extra):
    """Per-request cache regions of L_b + extra rows, prefix copied in, the rest a sentinel.
    Returns (host cache [R, Dl+Dr] in raw storage type, dest_rows int64 [B])."""
    kv = host_rows(w, w.kv)
    starts, R = [], 0
    for b in range(w.B):
        starts.append(R)
        R += int(w.prefix_lens[b]) + extra
    cache = np.full((R, w.Dl + w.Dr), SENTINEL[w.dtype], dtype=kv.dtype)
    for b in range(w.B):
        s0, L = int(w.prefix_offsets[b]), int(w.prefix_lens[b])
        cache[starts[b]:starts[b] + L] = kv[s0:s0 + L]
    dest = np.array([starts[b] + int(w.prefix_lens[b]) for b in range(w.B)], np.int64)
    return cache, dest


def to_dev_raw(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(arr).to("cuda:0")


def from_dev_raw(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_compaction(w, dw, alen, nodes, extra=None, check_rows=None):
    """GPU compaction of (alen, nodes) into fresh per-request regions vs the oracle; bit-exact."""
    from oracle import compact_kv_ref
    extra = w.N if extra is None else extra
    cache, dest = cache_regions(w, extra)
    dev_cache = to_dev_raw(cache, w.dtype)
    dd.ddtree_compact_kv(dw.ckv_tree, dw.krope_tree, torch.from_numpy(np.ascontiguousarray(alen, np.int32)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(nodes, np.int32)).cuda(), torch.from_numpy(dest).cuda(),
                         dev_cache[:, :w.Dl], dev_cache[:, w.Dl:])
    torch.cuda.synchronize()
    kt = host_rows(w, w.kv_tree)
    exp = cache.copy()
    compact_kv_ref(kt[..., :w.Dl], kt[..., w.Dl:], alen, nodes, exp[:, :w.Dl], exp[:, w.Dl:], dest)
    got = from_dev_raw(dev_cache, w.dtype)
    rows = slice(None) if check_rows is None else check_rows(dest)
    assert np.array_equal(got[rows].view(np.uint8), exp[rows].view(np.uint8))
    return got, exp, dest


def random_paths(w, seed):
    """A random terminal per request and its root path, in the accept outputs' format."""
    rng = np.random.default_rng(seed)
    alen = np.zeros(w.B, np.int32)
    nodes = np.full((w.B, w.N), -1, np.int32)
    for b in range(w.B):
        path = [int(rng.integers(0, w.N))]
        while w.parents[b, path[-1]] != -1:
            path.append(int(w.parents[b, path[-1]]))
        path = path[::-1]
        alen[b] = len(path) - 1
        nodes[b, :len(path)] = path
    return alen, nodes


@pytest.mark.parametrize("k", [1, 2, 5])
def test_compact_kv_after_accept(k):
    """Compaction fed with the GPU accept outputs (equal to the oracle's) moves the accepted rows."""
    w, dw = config(k)
    _, alen_t, nodes_t, _ = dd.ddtree_greedy_accept(dw.logits, dw.tokens, dw.parents)
    _, alen, nodes, _ = check_accept(dw)
    assert np.array_equal(alen_t.cpu().numpy(), alen) and np.array_equal(nodes_t.cpu().numpy(), nodes)
    if k == 5:      # compare the regions around the written rows (the cache is 0.6 GB)
        sel = lambda dest: np.concatenate([np.arange(d - 64, d + w.N) for d in dest])
        run_compaction(w, dw, alen, nodes, check_rows=sel)
    else:
        run_compaction(w, dw, alen, nodes)


@pytest.mark.parametrize("k,seed", [(2, 7), (3, 1), (3, 2), (4, 3)])
def test_compact_kv_random_paths(k, seed):
    w, dw = config(k)
    alen, nodes = random_paths(w, seed)
    if k == 4:
        sel = lambda dest: np.concatenate([np.arange(d - 16, d + w.N) for d in dest])
        run_compaction(w, dw, alen, nodes, check_rows=sel)
    else:
        run_compaction(w, dw, alen, nodes)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dl,Dr", [(512, 64), (64, 32), (7, 0), (9, 3)])
def test_compact_kv_widths_and_edges(dtype, Dl, Dr):
    """Widths that force 16-, 4- and 2-byte copy pieces; accept_len 0, an invalid node entry (skipped),
    a negative dest row (request skipped) and a full-depth chain."""
    N = 12
    parents = np.array([[-1] + list(range(N - 1)), [-1, 0, 0, 1, 3, 2, 5, 6, 6, 8, 1, 4],
                        [-1, 0, 1, 1, 2, 4, 4, 6, 7, 0, 9, 10], [-1] + list(range(N - 1))], np.int32)
    w = make_workload(B=4, N=N, H=1, Dl=Dl, Dr=Dr, dtype=dtype, std=1.0, scale=1.0,
                      prefix=("list", [5, 0, 33, 2]), tree=("given", parents), seed=11)
    dw = DevWorkload(w)
    alen = np.array([0, 3, 5, N - 1], np.int32)
    nodes = np.full((4, N), -1, np.int32)
    nodes[0, 0] = 0
    nodes[1, :4] = [0, 1, 3, 4]
    nodes[2, :6] = [0, 1, 99, 4, 5, 6]          # entry 99 is skipped
    nodes[3, :] = np.arange(N)
    got, exp, dest = run_compaction(w, dw, alen, nodes)
    # the untouched request: negative dest row
    cache, dest = cache_regions(w, N)
    dev_cache = to_dev_raw(cache, dtype)
    dest_neg = dest.copy()
    dest_neg[1] = -1
    dd.ddtree_compact_kv(dw.ckv_tree, dw.krope_tree, torch.from_numpy(alen).cuda(), torch.from_numpy(nodes).cuda(),
                         torch.from_numpy(dest_neg).cuda(), dev_cache[:, :Dl], dev_cache[:, Dl:])
    torch.cuda.synchronize()
    got2 = from_dev_raw(dev_cache, dtype)
    b1 = slice(int(dest[1]), int(dest[1]) + N)
    assert np.array_equal(got2[b1].view(np.uint8), cache[b1].view(np.uint8))
    assert np.array_equal(got2[:int(dest[1])].view(np.uint8), got[:int(dest[1])].view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed,N,tree", [(0, 40, ("bounded", 8, 3)), (1, 40, ("bounded", 8, 3)),
                                         (2, 40, ("bounded", 8, 3)), (3, 100, ("chain",))])
def test_compact_kv_in_place(dtype, seed, N, tree):
    """Tree rows stored in the cache right after the prefix (node i at row dest + i), one call per request:
    the in-place move equals the oracle's move between separate buffers.  The 100-node chain is too long
    to stage in LDS and takes the row-by-row path."""
    from oracle import compact_kv_ref
    Dl, Dr = 512, 64
    w = make_workload(B=3, N=N, H=1, Dl=Dl, Dr=Dr, dtype=dtype, std=1.0, scale=1.0, prefix=("list", [17, 0, 64]),
                      tree=tree, seed=seed)
    alen, nodes = random_paths(w, seed + 100)
    if tree[0] == "chain":
        alen[:] = N - 1
        nodes[:] = np.arange(N)
    if seed == 0:          # the path 0 -> 2 -> 3 -> 4 reads row 2 (depth 1) before writing it (depth 2)
        w.parents[0, :5] = [-1, 0, 0, 2, 3]
        alen[0], nodes[0] = 3, -1
        nodes[0, :4] = [0, 2, 3, 4]
    cache, dest = cache_regions(w, N)
    kt = host_rows(w, w.kv_tree)
    for b in range(w.B):
        cache[dest[b]:dest[b] + N] = kt[b]          # tree rows in place
    exp = cache.copy()
    compact_kv_ref(kt[..., :Dl], kt[..., Dl:], alen, nodes, exp[:, :Dl], exp[:, Dl:], dest)
    dev_cache = to_dev_raw(cache, dtype)
    for b in range(w.B):
        d = int(dest[b])
        tree_c = dev_cache[d:d + N, :Dl].unsqueeze(0)
        tree_r = dev_cache[d:d + N, Dl:].unsqueeze(0)
        dd.ddtree_compact_kv(tree_c, tree_r, torch.from_numpy(alen[b:b + 1].copy()).cuda(),
                             torch.from_numpy(nodes[b:b + 1].copy()).cuda(), torch.tensor([d], dtype=torch.int64).cuda(),
                             dev_cache[:, :Dl], dev_cache[:, Dl:])
    torch.cuda.synchronize()
    got = from_dev_raw(dev_cache, dtype)
    for b in range(w.B):
        rows = slice(int(dest[b]), int(dest[b]) + int(alen[b]) + 1)
        assert np.array_equal(got[rows].view(np.uint8), exp[rows].view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compact_kv_long_paths_separate_buffers(dtype):
    """Paths too long for the LDS stage (a 160-node chain) take the row-by-row path."""
    N = 160
    w = make_workload(B=2, N=N, H=1, Dl=512, Dr=64, dtype=dtype, std=1.0, scale=1.0, prefix=("list", [3, 40]),
                      tree=("chain",), seed=5)
    dw = DevWorkload(w)
    alen = np.array([N - 1, 77], np.int32)
    nodes = np.tile(np.arange(N, dtype=np.int32), (2, 1))
    nodes[1, 78:] = -1
    run_compaction(w, dw, alen, nodes)


# ---------------------------------------------------------------- best-first tree builder

def check_build_tree(c, N):
    from oracle import build_tree_ref
    dev = "cuda:0"
    got = dd.ddtree_build_tree(torch.from_numpy(c.root_tokens).to(dev), torch.from_numpy(c.cand_tokens).to(dev),
                               torch.from_numpy(c.cand_logp).to(dev), N)
    torch.cuda.synchronize()
    ref = build_tree_ref(c.root_tokens, c.cand_tokens, c.cand_logp, N)
    for g, r in zip(got, ref):
        g = g.cpu().numpy()
        assert np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                              r.view(np.uint32) if r.dtype == np.float32 else r)
    return got


@pytest.mark.parametrize("B,D,K,N,seed", [(4, 7, 4, 64, 0), (2, 7, 8, 128, 1), (3, 16, 2, 256, 2), (1, 3, 3, 40, 3),
                                          (5, 8, 1, 9, 4), (2, 64, 64, 256, 5), (16, 12, 4, 128, 6), (1, 1, 1, 2, 7)])
def test_build_tree_matches_oracle(B, D, K, N, seed):
    c = make_draft_candidates(B=B, D=D, K=K, V=1000, seed=seed)
    check_build_tree(c, N)


@pytest.mark.parametrize("seed", [0, 1])
def test_build_tree_ties_and_oracle_drafter(seed):
    check_build_tree(make_draft_candidates(B=3, D=6, K=5, V=200, seed=seed, tie_step=0.5), 100)
    c = make_draft_candidates(B=2, D=7, K=4, V=512, seed=seed, golden_p=0.9)
    parents, tokens, _, _ = check_build_tree(c, 24)
    assert parents[:, 1:8].cpu().numpy().tolist() == [list(range(7))] * 2


def test_build_tree_feeds_build_mask():
    """The GPU-built trees are valid inputs of ddtree_build_mask, with matching depths."""
    c = make_draft_candidates(B=4, D=12, K=4, V=5000, seed=11)
    parents, tokens, depth, _ = check_build_tree(c, 128)
    mask, mdepth, pos, ok = dd.ddtree_build_mask(parents)
    torch.cuda.synchronize()
    assert (ok.cpu() == 1).all() and torch.equal(mdepth.cpu(), depth.cpu())


# ---------------------------------------------------------------- NeoX RoPE at tree positions

def rope_expected(x_f32, pos, inv, dtype):
    from oracle import rope_neox_ref
    from synth import bf16_bits
    y = rope_neox_ref(x_f32, pos, inv)
    return bf16_bits(y.astype(np.float32)) if dtype == "bf16" else y.astype(np.float32)


def max_ulp(a, b, dtype):
    ia = a.view(np.uint16).astype(np.int64) if dtype == "bf16" else a.view(np.uint32).astype(np.int64)
    ib = b.view(np.uint16).astype(np.int64) if dtype == "bf16" else b.view(np.uint32).astype(np.int64)
    # same-sign values: the bit-pattern distance is the ulp distance
    return int(np.abs(ia - ib).max()) if ia.size else 0


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_rope_tree_configs(k):
    """Queries (all heads) and tree keys rotated at their build_mask positions: within 1 ulp of the
    float64 oracle rounded to the storage type (the last bit may differ where the libraries' sin/cos do)."""
    from oracle import rope_inv_freq
    w, dw = config(k)
    _, _, pos, _ = dw.build_mask()
    inv = rope_inv_freq(w.Dr, 10000.0)
    q = dw.q_rope.clone()
    kt = dw.kv_tree.clone()
    dd.ddtree_rope_tree(q, kt[..., w.Dl:], pos, torch.from_numpy(inv).cuda())
    torch.cuda.synchronize()
    p = pos.cpu().numpy()
    exp_q = rope_expected(w.f32("q_rope"), p[:, :, None], inv, w.dtype)
    exp_k = rope_expected(w.f32("kv_tree")[..., w.Dl:], p, inv, w.dtype)
    got_q = from_dev_raw(q, w.dtype)
    got_k = from_dev_raw(kt, w.dtype)[..., w.Dl:]
    assert max_ulp(np.ascontiguousarray(got_q), exp_q, w.dtype) <= 1
    assert max_ulp(np.ascontiguousarray(got_k), np.ascontiguousarray(exp_k), w.dtype) <= 1
    # the latent part of the tree rows is untouched
    assert np.array_equal(from_dev_raw(kt, w.dtype)[..., :w.Dl], host_rows(w, w.kv_tree)[..., :w.Dl])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_tree_queries_or_keys_alone_and_large_positions(dtype):
    from oracle import rope_inv_freq
    w = make_workload(B=2, N=9, H=3, Dl=8, Dr=128, dtype=dtype, std=1.0, scale=1.0, prefix=("list", [0, 5]),
                      tree=("uniform",), seed=4)
    dw = DevWorkload(w)
    inv = rope_inv_freq(w.Dr, 500000.0)
    pos = np.array([[0] * 9, list(range(2 ** 40, 2 ** 40 + 9))], np.int64)
    q = dw.q_rope.clone()
    dd.ddtree_rope_tree(q, None, torch.from_numpy(pos).cuda(), torch.from_numpy(inv).cuda())
    kt = dw.kv_tree.clone()
    dd.ddtree_rope_tree(None, kt[..., w.Dl:], torch.from_numpy(pos).cuda(), torch.from_numpy(inv).cuda())
    torch.cuda.synchronize()
    assert max_ulp(from_dev_raw(q, dtype), rope_expected(w.f32("q_rope"), pos[:, :, None], inv, dtype), dtype) <= 1
    got_k = np.ascontiguousarray(from_dev_raw(kt, dtype)[..., w.Dl:])
    exp_k = np.ascontiguousarray(rope_expected(w.f32("kv_tree")[..., w.Dl:], pos, inv, dtype))
    assert max_ulp(got_k, exp_k, dtype) <= 1
    # position 0 is the identity
    assert np.array_equal(from_dev_raw(q, dtype)[0], host_rows(w, w.q_rope)[0])
