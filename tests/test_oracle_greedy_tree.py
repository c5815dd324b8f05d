"""Pins of the oracle's greedy and tree verification.

Greedy speculation must reproduce plain greedy decoding ("推测解码与 MTP"
§11); the stochastic rule at vanishing temperature with one-hot drafts must
agree with it; a chain-shaped tree is greedy verification; brute force over
root-to-node paths checks the tree rule of §3.3; the 3x3x2 tree of §3.3 has
18 candidate paths (tests/golden/medusa_tree_3x3x2.json).
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, make, medusa_tree_parents

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def slow_argmax(row):
    m = max(row)
    return min(j for j, v in enumerate(row) if v == m)


def test_argmax_lowest_index_on_ties():
    row = [1.0, 3.0, -2.0, 3.0, 3.0]
    assert oracle.argmax_lowest(row) == 1 == slow_argmax(row)
    assert oracle.argmax_lowest([-np.inf, -np.inf]) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_reproduces_plain_greedy(dtype):
    rng = np.random.default_rng(21)
    B, K, V = 40, 4, 300
    x32 = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    tgt = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    vals = oracle.logits_f64(tgt.reshape(-1), dtype).reshape(B, K + 1, V)
    g = np.array([[slow_argmax(vals[b, i].tolist()) for i in range(K + 1)] for b in range(B)])
    drafts = np.where(rng.random((B, K)) < 0.7, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    tok, alen, gg = oracle.spec_verify_greedy(tgt, drafts, dtype)
    np.testing.assert_array_equal(gg, g)
    for b in range(B):
        a = alen[b] - 1
        # the emitted tokens are exactly plain greedy decoding's next a+1 tokens
        np.testing.assert_array_equal(tok[b, :a + 1], g[b, :a + 1])
        assert np.all(drafts[b, :a] == g[b, :a])
        assert a == K or drafts[b, a] != g[b, a]
        assert np.all(tok[b, a + 1:] == -1)


def test_sampling_rule_at_vanishing_temperature_is_greedy():
    rng = np.random.default_rng(22)
    B, K, V = 30, 3, 200
    tgt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    srt = np.sort(tgt, axis=-1)
    gap_ok = (srt[..., -1] - srt[..., -2]) > 0.02
    tgt = tgt[gap_ok.all(axis=1)]
    B = tgt.shape[0]
    g = tgt.argmax(-1)
    drafts = np.where(rng.random((B, K)) < 0.6, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    T = np.full(B, 1e-4, np.float32)
    seeds = np.arange(B, dtype=np.uint64)
    s_tok, s_len, *_ = oracle.spec_verify_sample(tgt, None, drafts, T, seeds, 0)
    g_tok, g_len, _ = oracle.spec_verify_greedy(tgt, drafts)
    np.testing.assert_array_equal(s_len, g_len)
    np.testing.assert_array_equal(s_tok, g_tok)


def test_chain_tree_is_greedy():
    rng = np.random.default_rng(23)
    B, K, V = 25, 5, 100
    tgt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    g = tgt.argmax(-1)
    drafts = np.where(rng.random((B, K)) < 0.8, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    parents = np.arange(-1, K, dtype=np.int32)             # node n's parent is n-1
    node_tok = np.concatenate([np.full((B, 1), -1, np.int32), drafts], axis=1)
    t_tok, t_len, best = oracle.spec_verify_tree(tgt, node_tok, parents)
    g_tok, g_len, _ = oracle.spec_verify_greedy(tgt, drafts)
    np.testing.assert_array_equal(t_len, g_len)
    np.testing.assert_array_equal(t_tok[:, :K + 1], g_tok)
    np.testing.assert_array_equal(best, g_len - 1)


def _paths(parents):
    out = {0: [0]}
    for n in range(1, len(parents)):
        out[n] = out[int(parents[n])] + [n]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_tree_brute_force_over_paths(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(2, 20))
    parents = np.array([-1] + [int(rng.integers(0, n)) for n in range(1, N)], np.int32)
    B, V = 12, 6                       # tiny vocab: many matches and duplicate siblings
    tgt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    node_tok = rng.integers(0, V, (B, N)).astype(np.int32)
    tok, alen, best = oracle.spec_verify_tree(tgt, node_tok, parents)
    paths = _paths(parents)
    for b in range(B):
        g = [slow_argmax(tgt[b, n].tolist()) for n in range(N)]
        ok = [n for n, path in paths.items()
              if all(node_tok[b, c] == g[p] for p, c in zip(path[:-1], path[1:]))]
        deepest = max(len(paths[n]) for n in ok)
        want = min(n for n in ok if len(paths[n]) == deepest)
        assert best[b] == want
        seq = [int(node_tok[b, n]) for n in paths[want][1:]] + [g[want]]
        assert alen[b] == len(seq)
        np.testing.assert_array_equal(tok[b, :len(seq)], seq)
        assert np.all(tok[b, len(seq):] == -1)


@pytest.mark.parametrize("seed", range(3))
def test_tree_per_request_brute_force_over_paths(seed):
    """A tree per request ([B, N] parents, dynamic trees): each request against
    the brute force over its own tree's paths; a row that is not a tree
    refuses only its own request."""
    rng = np.random.default_rng(200 + seed)
    B, N, V = 10, int(rng.integers(2, 16)), 5
    parents = np.array([[-1] + [int(rng.integers(0, n)) for n in range(1, N)] for _ in range(B)], np.int32)
    bad = {3: (0, 0), 7: (N - 1, N - 1)}             # root with a parent; a node its own parent
    for b, (n, v) in bad.items():
        parents[b, n] = v
    tgt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    node_tok = rng.integers(0, V, (B, N)).astype(np.int32)
    tok, alen, best = oracle.spec_verify_tree(tgt, node_tok, parents)
    for b in range(B):
        if b in bad:
            assert (alen[b], best[b]) == (0, -1) and np.all(tok[b] == -1)
            continue
        paths = _paths(parents[b])
        g = [slow_argmax(tgt[b, n].tolist()) for n in range(N)]
        ok = [n for n, path in paths.items()
              if all(node_tok[b, c] == g[p] for p, c in zip(path[:-1], path[1:]))]
        deepest = max(len(paths[n]) for n in ok)
        want = min(n for n in ok if len(paths[n]) == deepest)
        assert best[b] == want
        seq = [int(node_tok[b, n]) for n in paths[want][1:]] + [g[want]]
        assert alen[b] == len(seq)
        np.testing.assert_array_equal(tok[b, :len(seq)], seq)
        assert np.all(tok[b, len(seq):] == -1)


def test_tree_shared_parents_equal_per_request_rows():
    wl = make("c5_tree", data_seed=6, B=5, V=300)
    par = wl["parents"]
    a = oracle.spec_verify_tree(wl["target"], wl["draft_tokens"], par)
    b = oracle.spec_verify_tree(wl["target"], wl["draft_tokens"], np.tile(par, (5, 1)))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_medusa_tree_golden():
    with open(os.path.join(GOLDEN, "medusa_tree_3x3x2.json")) as f:
        gold = json.load(f)
    parents = medusa_tree_parents(tuple(gold["branching"]))
    assert parents.tolist() == gold["parents"]
    assert len(parents) == gold["nodes"]
    depth = oracle.tree_depths(parents)
    leaves = [n for n in range(len(parents)) if n not in set(parents[1:].tolist())]
    assert len(leaves) == gold["leaf_paths"] == 3 * 3 * 2
    assert max(depth) == gold["max_depth"]


def test_tree_rejects_malformed_parents():
    with pytest.raises(ValueError):
        oracle.tree_depths([0, 0])
    with pytest.raises(ValueError):
        oracle.tree_depths([-1, 2, 0])


def test_tree_workload_recipe():
    wl = make("c5_tree", data_seed=5, B=4, V=500)
    parents = wl["parents"]
    tok = wl["draft_tokens"]
    kids = {}
    for n in range(1, len(parents)):
        kids.setdefault(int(parents[n]), []).append(n)
    for b in range(4):
        for p, ch in kids.items():
            vals = [int(tok[b, c]) for c in ch]
            assert len(set(vals)) == len(vals)          # distinct siblings
