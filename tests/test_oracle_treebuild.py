"""Pins for the tree-construction oracle (per-depth top-k of the draft
distribution, best-first growth on cumulative log-probability)."""
import itertools

import numpy as np
import pytest

from oracle import treebuild as TB


def test_log_softmax_closed_forms():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 1000)) * 8
    lp = TB.log_softmax(z)
    np.testing.assert_allclose(np.exp(lp).sum(-1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(TB.log_softmax(z + 123.0), lp, rtol=0, atol=1e-12)
    # two tokens: log p_0 = -log(1 + exp(z_1 - z_0))
    a, b = 0.7, -1.9
    np.testing.assert_allclose(TB.log_softmax(np.array([a, b]))[0], -np.log1p(np.exp(b - a)), atol=1e-15)


def test_topk_ties_and_order():
    row = np.array([[[1.0, 3.0, 3.0, 2.0, 3.0, -5.0]]])
    tok, lp = TB.draft_topk(row, 4)
    assert tok[0, 0].tolist() == [1, 2, 4, 3]          # equal logits: lower token id first
    full = TB.log_softmax(row[0, 0])
    np.testing.assert_allclose(lp[0, 0], full[[1, 2, 4, 3]], atol=0)


def test_topk_brute_force():
    rng = np.random.default_rng(2)
    x = np.round(rng.standard_normal((2, 3, 50)) * 4) / 4   # coarse values: many ties
    tok, lp = TB.draft_topk(x, 7)
    for b in range(2):
        for d in range(3):
            ref = sorted(range(50), key=lambda v: (-x[b, d, v], v))[:7]
            assert tok[b, d].tolist() == ref


def _paths_by_score(lp):
    """Every node of the K-ary trie of depth L with its float32 cumulative
    log-probability, summed root to leaf (one rounding per step)."""
    L, K = lp.shape
    out = []
    for depth in range(1, L + 1):
        for ranks in itertools.product(range(K), repeat=depth):
            s = np.float32(0.0)
            for d, r in enumerate(ranks):
                s = np.float32(s + np.float32(lp[d, r])) if d else np.float32(lp[d, r])
            out.append((float(s), ranks))
    return out


@pytest.mark.parametrize("K,L,N", [(3, 4, 20), (2, 6, 40), (5, 3, 64), (4, 4, 128)])
def test_sequential_is_top_n_of_the_trie(K, L, N):
    """w = 1 with distinct scores: the tree is the N highest cumulative
    log-probabilities of the K-ary depth-L trie (parents always score at
    least their children and better siblings at least worse ones)."""
    rng = np.random.default_rng(K * 100 + L)
    lp = -np.sort(rng.exponential(1.0, size=(L, K)), axis=1).astype(np.float32)
    tok = np.arange(L * K).reshape(L, K) + 1000
    res = TB.tree_build(tok[None], lp[None], N, 1)
    allp = _paths_by_score(lp)
    best = sorted(allp, key=lambda e: -e[0])[:N]
    # the tree's nodes as rank tuples
    n = int(res["num_nodes"][0])
    assert n == min(N, len(allp))
    got = set()
    for t in range(n):
        ranks = []
        cur = t
        while cur >= 0:
            d = int(res["depth"][0, cur])
            ranks.append(int(np.where(tok[d - 1] == res["tokens"][0, cur])[0][0]))
            cur = int(res["parent"][0, cur])
        got.add(tuple(ranks[::-1]))
    assert got == {r for _, r in best}
    # scores are those cumulative values
    by_ranks = {r: s for s, r in allp}
    for t in range(n):
        ranks = []
        cur = t
        while cur >= 0:
            d = int(res["depth"][0, cur])
            ranks.append(int(np.where(tok[d - 1] == res["tokens"][0, cur])[0][0]))
            cur = int(res["parent"][0, cur])
        assert res["score"][0, t] == np.float32(by_ranks[tuple(ranks[::-1])])


def test_structure_and_spine():
    rng = np.random.default_rng(5)
    L, K, N = 8, 8, 64
    lp = -np.sort(rng.exponential(2.0, size=(L, K)), axis=1).astype(np.float32)
    tok = rng.permutation(10000)[:L * K].reshape(L, K)
    res = TB.tree_build(tok[None], lp[None], N, 1)
    par, dep = res["parent"][0], res["depth"][0]
    assert int(res["num_nodes"][0]) == N
    assert np.all(np.diff(dep) >= 0)                       # flattened by depth
    for t in range(N):
        assert par[t] < t
        assert dep[t] == (1 if par[t] < 0 else dep[par[t]] + 1)
    # the spine (rank 0 at every depth) is the first node of its depth
    for d in range(1, dep.max() + 1):
        first = int(np.argmax(dep == d))
        assert res["tokens"][0, first] == tok[d - 1, 0]
        if d > 1:
            assert par[first] == int(np.argmax(dep == d - 1))


def test_budget_past_the_trie():
    lp = np.array([[-0.5, -1.0], [-0.25, -2.0]], dtype=np.float32)
    res = TB.tree_build(np.array([[[1, 2], [3, 4]]]), lp[None], 10, 1)
    assert int(res["num_nodes"][0]) == 6                   # 2 + 4 nodes in the trie
    assert res["tokens"][0, 6:].tolist() == [-1] * 4 and np.all(np.isneginf(res["score"][0, 6:]))


def test_equal_scores_follow_push_order():
    """All log-probabilities equal: the queue falls back to push order.  Roots
    r0 r1 are pushed first; popping r0 pushes its first child, popping r1
    pushes its first child, and so on."""
    lp = np.full((2, 2), -1.0, dtype=np.float32)
    tok = np.array([[10, 11], [20, 21]])
    res = TB.tree_build(tok[None], lp[None], 6, 1)
    assert res["tokens"][0].tolist() == [10, 11, 20, 20, 21, 21]
    assert res["parent"][0].tolist() == [-1, -1, 0, 1, 0, 1]


def test_batched_rounds_differ_from_sequential():
    """w = 2 pops both roots in the first round, even the poor one; w = 1
    spends the budget under the good root."""
    lp = np.array([[-0.1, -5.0], [-0.01, -0.02]], dtype=np.float32)
    tok = np.array([[1, 2], [3, 4]])
    seq = TB.tree_build(tok[None], lp[None], 3, 1)
    bat = TB.tree_build(tok[None], lp[None], 3, 2)
    assert seq["tokens"][0].tolist() == [1, 3, 4] and seq["parent"][0].tolist() == [-1, 0, 0]
    assert bat["tokens"][0].tolist() == [1, 2, 3] and bat["parent"][0].tolist() == [-1, -1, 0]


@pytest.mark.parametrize("w", [1, 3, 8, 64])
def test_batched_invariants(w):
    rng = np.random.default_rng(w)
    L, K, N = 6, 4, 50
    lp = -np.sort(rng.exponential(1.0, size=(3, L, K)), axis=2).astype(np.float32)
    tok = rng.integers(0, 1000, size=(3, L, K))
    res = TB.tree_build(tok, lp, N, w)
    for b in range(3):
        par, dep = res["parent"][b], res["depth"][b]
        assert int(res["num_nodes"][b]) == N
        assert np.all(np.diff(dep) >= 0)
        for t in range(N):
            assert par[t] < t and dep[t] == (1 if par[t] < 0 else dep[par[t]] + 1)
            if par[t] >= 0:   # a node never scores above its parent
                assert res["score"][b, t] <= res["score"][b, par[t]]
