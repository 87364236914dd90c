"""Pins for the mask oracle (ancestor-or-self mask, depth, position ids)."""
import json
import os

import numpy as np
import pytest

from oracle import mask as M
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ddtree_worked_example.json")


def test_worked_example_depths():
    """DDTree validation post, 'The Successful Test': the printed parents must
    give exactly the printed depths (10 nodes at depth 1, 22 at depth 2)."""
    g = json.load(open(GOLDEN))
    par = np.array([g["parents"]])
    r = M.tree_mask(par, [100])
    assert r["status"][0] == 0
    assert r["depth"][0].tolist() == g["depths"]
    assert (r["depth"][0] == 1).sum() == 10 and (r["depth"][0] == 2).sum() == 22


def test_worked_example_mask_shape():
    """Same post: the dense mask is [1, 1, 32, 132], read as 32 nodes over
    100 context + 32 node columns."""
    g = json.load(open(GOLDEN))
    par = np.array([g["parents"]])
    ctx = g["mask_context_len_reading"]
    r = M.tree_mask(par, [ctx])
    dense = M.dense_mask(r["vis"][0], ctx)[None, None]
    assert list(dense.shape) == g["mask_shape"]
    # depth-2 node 10 (parent 0) sees node 0 and itself, not node 16 (a sibling)
    assert dense[0, 0, 10, ctx + 0] and dense[0, 0, 10, ctx + 10]
    assert not dense[0, 0, 10, ctx + 16] and not dense[0, 0, 10, ctx + 1]


@pytest.mark.parametrize("n", [1, 2, 7, 32, 64, 65, 128])
def test_chain_is_lower_triangular(n):
    par = np.arange(-1, n - 1)[None]
    r = M.tree_mask(par, [37])
    assert np.array_equal(r["vis"][0], np.tril(np.ones((n, n), dtype=bool)))
    assert r["depth"][0].tolist() == list(range(1, n + 1))
    assert r["pos"][0].tolist() == list(range(37, 37 + n))


@pytest.mark.parametrize("n", [1, 5, 64, 100, 128])
def test_star_is_identity(n):
    r = M.tree_mask(np.full((1, n), -1), [9])
    assert np.array_equal(r["vis"][0], np.eye(n, dtype=bool))
    assert np.all(r["depth"] == 1) and np.all(r["pos"] == 9)
    assert [M.anc_value(w) for w in r["anc"][0]] == [1 << i for i in range(n)]
    assert r["anc"].shape == (1, n, (n + 63) // 64)


def test_word_layout():
    """Node j is bit j % 64 of word j // 64: the chain's node 100 holds nodes
    0..63 in word 0 and 64..100 in word 1."""
    r = M.tree_mask(np.arange(-1, 127)[None], [1])
    w = r["anc"][0, 100]
    assert int(w[0]) == (1 << 64) - 1 and int(w[1]) == (1 << 37) - 1
    assert r["anc"][0, 63].tolist() == [(1 << 64) - 1, 0]
    assert r["anc"][0, 64].tolist() == [(1 << 64) - 1, 1]


def test_leaf_sibling_closed_form():
    """Spine of depth 8 with 3 extra candidates per position: a node of depth
    d sees the spine nodes of depth < d and itself only."""
    tb = W.make_trees(2, "leaf_sibling", 1, 32, 1000)
    r = M.tree_mask(tb.parent, [4096])
    vis = r["vis"][0]
    for t in range(32):
        d = t // 4 + 1
        expect = {4 * (e - 1) for e in range(1, d)} | {t}
        assert set(np.flatnonzero(vis[t]).tolist()) == expect
    assert np.array_equal(r["depth"][0], tb.depth[0])


def _ancestor_matrix_by_powers(par):
    """Independent form: with A[t, p] = 1 for p = parent(t), the set of
    ancestors-or-self is the support of I + A + A^2 + ... (A is nilpotent)."""
    n = len(par)
    A = np.zeros((n, n), dtype=np.int64)
    for t, p in enumerate(par):
        if p >= 0:
            A[t, p] = 1
    acc = np.eye(n, dtype=np.int64)
    Ak = np.eye(n, dtype=np.int64)
    for _ in range(n):
        Ak = Ak @ A
        acc += Ak
    return acc > 0


@pytest.mark.parametrize("kind,n", [("random_parent", 16), ("random_parent", 64),
                                    ("spine_first", 32), ("ddtree", 24), ("random_parent", 128),
                                    ("ddtree", 128), ("random_parent", 77)])
def test_against_matrix_powers_and_invariants(kind, n):
    kw = dict(max_depth=8) if kind == "spine_first" else {}
    vocab = 64 if kind == "ddtree" else 1000
    tb = W.make_trees(7, kind, 3, n, vocab, **kw)
    ctx = np.array([5, 100, 3000])
    r = M.tree_mask(tb.parent, ctx)
    assert np.all(r["status"] == 0)
    for b in range(3):
        par = tb.parent[b]
        vis = r["vis"][b]
        assert np.array_equal(vis, _ancestor_matrix_by_powers(par))
        # popcount(anc) == depth; anc is the packed row of vis
        for t in range(n):
            a = M.anc_value(r["anc"][b, t])
            assert bin(a).count("1") == r["depth"][b, t]
            assert a == sum(1 << int(j) for j in np.flatnonzero(vis[t]))
            # recurrence: own bit plus the parent's set
            if par[t] >= 0:
                assert a == (1 << t) | M.anc_value(r["anc"][b, par[t]])
                assert r["depth"][b, t] == r["depth"][b, par[t]] + 1
            else:
                assert a == 1 << t and r["depth"][b, t] == 1
        assert np.array_equal(r["pos"][b], ctx[b] - 1 + r["depth"][b])
        if tb.depth is not None:
            assert np.array_equal(r["depth"][b], tb.depth[b])


def test_status_codes():
    ok = np.array([-1, 0, 0, 1])
    cases = [
        (np.array([[-1, 1, 0, 1]]), None, [5], M.TREE_BAD_PARENT),   # parent == self
        (np.array([[-1, 0, 3, 1]]), None, [5], M.TREE_BAD_PARENT),   # forward parent
        (np.array([[-2, 0, 0, 1]]), None, [5], M.TREE_BAD_PARENT),   # below -1
        (ok[None], np.array([[1, 2, 2, 2]]), [5], M.TREE_BAD_DEPTH),
        (ok[None], np.array([[1, 2, 2, 3]]), [0], M.TREE_BAD_CTX),
        (ok[None], np.array([[1, 2, 2, 3]]), [5], M.TREE_OK),
        (np.array([[-1, 1, 0, 1]]), np.array([[9, 9, 9, 9]]), [0], M.TREE_BAD_PARENT),  # order
        (ok[None], np.array([[1, 1, 2, 3]]), [0], M.TREE_BAD_DEPTH),
    ]
    for par, dep, ctx, code in cases:
        r = M.tree_mask(par, ctx, dep)
        assert r["status"][0] == code, (par, dep, ctx)
    # star fallback on a bad parent
    r = M.tree_mask(np.array([[-1, 1, 0, 1]]), [5])
    assert np.array_equal(r["vis"][0], np.eye(4, dtype=bool)) and np.all(r["depth"] == 1)


def test_node_bias():
    r = M.tree_mask(np.array([[-1, 0, -1]]), [3])
    bias = M.node_bias(r["vis"][0])
    assert bias[1, 0] == 0.0 and bias[1, 1] == 0.0 and np.isneginf(bias[1, 2])
    assert np.isneginf(bias[0, 1]) and np.isneginf(bias[2, 0])
