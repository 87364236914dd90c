"""Pins for the tree-walk oracle.

The main pin is greedy identity (serve-integration spec, "What's proven"):
for any tree the walk emits exactly the tokens plain greedy decoding would,
under a deterministic toy target.  Brute force over root paths, tie rules and
the DDTree post's printed acceptance line are checked as well.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

from oracle import walk as Wk
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ddtree_worked_example.json")


def toy_target(prefix, vocab):
    """Deterministic 'model': next token = hash(prefix) mod vocab."""
    h = hashlib.blake2b(np.asarray(prefix, dtype=np.int64).tobytes(), digest_size=8).digest()
    return int.from_bytes(h, "little") % vocab


def greedy_decode(history, steps, vocab):
    seq = list(history)
    out = []
    for _ in range(steps):
        nxt = toy_target(seq, vocab)
        out.append(nxt)
        seq.append(nxt)
    return out


def logits_from_target(history, tokens, parent, vocab, rng, ties=False):
    """Row 0: the target's prediction after the history; row 1+i: after
    history ++ (root path of node i).  The predicted token gets the unique
    maximum (noise below it), or with ``ties`` a tie with a later index."""
    N = len(tokens)
    L = rng.standard_normal((N + 1, vocab))
    for r in range(N + 1):
        if r == 0:
            pre = list(history)
        else:
            path = []
            cur = r - 1
            while cur >= 0:
                path.append(int(tokens[cur]))
                cur = int(parent[cur])
            pre = list(history) + path[::-1]
        tgt = toy_target(pre, vocab)
        top = L[r].max() + 1.0
        L[r, tgt] = top
        if ties:
            later = np.arange(tgt + 1, vocab)
            if len(later):
                L[r, rng.choice(later, size=min(3, len(later)), replace=False)] = top
    return L


def plant_greedy_path(tokens, parent, history, vocab, rng, depth_hint=None):
    """Overwrite the tokens of one random root path so that it follows greedy
    decoding for a random number of steps (makes walks go deep)."""
    N = len(tokens)
    leaf = int(rng.integers(0, N))
    path = []
    cur = leaf
    while cur >= 0:
        path.append(cur)
        cur = int(parent[cur])
    path = path[::-1]
    k = len(path) if depth_hint is None else min(depth_hint, len(path))
    g = greedy_decode(history, k, vocab)
    tokens = tokens.copy()
    for i in range(k):
        tokens[path[i]] = g[i]
    return tokens


def check_greedy_identity(tokens, parent, history, vocab, rng, ties=False):
    L = logits_from_target(history, tokens, parent, vocab, rng, ties=ties)
    r = Wk.tree_walk(tokens[None], parent[None], L[None])
    a = int(r["num_accepted"][0])
    toks = r["accepted_tokens"][0, :a + 1].tolist()
    assert toks == greedy_decode(history, a + 1, vocab)
    assert np.all(r["accepted_tokens"][0, a + 1:] == -1)
    nodes = r["accepted_nodes"][0, :a].tolist()
    assert np.all(r["accepted_nodes"][0, a:] == -1)
    # the accepted nodes form a root path carrying the accepted tokens
    prev = -1
    for i, n in enumerate(nodes):
        assert parent[n] == prev and tokens[n] == toks[i]
        prev = n
    # maximality: no child of the last accepted node carries the bonus token
    assert not any(parent[i] == prev and tokens[i] == toks[-1] for i in range(len(tokens)))
    return a


@pytest.mark.parametrize("kind,n", [("random_parent", 16), ("spine_first", 32),
                                    ("leaf_sibling", 32), ("random_parent", 64), ("chain", 8),
                                    ("random_parent", 128)])
def test_greedy_identity_random_trees(kind, n):
    vocab = 50
    tb = W.make_trees(21, kind, 40, n, vocab, max_depth=8)
    rng = np.random.default_rng(3)
    depths = []
    for b in range(40):
        hist = rng.integers(0, vocab, size=5).tolist()
        toks = plant_greedy_path(tb.tokens[b], tb.parent[b], hist, vocab, rng,
                                 depth_hint=int(rng.integers(0, 9)))
        depths.append(check_greedy_identity(toks, tb.parent[b], hist, vocab, rng,
                                            ties=bool(b % 2)))
    assert max(depths) >= 2  # the planted paths make walks go deep


def _linear_dfs_scan(tokens, parent, am):
    """The chain-style scan the DDTree post warns about: walk nodes in index
    order and stop at the first node that does not match.  Used only as a
    contrast: it is NOT the tree walk."""
    out, cur, row = [], -1, 0
    for i in range(len(tokens)):
        if parent[i] != cur:
            continue
        if tokens[i] != am[row]:
            break
        out.append(int(tokens[i]))
        cur, row = i, 1 + i
    return out


def test_adversarial_cases():
    vocab = 40
    rng = np.random.default_rng(9)
    hist = [1, 2, 3]
    g = greedy_decode(hist, 10, vocab)
    other = [t for t in range(vocab) if t not in g]

    # matching child is the last sibling of a star
    toks = np.array(other[:5] + [g[0]])
    par = np.full(6, -1)
    assert check_greedy_identity(toks, par, hist, vocab, rng) == 1

    # duplicate sibling tokens: the first of the two is accepted
    toks = np.array([other[0], g[0], g[0], g[1]])
    par = np.array([-1, -1, -1, 2])
    L = logits_from_target(hist, toks, par, vocab, rng)
    r = Wk.tree_walk(toks[None], par[None], L[None])
    assert r["accepted_nodes"][0, 0] == 1 and r["num_accepted"][0] == 1

    # cousin trap: the right depth-2 token sits under a non-accepted node
    toks = np.array([g[0], other[0], other[1], g[1]])
    par = np.array([-1, -1, 0, 1])
    a = check_greedy_identity(toks, par, hist, vocab, rng)
    assert a == 1
    # siblings must be checked: an index-order scan that stops at the first
    # mismatch rejects a tree whose matching node is not the first sibling
    toks2 = np.array([other[0], g[0], other[1], g[1]])
    par2 = np.array([-1, -1, 1, 1])
    L2 = logits_from_target(hist, toks2, par2, vocab, rng)
    r2 = Wk.tree_walk(toks2[None], par2[None], L2[None])
    assert r2["num_accepted"][0] == 2
    assert _linear_dfs_scan(toks2, par2, Wk.row_argmax(L2)) != r2["accepted_tokens"][0, :2].tolist()

    # full-depth acceptance of a chain, with the bonus after the last node
    toks = np.array(g[:7])
    par = np.arange(-1, 6)
    assert check_greedy_identity(toks, par, hist, vocab, rng) == 7

    # zero acceptance: only the bonus
    toks = np.array(other[:4])
    par = np.array([-1, 0, -1, 2])
    assert check_greedy_identity(toks, par, hist, vocab, rng) == 0

    # a single node, matching and not matching
    assert check_greedy_identity(np.array([g[0]]), np.array([-1]), hist, vocab, rng) == 1
    assert check_greedy_identity(np.array([other[0]]), np.array([-1]), hist, vocab, rng) == 0

    # tokens outside the vocabulary never match
    assert check_greedy_identity(np.array([-5, vocab + 3]), np.array([-1, -1]), hist, vocab, rng) == 0


@pytest.mark.parametrize("n", [64, 128])
def test_max_nodes_chain(n):
    vocab = 1000
    hist = [7]
    g = greedy_decode(hist, n + 1, vocab)
    toks = np.array(g[:n])
    par = np.arange(-1, n - 1)
    rng = np.random.default_rng(0)
    assert check_greedy_identity(toks, par, hist, vocab, rng) == n


def _brute_force(tokens, parent, am):
    """Enumerate every root path; keep those whose every node carries the
    argmax of its parent's row; return the deepest one."""
    N = len(tokens)
    best = []
    for leaf in range(N):
        path = []
        cur = leaf
        while cur >= 0:
            path.append(cur)
            cur = int(parent[cur])
        path = path[::-1]
        for k in range(1, len(path) + 1):
            pre = path[:k]
            rows = [0] + [1 + p for p in pre[:-1]]
            if all(tokens[pre[i]] == am[rows[i]] for i in range(k)) and k > len(best):
                best = pre
    return best


def test_brute_force_small_trees():
    """Trees whose siblings carry distinct tokens have at most one matching
    path; the walk must return the deepest matching root path."""
    rng = np.random.default_rng(17)
    vocab = 4
    for trial in range(300):
        n = int(rng.integers(1, 9))
        parent = np.array([int(rng.integers(-1, i)) for i in range(n)])
        tokens = np.empty(n, dtype=np.int64)
        for c in range(-1, n):
            kids = [i for i in range(n) if parent[i] == c]
            tokens[kids] = rng.permutation(vocab)[:len(kids)] if len(kids) <= vocab else 0
        if any(len([i for i in range(n) if parent[i] == c]) > vocab for c in range(-1, n)):
            continue
        L = rng.integers(0, 3, size=(n + 1, vocab)).astype(np.float64)  # many ties
        r = Wk.tree_walk(tokens[None], parent[None], L[None])
        am = np.array([int(torch.argmax(torch.from_numpy(L[i]))) for i in range(n + 1)])
        best = _brute_force(tokens, parent, am)
        a = int(r["num_accepted"][0])
        assert r["accepted_nodes"][0, :a].tolist() == best
        last_row = 0 if not best else 1 + best[-1]
        assert r["accepted_tokens"][0, a] == am[last_row]


def test_argmax_ties_first_occurrence():
    """Ties go to the lowest index, as torch.argmax documents; checked on
    bf16-rounded rows where ties are frequent."""
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((200, 5000)).astype(np.float32)).to(torch.bfloat16)
    got = Wk.row_argmax(x.double().numpy())
    ref = torch.argmax(x.float(), dim=-1).numpy()
    assert np.array_equal(got, ref)
    ties = sum(int((x[i] == x[i].max()).sum()) > 1 for i in range(200))
    assert ties > 0
    for i in range(5):
        assert Wk.argmax_first(x[i].double().numpy()) == got[i]


def test_worked_example_acceptance_line():
    """The DDTree post prints 'Accepted 2 tokens: [701, 701]' for its tree
    without printing the target logits.  Under a logit table where the root's
    argmax is 701 (node 0's token) and node 0's argmax is a token none of its
    children carry (the unprinted node tokens are drawn avoiding 701), our
    reading emits [701, 701]: one accepted node plus the bonus.  This only
    shows the reading is consistent with the print; the line itself is
    parity unpinned."""
    g = json.load(open(GOLDEN))
    par = np.array(g["parents"])
    rng = np.random.default_rng(0)
    toks = np.array(g["tokens_first10"] + [int(t) for t in rng.integers(0, 700, size=22)])
    L = rng.standard_normal((33, 1000))
    L[0, 701] = 10.0
    L[1, 701] = 10.0
    r = Wk.tree_walk(toks[None], par[None], L[None])
    a = int(r["num_accepted"][0])
    assert r["accepted_tokens"][0, :a + 1].tolist() == g["accepted_tokens"]
    assert a == 1


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        Wk.row_argmax(np.array([[0.0, np.nan]]))
