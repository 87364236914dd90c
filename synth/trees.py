"""Seeded draft-tree generators (test and benchmark inputs only).

Each generator returns ``parent`` (int32 [N], -1 = child of the last accepted
token), ``tokens`` (int32 [N]) and, where the construction fixes it, the
``depth`` it built each node at (int32 [N]; None where the tree shape is drawn
without reference to depth).  Nothing here verifies a tree: the ancestor
mask, positions and depth derivation of the verify step live in the library
and, independently, in the oracle.

Tree shapes follow the workloads the pages describe:

* random parents (each parent drawn uniformly among the earlier nodes or -1);
* the leaf-sibling tree of the serve-integration spec (a spine plus top-W
  candidates per spine position), page 1, "What's proven" and "1. Proposer";
* a random spine-first tree (a spine of fixed depth, the remaining nodes
  hung under uniformly chosen shallower nodes, then flattened spine-first per
  depth as the page 1 "Layout contract" asks);
* the DDTree best-first heap expansion over per-depth draft marginals,
  page 2, "The Failed First Attempt" (priority queue on cumulative log
  probability; pop, then push the next sibling and the first child).
"""
from __future__ import annotations

import heapq

import numpy as np


def rng_for(config: int, tag: int, index: int = 0) -> np.random.Generator:
    """PCG64 stream for (workload id, tensor tag, sequence index)."""
    return np.random.default_rng([int(config), int(tag), int(index) + 1])


def _flatten_by_depth(parent_list, depth_list, tokens_list, spine_nodes):
    """Stable-sort nodes by depth, spine node first within each depth, and
    remap parent indices to the new order."""
    n = len(parent_list)
    spine = set(spine_nodes)
    order = sorted(range(n), key=lambda i: (depth_list[i], 0 if i in spine else 1, i))
    new_index = {old: new for new, old in enumerate(order)}
    parent = np.array(
        [-1 if parent_list[o] < 0 else new_index[parent_list[o]] for o in order], dtype=np.int32
    )
    depth = np.array([depth_list[o] for o in order], dtype=np.int32)
    tokens = np.array([tokens_list[o] for o in order], dtype=np.int32)
    return parent, tokens, depth


def random_parent_tree(rng: np.random.Generator, n: int, vocab: int):
    """parent[i] uniform over {-1, ..., i-1}; tokens uniform in [0, vocab)."""
    parent = np.array([rng.integers(-1, i) if i > 0 else -1 for i in range(n)], dtype=np.int32)
    tokens = rng.integers(0, vocab, size=n).astype(np.int32)
    return parent, tokens, None


def chain_tree(rng: np.random.Generator, n: int, vocab: int):
    """A single path of n nodes (the chain-speculation special case)."""
    parent = np.arange(-1, n - 1, dtype=np.int32)
    tokens = rng.integers(0, vocab, size=n).astype(np.int32)
    depth = np.arange(1, n + 1, dtype=np.int32)
    return parent, tokens, depth


def star_tree(rng: np.random.Generator, n: int, vocab: int):
    """n candidates that all hang directly under the last accepted token."""
    parent = np.full(n, -1, dtype=np.int32)
    tokens = rng.integers(0, vocab, size=n).astype(np.int32)
    depth = np.ones(n, dtype=np.int32)
    return parent, tokens, depth


def leaf_sibling_tree(rng: np.random.Generator, spine_depth: int, width: int, vocab: int):
    """Spine of ``spine_depth`` nodes; at every spine position ``width - 1``
    extra candidates share the spine node's parent.  Node width*(d-1) is the
    spine node of depth d, followed by its siblings."""
    parent, depth = [], []
    for d in range(1, spine_depth + 1):
        par = -1 if d == 1 else width * (d - 2)
        for _ in range(width):
            parent.append(par)
            depth.append(d)
    n = len(parent)
    tokens = rng.integers(0, vocab, size=n).astype(np.int32)
    return np.array(parent, dtype=np.int32), tokens, np.array(depth, dtype=np.int32)


def spine_first_tree(rng: np.random.Generator, n: int, max_depth: int, vocab: int):
    """A spine of ``max_depth`` nodes, then ``n - max_depth`` nodes each hung
    under a uniformly chosen existing node of depth < max_depth; flattened
    spine-first per depth."""
    assert 1 <= max_depth <= n
    parent_l, depth_l = [], []
    for d in range(1, max_depth + 1):
        parent_l.append(-1 if d == 1 else d - 2)
        depth_l.append(d)
    spine = list(range(max_depth))
    for _ in range(n - max_depth):
        # the candidate attach points: -1 (the last accepted token) or any
        # node still shallower than max_depth
        cands = [-1] + [i for i in range(len(parent_l)) if depth_l[i] < max_depth]
        par = cands[int(rng.integers(0, len(cands)))]
        parent_l.append(par)
        depth_l.append(1 if par < 0 else depth_l[par] + 1)
    tokens_l = rng.integers(0, vocab, size=n).astype(np.int32).tolist()
    return _flatten_by_depth(parent_l, depth_l, tokens_l, spine)


def ddtree(rng: np.random.Generator, vocab: int, top_k: int, budget: int, max_depth: int,
           sigma: float = 8.0):
    """Best-first tree over factorised per-depth draft marginals.

    For every depth d the draft logits are sigma * N(0, 1) over ``vocab``;
    their log-softmax top-``top_k`` gives the candidate tokens of depth d in
    decreasing probability.  A heap ordered on -(cumulative log prob), ties
    broken by push order, starts with the best depth-1 candidate; each pop
    appends a node and pushes its next sibling and its first child.  The
    result is flattened by depth (the spine, i.e. the first node popped at each
    depth, comes first)."""
    cand_tok = np.empty((max_depth, top_k), dtype=np.int64)
    cand_lp = np.empty((max_depth, top_k), dtype=np.float64)
    for d in range(max_depth):
        z = rng.standard_normal(vocab, dtype=np.float32).astype(np.float64) * sigma
        zmax = z.max()
        lse = zmax + np.log(np.exp(z - zmax).sum())
        top = np.argsort(-z, kind="stable")[:top_k]
        cand_tok[d] = top
        cand_lp[d] = z[top] - lse
    parent_l, depth_l, tok_l, score_l = [], [], [], []
    heap = []
    counter = 0
    heapq.heappush(heap, (-cand_lp[0, 0], counter, 1, 0, -1))
    counter += 1
    first_at_depth = {}
    while heap and len(parent_l) < budget:
        neg, _, d, r, par = heapq.heappop(heap)
        me = len(parent_l)
        parent_l.append(par)
        depth_l.append(d)
        tok_l.append(int(cand_tok[d - 1, r]))
        score_l.append(-neg)
        first_at_depth.setdefault(d, me)
        base = 0.0 if par < 0 else score_l[par]
        if r + 1 < top_k:
            heapq.heappush(heap, (-(base + cand_lp[d - 1, r + 1]), counter, d, r + 1, par))
            counter += 1
        if d < max_depth:
            heapq.heappush(heap, (-(score_l[me] + cand_lp[d, 0]), counter, d + 1, 0, me))
            counter += 1
    spine = list(first_at_depth.values())
    return _flatten_by_depth(parent_l, depth_l, tok_l, spine)
