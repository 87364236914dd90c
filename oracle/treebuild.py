"""Oracle: draft-tree construction (test infrastructure only).

Follows the DDTree validation post ("From Linear to Tree-Walk"), section
"The Failed First Attempt", which describes the construction under test:
the tree grows best-first from a priority queue on cumulative
log-probability, starting from the top-k tokens of the first position as
roots; each popped node joins the tree and its siblings and children go
back on the queue, until the node budget is spent or a maximum depth stops
the growth.  The DFlash-TfM summary, section "2. Boomconstructie", batches
this: the top-w candidates leave the queue at once and are expanded
together, so a budget of n nodes takes ceil(n / w) rounds.  The draft
distribution is factorised per depth (the summary's "trees from
marginals"): depth d has one list of K candidates, the same under every
parent.

Readings of the points the pages leave open:
  * candidates of a depth: the K tokens of largest draft logit, ties to the
    lower token id; their log-probabilities are the log-softmax over the
    whole vocabulary;
  * the queue starts with the K depth-1 candidates (the roots) in rank
    order; a popped node of depth d >= 2 pushes its next sibling (same
    parent, next rank), and a popped node below the maximum depth pushes its
    first child (rank 0 of depth d + 1); depth-1 siblings are already queued;
  * the queue orders by cumulative log-probability, higher first, equal
    values in push order; cumulative values are sums in float32 (the
    parent's value plus the candidate's log-probability, one rounding per
    node), the precision in which the GPU takes the same decisions;
  * a round pops min(w, budget left, queue size) candidates in queue order,
    then pushes the successors of each popped node in pop order;
  * output order: pop order, stable-sorted by depth (the first node popped
    at each depth comes first), parents renumbered; parent -1 marks a child
    of the last accepted token.
"""
from __future__ import annotations

import heapq

import numpy as np


def log_softmax(z):
    """log p_v = z_v - log sum_u exp(z_u), in float64 with the maximum
    subtracted first."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


def draft_topk(logits, K):
    """logits [B, L, V] -> (tokens int64 [B, L, K], logprob float64 [B, L, K]):
    per (sequence, depth) the K largest logits, ties to the lower token id,
    with their log-softmax values."""
    x = np.asarray(logits, dtype=np.float64)
    B, L, V = x.shape
    tok = np.empty((B, L, K), dtype=np.int64)
    lp = np.empty((B, L, K), dtype=np.float64)
    for b in range(B):
        for d in range(L):
            row = x[b, d]
            order = np.argsort(-row, kind="stable")[:K]  # stable: equal values keep index order
            tok[b, d] = order
            lp[b, d] = log_softmax(row)[order]
    return tok, lp


def build_one(cand_tok, cand_lp, N, w):
    """One sequence: cand_tok [L, K], cand_lp [L, K] (float32 values) ->
    (tokens, parent, depth, score) lists in output order."""
    L, K = cand_tok.shape
    lp = np.asarray(cand_lp, dtype=np.float32)
    heap = []          # (-score, push counter, depth, rank, parent pop index)
    counter = 0
    for r in range(K):
        heapq.heappush(heap, (-float(lp[0, r]), counter, 1, r, -1))
        counter += 1
    popped = []        # (score, depth, rank, parent pop index)
    while heap and len(popped) < N:
        take = min(w, N - len(popped), len(heap))
        batch = [heapq.heappop(heap) for _ in range(take)]
        first = len(popped)
        for (neg, _, d, r, par) in batch:
            popped.append((np.float32(-neg), d, r, par))
        for i, (neg, _, d, r, par) in enumerate(batch):
            me = first + i
            score = np.float32(-neg)
            if d >= 2 and r + 1 < K:
                s = np.float32(popped[par][0] + lp[d - 1, r + 1])
                heapq.heappush(heap, (-float(s), counter, d, r + 1, par))
                counter += 1
            if d < L:
                s = np.float32(score + lp[d, 0])
                heapq.heappush(heap, (-float(s), counter, d + 1, 0, me))
                counter += 1
    # stable sort by depth, parents renumbered
    order = sorted(range(len(popped)), key=lambda i: popped[i][1])
    new = {old: k for k, old in enumerate(order)}
    tokens, parent, depth, score = [], [], [], []
    for old in order:
        sc, d, r, par = popped[old]
        tokens.append(int(cand_tok[d - 1, r]))
        parent.append(-1 if par < 0 else new[par])
        depth.append(d)
        score.append(float(sc))
    return tokens, parent, depth, score


def tree_build(cand_tok, cand_lp, N, w=1):
    """Batched form: cand_tok [B, L, K], cand_lp [B, L, K] -> dict of
    tokens, parent, depth (int64 [B, N]; -1, -1, 0 past the tree), score
    (float32 [B, N]; -inf past the tree) and num_nodes [B]."""
    cand_tok = np.asarray(cand_tok)
    B = cand_tok.shape[0]
    out = dict(tokens=np.full((B, N), -1, dtype=np.int64), parent=np.full((B, N), -1, dtype=np.int64),
               depth=np.zeros((B, N), dtype=np.int64), score=np.full((B, N), -np.inf, dtype=np.float32),
               num_nodes=np.zeros(B, dtype=np.int64))
    for b in range(B):
        t, p, d, s = build_one(cand_tok[b], cand_lp[b], N, w)
        n = len(t)
        out["tokens"][b, :n] = t
        out["parent"][b, :n] = p
        out["depth"][b, :n] = d
        out["score"][b, :n] = s
        out["num_nodes"][b] = n
    return out
