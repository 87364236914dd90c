"""Oracle: greedy tree-walk acceptance with the bonus token.

Follows the serve-integration spec, sections "What's proven" and
"3. Rejection sampler: tree walk": starting at the last accepted token (the
root), take the target's argmax at the current node, move to the child whose
token equals it, and repeat; when no child matches, emit the argmax at the
current node as the bonus token.  Acceptance is exact argmax, no sampling.

Readings of the points the page leaves open:
  * logits row 0 belongs to the root (the last accepted token), row 1 + i to
    draft node i;
  * the argmax of a row is its lowest index among equal maxima;
  * if several children of the current node carry the predicted token, the
    lowest-index child is taken;
  * num_accepted counts accepted draft nodes a; a + 1 tokens are emitted,
    the bonus last.
"""
from __future__ import annotations

import numpy as np


def argmax_first(row):
    """Index of the first occurrence of the maximum of a finite row."""
    row = np.asarray(row, dtype=np.float64)
    if not np.all(np.isfinite(row)):
        raise ValueError("logits must be finite")
    best = 0
    for v in range(1, row.shape[0]):
        if row[v] > row[best]:
            best = v
    return best


def row_argmax(logits):
    """argmax over the last axis, lowest index on ties (vectorised form of
    argmax_first; numpy documents that argmax returns the first occurrence)."""
    x = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("logits must be finite")
    return np.argmax(x, axis=-1).astype(np.int64)


def children(parent, c):
    """Nodes whose parent is c, in increasing index order."""
    return [i for i in range(len(parent)) if int(parent[i]) == c]


def walk_one(tokens, parent, am):
    """Greedy walk of one sequence given the per-row argmax am [N+1].
    Returns (accepted tokens incl. bonus, accepted node indices)."""
    cur, row = -1, 0
    out_tokens, out_nodes = [], []
    while True:
        pred = int(am[row])
        nxt = None
        for i in children(parent, cur):
            if int(tokens[i]) == pred:
                nxt = i
                break
        if nxt is None:
            out_tokens.append(pred)  # bonus
            return out_tokens, out_nodes
        out_tokens.append(pred)
        out_nodes.append(nxt)
        cur, row = nxt, 1 + nxt


def tree_walk(tokens, parent, logits):
    """tokens, parent [B, N]; logits [B, N+1, V].  Returns
    accepted_tokens [B, N+1] (a+1 valid, then -1), accepted_nodes [B, N]
    (a valid, then -1), num_accepted [B]."""
    tokens = np.asarray(tokens)
    parent = np.asarray(parent)
    B, N = tokens.shape
    am = row_argmax(logits)
    acc_tok = np.full((B, N + 1), -1, dtype=np.int32)
    acc_node = np.full((B, N), -1, dtype=np.int32)
    num = np.zeros(B, dtype=np.int32)
    for b in range(B):
        t, n = walk_one(tokens[b], parent[b], am[b])
        acc_tok[b, :len(t)] = t
        acc_node[b, :len(n)] = n
        num[b] = len(n)
    return dict(accepted_tokens=acc_tok, accepted_nodes=acc_node, num_accepted=num, argmax=am)
