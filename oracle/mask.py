"""Oracle: ancestor-or-self tree mask, depth and position ids.

Follows the serve-integration spec (page "tree_dev/SERVE_INTEGRATION_SPEC.md"),
section "2. Verify: tree attention mask": a node sees the whole context and,
among the draft nodes, exactly its ancestors and itself; its position id is
ctx_len - 1 + depth.  Section "Layout contract": parent[i] is a node index,
-1 meaning the node hangs under the last accepted token, and nodes are
flattened by depth.  The DDTree validation post ("The Successful Test") prints
depth 1 for every node whose parent is -1, which fixes the depth origin.

Trees of up to 128 nodes are covered: the ancestor set of a node is packed
into ceil(N / 64) 64-bit words, word w holding nodes 64 w .. 64 w + 63 (bit
j % 64 of word j // 64 stands for node j).  The pages' trees stop near 32
nodes; 128 is the tree size the DFlash-TfM summary measures its fused GDN
verify at.

Status codes per sequence (the same numbering as the library):
  0 ok, 1 a parent index outside [-1, i), 2 a given depth that differs from
  the derived one, 3 ctx_len < 1.  Checks apply in that order; the first that
  fails is reported.  A sequence with status 1 gets the star-tree fallback
  (every node sees only itself, depth 1); otherwise the derived values are
  reported even when the status is 2 or 3.
"""
from __future__ import annotations

import numpy as np

TREE_OK, TREE_BAD_PARENT, TREE_BAD_DEPTH, TREE_BAD_CTX = 0, 1, 2, 3


def path_to_root(parent, t):
    """Set P(t): t and every node reached by following parent pointers."""
    seen = []
    cur = int(t)
    while cur != -1:
        seen.append(cur)
        cur = int(parent[cur])
    return seen


def anc_words(nodes, n):
    """Pack a set of node indices into ceil(n / 64) uint64 words."""
    w = np.zeros((n + 63) // 64, dtype=np.uint64)
    for j in nodes:
        w[j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return w


def anc_value(words):
    """The packed words of one node as one Python integer (bit j = node j)."""
    return sum(int(x) << (64 * i) for i, x in enumerate(np.asarray(words, dtype=np.uint64)))


def tree_mask(parent, ctx_len, depth_in=None):
    """Returns dict with
       vis    bool   [B, N, N]  vis[b, t, j] = (j is t or an ancestor of t)
       anc    uint64 [B, N, W]  visible j packed into W = ceil(N / 64) words
       depth  int32  [B, N]     |P(t)|
       pos    int64  [B, N]     ctx_len[b] - 1 + depth
       status int32  [B]
    """
    parent = np.asarray(parent, dtype=np.int64)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    B, N = parent.shape
    vis = np.zeros((B, N, N), dtype=bool)
    anc = np.zeros((B, N, (N + 63) // 64), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    pos = np.zeros((B, N), dtype=np.int64)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        par = parent[b]
        bad_parent = any(not (-1 <= par[i] < i) for i in range(N))
        if bad_parent:
            status[b] = TREE_BAD_PARENT
            for t in range(N):
                vis[b, t, t] = True
                anc[b, t] = anc_words([t], N)
                depth[b, t] = 1
                pos[b, t] = ctx_len[b]
            continue
        for t in range(N):
            P = path_to_root(par, t)
            for j in P:
                vis[b, t, j] = True
            anc[b, t] = anc_words(P, N)
            depth[b, t] = len(P)
            pos[b, t] = ctx_len[b] - 1 + len(P)
        if depth_in is not None and np.any(np.asarray(depth_in)[b] != depth[b]):
            status[b] = TREE_BAD_DEPTH
        elif ctx_len[b] < 1:
            status[b] = TREE_BAD_CTX
    return dict(vis=vis, anc=anc, depth=depth, pos=pos, status=status)


def dense_mask(vis_b, ctx_len):
    """Full boolean mask of one sequence, shape [N, ctx_len + N]: every context
    column is visible, node column j iff j is an ancestor-or-self."""
    N = vis_b.shape[0]
    out = np.zeros((N, int(ctx_len) + N), dtype=bool)
    out[:, :ctx_len] = True
    out[:, ctx_len:] = vis_b
    return out


def node_bias(vis):
    """The N x N additive node-block bias: 0 where visible, -inf elsewhere."""
    return np.where(vis, 0.0, -np.inf)
