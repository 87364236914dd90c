"""Oracle: tree-masked attention over a paged context (float64).

Follows the serve-integration spec, section "2. Verify: tree attention mask":
every draft node attends to all committed context keys and, among the draft
nodes, only to its ancestors and itself, never to siblings or cousins; the
mask composes with the layer's sliding window.

Readings of the points the page leaves open:
  * context position j of sequence b lives in page block_table[b][j // 16],
    slot j % 16; its key/value for kv head g is k_cache[page, g, slot, :];
  * query head h reads kv head h // (Hq / Hkv);
  * a key at position k is visible to a query at position p iff
    0 <= p - k < W; W <= 0 means no window.  The same rule applies to node
    keys, with their own position ids;
  * scores are scale * <q, k>; no soft cap; q and k arrive already rotated.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def context_kv(k_cache, v_cache, block_table_b, g, ctx):
    """Gather the ctx context keys/values of one sequence and kv head: position
    j lives in page block_table_b[j // 16], slot j % 16."""
    D = k_cache.shape[-1]
    j = np.arange(ctx)
    pages = np.asarray(block_table_b)[j // BLOCK].astype(np.int64)
    K = np.asarray(k_cache[pages, g, j % BLOCK], dtype=np.float64).reshape(ctx, D)
    V = np.asarray(v_cache[pages, g, j % BLOCK], dtype=np.float64).reshape(ctx, D)
    return K, V


def visible_keys(p, ctx, vis_t, pos_nodes, window):
    """Boolean visibility of the ctx context keys and the N node keys for a
    query at position p whose ancestor-or-self set is vis_t."""
    kpos = np.arange(ctx)
    ctx_vis = np.ones(ctx, dtype=bool)
    node_vis = vis_t.copy()
    if window > 0:
        ctx_vis &= (p - kpos < window) & (p - kpos >= 0)
        node_vis &= (p - pos_nodes < window) & (p - pos_nodes >= 0)
    return ctx_vis, node_vis


def tree_attn_group(q_g, Kc, Vc, Kn, Vn, vis, pos, window, scale, nodes=None):
    """One (sequence, kv head): q_g [N, G, D] (the G query heads of the
    group), Kc/Vc [ctx, D] context, Kn/Vn [N, D] node keys/values, vis [N, N],
    pos [N].  Returns [N, G, D]; rows not in ``nodes`` are left as NaN.

    Every query row (node t, head) takes the softmax of scale * <q, k> over
    the keys visible to t (``visible_keys``) and the weighted sum of their
    values; all rows of the group are written as one score matrix with the
    invisible keys at -inf.  Keys that no row sees are left out of it."""
    N, G, D = q_g.shape
    ctx = Kc.shape[0]
    out = np.full((N, G, D), np.nan)
    rows = list(range(N)) if nodes is None else list(nodes)
    if not rows:
        return out
    K = np.concatenate([Kc, Kn], axis=0)
    V = np.concatenate([Vc, Vn], axis=0)
    allowed = np.stack([np.concatenate(visible_keys(int(pos[t]), ctx, vis[t], pos, window))
                        for t in rows])                            # [R, ctx + N]
    cols = np.flatnonzero(allowed.any(axis=0))
    Q = np.asarray(q_g, dtype=np.float64)[rows].reshape(len(rows) * G, D)
    s = scale * (Q @ K[cols].T)                                    # [R * G, C]
    s = np.where(np.repeat(allowed[:, cols], G, axis=0), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=1, keepdims=True)
    out[rows] = (w @ V[cols]).reshape(len(rows), G, D)
    return out


def tree_attn(q, k_node, v_node, k_cache, v_cache, block_table, ctx_len, vis, pos,
              window, scale):
    """Whole layer.  q [B, N, Hq, D]; k_node, v_node [B, N, Hkv, D];
    k_cache, v_cache [num_blocks, Hkv, 16, D]; block_table [B, max_blocks];
    ctx_len [B]; vis [B, N, N]; pos [B, N].  Returns float64 [B, N, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    B, N, Hq, D = q.shape
    Hkv = k_node.shape[2]
    G = Hq // Hkv
    out = np.empty((B, N, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            Kc, Vc = context_kv(k_cache, v_cache, block_table[b], g, int(ctx_len[b]))
            out[b, :, g * G:(g + 1) * G] = tree_attn_group(
                q[b, :, g * G:(g + 1) * G], Kc, Vc,
                np.asarray(k_node[b, :, g], dtype=np.float64),
                np.asarray(v_node[b, :, g], dtype=np.float64),
                vis[b], pos[b], window, scale)
    return out
