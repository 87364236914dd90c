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
    """Gather the ctx context keys/values of one sequence and kv head by
    following the block table page by page."""
    D = k_cache.shape[-1]
    K = np.empty((ctx, D), dtype=np.float64)
    V = np.empty((ctx, D), dtype=np.float64)
    for j in range(ctx):
        page = int(block_table_b[j // BLOCK])
        K[j] = k_cache[page, g, j % BLOCK]
        V[j] = v_cache[page, g, j % BLOCK]
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


def attend(qvec, K, V, visible, scale):
    """softmax(scale * K q) over the visible keys, then the weighted sum of V."""
    s = scale * (K[visible] @ qvec)
    s = s - s.max()
    w = np.exp(s)
    w = w / w.sum()
    return w @ V[visible]


def tree_attn_group(q_g, Kc, Vc, Kn, Vn, vis, pos, window, scale, nodes=None):
    """One (sequence, kv head): q_g [N, G, D] (the G query heads of the
    group), Kc/Vc [ctx, D] context, Kn/Vn [N, D] node keys/values, vis [N, N],
    pos [N].  Returns [N, G, D]; rows not in ``nodes`` are left as NaN."""
    N, G, D = q_g.shape
    ctx = Kc.shape[0]
    out = np.full((N, G, D), np.nan)
    K = np.concatenate([Kc, Kn], axis=0)
    V = np.concatenate([Vc, Vn], axis=0)
    for t in (range(N) if nodes is None else nodes):
        cv, nv = visible_keys(int(pos[t]), ctx, vis[t], pos, window)
        visible = np.concatenate([cv, nv])
        for hl in range(G):
            out[t, hl] = attend(q_g[t, hl], K, V, visible, scale)
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
