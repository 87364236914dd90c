"""Oracle: commit of the accepted path's keys and values to the paged cache.

After the walk the accepted nodes become context: accepted node s (depth
s + 1, the child of accepted node s - 1) takes position ctx_len + s, one past
the last accepted token at ctx_len - 1 (serve-integration spec, layout
contract and "3. Rejection sampler: tree walk": the node's position id is
ctx_len - 1 + depth).  Its key and value rows, computed by the verify pass,
are copied into the page the block table gives for that position.

Readings: position j of sequence b lives in page block_table[b][j // 16],
slot j % 16, of the [num_blocks, Hkv, 16, D] caches (as in the attention
oracle); the caller has allocated the pages; a position whose page index is
outside the table or the pool, or a node index outside [0, N), is not
written.

Test infrastructure: only tests, smoke() and the benchmark's CPU baseline use
this module.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def kv_commit(k_cache, v_cache, k_node, v_node, accepted_nodes, num_accepted, ctx_len,
              block_table):
    """Returns updated copies of k_cache, v_cache [num_blocks, Hkv, 16, D]
    (same dtype); k_node, v_node [B, N, Hkv, D]; accepted_nodes [B, N];
    num_accepted, ctx_len [B]; block_table [B, max_blocks]."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B = len(num_accepted)
    for b in range(B):
        for s in range(int(num_accepted[b])):
            t = int(accepted_nodes[b, s])
            p = int(ctx_len[b]) + s
            if not 0 <= t < k_node.shape[1] or p < 0 or p // BLOCK >= block_table.shape[1]:
                continue
            page = int(block_table[b, p // BLOCK])
            if not 0 <= page < kc.shape[0]:
                continue
            kc[page, :, p % BLOCK] = k_node[b, t]
            vc[page, :, p % BLOCK] = v_node[b, t]
    return kc, vc
