"""Pins for the attention oracle (tree-masked attention over a paged context)."""
import numpy as np
import pytest
import torch

from oracle import attn as A
from oracle import mask as M
from synth import workloads as W


def _np(x):
    return x.double().numpy()


def _case(tree="random_parent", B=2, N=12, Hq=4, Hkv=2, D=32, ctx=(37, 70), window=0,
          config=11, trees=None, ctx_len=None):
    return W.attn_inputs(config, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, ctx_lo=ctx[0], ctx_hi=ctx[1],
                         tree=tree, dtype=torch.float32, window=window, trees=trees,
                         ctx_len=ctx_len)


def _run_oracle(x, window=None):
    m = M.tree_mask(x.trees.parent, x.ctx_len.numpy())
    out = A.tree_attn(_np(x.q), _np(x.k_node), _np(x.v_node), _np(x.k_cache), _np(x.v_cache),
                      x.block_table.numpy(), x.ctx_len.numpy(), m["vis"], m["pos"],
                      x.window if window is None else window, x.scale)
    return out, m


def _contiguous_ctx(x, b, g):
    """Context K/V of (b, g) laid out contiguously, by flat indexing of the
    page pool (independent of the oracle's gather loop)."""
    ctx = int(x.ctx_len[b])
    pages = x.block_table[b, :(ctx + 15) // 16].long()
    K = x.k_cache[pages, g].reshape(-1, x.D)[:ctx].double()
    V = x.v_cache[pages, g].reshape(-1, x.D)[:ctx].double()
    return K, V


def _sdpa(qrows, K, V, allowed, scale):
    """torch's scaled_dot_product_attention in float64 with a boolean mask."""
    return torch.nn.functional.scaled_dot_product_attention(
        qrows[None, None], K[None, None], V[None, None], attn_mask=allowed[None, None],
        scale=scale)[0, 0]


@pytest.mark.parametrize("N", [9, 128])
def test_chain_equals_causal_attention(N):
    """A chain tree is plain causal attention over context ++ chain (the chain
    verify the serve spec starts from); at 128 nodes the ancestor sets span
    two words."""
    x = _case(tree="chain", N=N, ctx=(45, 45))
    out, _ = _run_oracle(x)
    G = x.Hq // x.Hkv
    for b in range(x.B):
        ctx = int(x.ctx_len[b])
        for h in range(x.Hq):
            g = h // G
            Kc, Vc = _contiguous_ctx(x, b, g)
            K = torch.cat([Kc, x.k_node[b, :, g].double()])
            V = torch.cat([Vc, x.v_node[b, :, g].double()])
            L = ctx + N
            # query i sits at sequence position ctx + i: causal = keys 0..ctx+i
            allowed = torch.ones(N, L, dtype=torch.bool).tril(diagonal=ctx)
            ref = _sdpa(x.q[b, :, h].double(), K, V, allowed, x.scale)
            np.testing.assert_allclose(out[b, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_empty_and_ragged_contexts_equal_causal_attention():
    """Contexts of 0, 1, 15, 16 and 17 tokens (no page, a partial page, page
    boundaries) with a chain of nodes: still plain causal attention over
    context ++ chain; with no context, over the chain alone."""
    trees = W.make_trees(12, "chain", 5, 6, 100)
    x = _case(tree="chain", B=5, N=6, trees=trees, ctx_len=np.array([0, 1, 15, 16, 17], dtype=np.int32))
    out, _ = _run_oracle(x)
    G = x.Hq // x.Hkv
    for b in range(x.B):
        ctx = int(x.ctx_len[b])
        for h in range(x.Hq):
            g = h // G
            Kc, Vc = _contiguous_ctx(x, b, g)
            K = torch.cat([Kc, x.k_node[b, :, g].double()])
            V = torch.cat([Vc, x.v_node[b, :, g].double()])
            allowed = torch.ones(x.N, ctx + x.N, dtype=torch.bool).tril(diagonal=ctx)
            ref = _sdpa(x.q[b, :, h].double(), K, V, allowed, x.scale)
            np.testing.assert_allclose(out[b, :, h], ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("tree", ["random_parent", "spine_first", "leaf_sibling"])
def test_each_node_is_attention_over_its_root_path(tree):
    """Every node's output equals ordinary attention of its query over the
    contiguous sequence context ++ (its root path), i.e. a union of chains."""
    N = 16
    x = _case(tree=tree, N=N, ctx=(20, 53), config=12)
    out, _ = _run_oracle(x)
    G = x.Hq // x.Hkv
    for b in range(x.B):
        par = x.trees.parent[b]
        for t in range(N):
            path = []
            cur = t
            while cur >= 0:
                path.append(cur)
                cur = int(par[cur])
            path = path[::-1]
            for h in range(x.Hq):
                g = h // G
                Kc, Vc = _contiguous_ctx(x, b, g)
                K = torch.cat([Kc, x.k_node[b, path, g].double()])
                V = torch.cat([Vc, x.v_node[b, path, g].double()])
                ref = _sdpa(x.q[b, t, h].double()[None], K, V,
                            torch.ones(1, K.shape[0], dtype=torch.bool), x.scale)[0]
                np.testing.assert_allclose(out[b, t, h], ref.numpy(), rtol=0, atol=1e-12)


def test_star_is_decode_attention():
    x = _case(tree="star", N=6, ctx=(30, 31))
    out, _ = _run_oracle(x)
    G = x.Hq // x.Hkv
    for b in range(x.B):
        for t in range(6):
            for h in range(x.Hq):
                g = h // G
                Kc, Vc = _contiguous_ctx(x, b, g)
                K = torch.cat([Kc, x.k_node[b, t:t + 1, g].double()])
                V = torch.cat([Vc, x.v_node[b, t:t + 1, g].double()])
                s = x.scale * (K @ x.q[b, t, h].double())
                ref = torch.softmax(s, 0) @ V
                np.testing.assert_allclose(out[b, t, h], ref.numpy(), rtol=0, atol=1e-12)


def test_window_one_returns_own_value():
    """W = 1: a query sees only its own key, so the output is exactly v_self."""
    x = _case(window=1)
    out, _ = _run_oracle(x)
    G = x.Hq // x.Hkv
    for h in range(x.Hq):
        np.testing.assert_array_equal(out[:, :, h], _np(x.v_node[:, :, h // G]))


@pytest.mark.parametrize("window", [0, 1, 2, 3, 5, 17, 40])
def test_zero_query_is_mean_of_visible_values(window):
    """q = 0 makes every visible key weigh the same, so each output is the
    mean of the visible values.  The visible set is written here in closed
    form: context positions max(0, ctx + depth - W) .. ctx-1 (all of them when
    W <= 0) and the ancestors s with depth(t) - depth(s) < W."""
    x = _case(window=window, N=14, ctx=(8, 25), config=13)
    x.q.zero_()
    out, m = _run_oracle(x)
    G = x.Hq // x.Hkv
    for b in range(x.B):
        ctx = int(x.ctx_len[b])
        par = x.trees.parent[b]
        for t in range(14):
            depth = 0
            anc = []
            cur = t
            while cur >= 0:
                anc.append(cur)
                cur = int(par[cur])
            depth = len(anc)
            lo = 0 if window <= 0 else max(0, ctx + depth - window)
            node_depth = {s: len(anc) - i for i, s in enumerate(anc)}
            keep = [s for s in anc if window <= 0 or depth - node_depth[s] < window]
            for h in range(x.Hq):
                g = h // G
                _, Vc = _contiguous_ctx(x, b, g)
                rows = torch.cat([Vc[lo:ctx], x.v_node[b, keep, g].double()])
                np.testing.assert_allclose(out[b, t, h], rows.mean(0).numpy(), rtol=0, atol=1e-12)


def test_large_window_is_global():
    x = _case(ctx=(30, 60), N=10)
    g_out, _ = _run_oracle(x, window=0)
    w_out, _ = _run_oracle(x, window=60 + 11)
    np.testing.assert_array_equal(g_out, w_out)


def test_kv_head_mapping():
    """Query head h reads kv head h // (Hq / Hkv): give kv head g constant
    values g + 1; every output of head h is then exactly h // G + 1."""
    x = _case(Hq=6, Hkv=3)
    for g in range(3):
        x.v_cache[:, g] = g + 1.0
        x.v_node[:, :, g] = g + 1.0
    out, _ = _run_oracle(x)
    for h in range(6):
        np.testing.assert_allclose(out[:, :, h], h // 2 + 1.0, rtol=0, atol=1e-13)


def test_page_permutation_invariance():
    """Relabelling the physical pages (and the table with them) changes nothing."""
    x = _case(ctx=(40, 77))
    out, _ = _run_oracle(x)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(x.num_blocks))
    inv = torch.argsort(perm)
    x.k_cache = x.k_cache[perm]
    x.v_cache = x.v_cache[perm]
    bt = x.block_table.clone()
    valid = bt >= 0
    bt[valid] = inv[bt[valid].long()].int()
    x.block_table = bt
    out2, _ = _run_oracle(x)
    np.testing.assert_array_equal(out, out2)


def test_node_relabelling_equivariance():
    """Reversing the order of two independent subtrees' nodes (keeping the
    topological order) permutes the outputs the same way."""
    par = np.array([[-1, -1, 0, 1, 2, 3]])
    x = _case(tree="star", B=1, N=6, trees=W.TreeBatch(par.astype(np.int32),
                                                      np.zeros((1, 6), np.int32), None))
    out, _ = _run_oracle(x)
    # swap the roles of the two chains 0-2-4 and 1-3-5
    sigma = [1, 0, 3, 2, 5, 4]
    x2 = _case(tree="star", B=1, N=6, trees=W.TreeBatch(par.astype(np.int32),
                                                       np.zeros((1, 6), np.int32), None))
    x2.q = x.q[:, sigma].clone()
    x2.k_node = x.k_node[:, sigma].clone()
    x2.v_node = x.v_node[:, sigma].clone()
    x2.ctx_len, x2.block_table, x2.k_cache, x2.v_cache = x.ctx_len, x.block_table, x.k_cache, x.v_cache
    out2, _ = _run_oracle(x2)
    np.testing.assert_allclose(out2, out[:, sigma], rtol=0, atol=1e-13)
