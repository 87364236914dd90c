"""Pins for the Gated DeltaNet tree oracle.

The recurrence is the DFlash-TfM summary's ("3. Rollback-vrije
Boom-verificatie voor GDN").  Its oracle is checked against closed forms that
a dropped term, a wrong sign, a wrong decay index or a transposed state would
break, against the plain token-by-token chain recurrence on each root path,
and against the masked triangular-solve form of the same section.
"""
import numpy as np
import pytest
import torch

from oracle import gdn as G
from synth import workloads as W


def _inputs(B=2, N=10, H=3, Dk=8, Dv=6, tree="random_parent", config=31, trees=None):
    x = W.gdn_inputs(config, B=B, N=N, H=H, Dk=Dk, Dv=Dv, tree=tree, dtype=torch.float32,
                     trees=trees, s0_std=0.5)
    return [t.double().numpy() for t in (x.q, x.k, x.v, x.alpha, x.beta, x.S0)], x.trees.parent


def _paths(parent):
    out = []
    for t in range(len(parent)):
        p, cur = [], t
        while cur >= 0:
            p.append(cur)
            cur = int(parent[cur])
        out.append(p[::-1])
    return out


def test_beta_zero_is_pure_decay():
    """beta = 0 leaves only the gates: o_t = (prod of alpha on the root path)
    S0^T q_t."""
    (q, k, v, a, b, S0), par = _inputs()
    b[:] = 0.0
    o = G.gdn_tree(q, k, v, a, b, S0, par)
    for bb in range(q.shape[0]):
        for t, path in enumerate(_paths(par[bb])):
            for h in range(q.shape[2]):
                gamma = np.prod([a[bb, i, h] for i in path])
                np.testing.assert_allclose(o[bb, t, h], gamma * (S0[bb, h].T @ q[bb, t, h]),
                                           rtol=1e-13, atol=1e-14)


def test_state_orientation():
    """With S0 = e_i e_j^T (one entry), beta = 0, alpha = 1 and q = e_i the
    output is e_j: the state is read as S^T q, keys index its rows."""
    (q, k, v, a, b, S0), par = _inputs(B=1, N=3, H=1, Dk=5, Dv=4)
    b[:] = 0.0
    a[:] = 1.0
    S0[:] = 0.0
    S0[0, 0, 2, 1] = 1.0
    q[:] = 0.0
    q[0, :, 0, 2] = 1.0
    o = G.gdn_tree(q, k, v, a, b, S0, par)
    np.testing.assert_array_equal(o[0, :, 0], np.tile(np.eye(4)[1], (3, 1)))


def test_unit_key_recall_is_exact():
    """beta = 1 and |k| = 1 make the delta rule overwrite the value stored
    under k: with q_t = k_t the output is v_t whatever alpha and S0 are."""
    (q, k, v, a, b, S0), par = _inputs(N=12)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q[:] = k
    b[:] = 1.0
    o = G.gdn_tree(q, k, v, a, b, S0, par)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_single_node_from_zero_state():
    """S0 = 0, one node: o = beta (k . q) v."""
    (q, k, v, a, b, S0), _ = _inputs(B=1, N=1, H=2)
    S0[:] = 0.0
    o = G.gdn_tree(q, k, v, a, b, S0, np.array([[-1]]))
    for h in range(2):
        np.testing.assert_allclose(o[0, 0, h], b[0, 0, h] * (k[0, 0, h] @ q[0, 0, h]) * v[0, 0, h],
                                   rtol=1e-13)


def test_orthonormal_chain_recall():
    """alpha = beta = 1, orthonormal keys along a chain from S0 = 0: the state
    after the chain maps every key to its own value, so querying node t's
    state with an earlier key k_i returns v_i."""
    N, Dk, Dv = 5, 8, 3
    rng = np.random.default_rng(4)
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:N][None, :, None, :]
    v = rng.standard_normal((1, N, 1, Dv))
    a = np.ones((1, N, 1))
    b = np.ones((1, N, 1))
    S0 = np.zeros((1, 1, Dk, Dv))
    par = np.arange(-1, N - 1)[None]
    for i in range(N):
        q = np.zeros((1, N, 1, Dk))
        q[0, N - 1, 0] = k[0, i, 0]
        o = G.gdn_tree(q, k, v, a, b, S0, par)
        np.testing.assert_allclose(o[0, N - 1, 0], v[0, i, 0], atol=1e-12)


def _chain_recurrence(qs, ks, vs, als, bes, S0):
    """Token-by-token recurrence with the explicit matrix I - beta k k^T."""
    S = S0.copy()
    outs = []
    I = np.eye(S0.shape[0])
    for qt, kt, vt, at, bt in zip(qs, ks, vs, als, bes):
        S = at * (I - bt * np.outer(kt, kt)) @ S + bt * np.outer(kt, vt)
        outs.append(S.T @ qt)
    return outs


@pytest.mark.parametrize("tree", ["random_parent", "spine_first", "chain", "star"])
def test_every_node_is_its_root_path_chain(tree):
    """Each node's output equals the chain recurrence run alone over its root
    path: siblings and cousins never leak into it (no speculative state)."""
    (q, k, v, a, b, S0), par = _inputs(N=14, tree=tree, config=33)
    o = G.gdn_tree(q, k, v, a, b, S0, par)
    for bb in range(q.shape[0]):
        for t, path in enumerate(_paths(par[bb])):
            for h in range(q.shape[2]):
                ref = _chain_recurrence(q[bb, path, h], k[bb, path, h], v[bb, path, h],
                                        a[bb, path, h], b[bb, path, h], S0[bb, h])[-1]
                np.testing.assert_allclose(o[bb, t, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("tree,n", [("random_parent", 16), ("spine_first", 32), ("chain", 9),
                                    ("star", 6), ("leaf_sibling", 32)])
def test_triangular_solve_form_matches_recurrence(tree, n):
    """The masked (I + X) U = beta V solve with its committed-state companion
    reproduces the recurrence to rounding."""
    (q, k, v, a, b, S0), par = _inputs(N=n, tree=tree, config=34, Dk=16, Dv=12)
    o1 = G.gdn_tree(q, k, v, a, b, S0, par)
    o2 = G.gdn_tree_solve(q, k, v, a, b, S0, par)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-11)


# ---- deferred state commit (the chain over the accepted nodes) ----

def _root_path(parent_b, t):
    p, cur = [], t
    while cur >= 0:
        p.append(cur)
        cur = int(parent_b[cur])
    return p[::-1]


def test_commit_without_accept_keeps_s0():
    (q, k, v, a, b, S0), par = _inputs()
    acc = np.full(par.shape, -1)
    S = G.gdn_commit(k, v, a, b, S0, acc, np.zeros(par.shape[0], dtype=int))
    np.testing.assert_array_equal(S, S0)


@pytest.mark.parametrize("tree", ["random_parent", "chain"])
def test_commit_equals_tree_state_of_last_accepted(tree):
    """Committing the root path of node t reproduces the state the tree
    recurrence holds at t: its output for any query equals S^T q (checked
    through both tree oracles, the plain recurrence and the solve form)."""
    (q, k, v, a, b, S0), par = _inputs(N=12, tree=tree)
    B, N, H = q.shape[:3]
    rng = np.random.default_rng(3)
    acc = np.full((B, N), -1)
    na = np.zeros(B, dtype=int)
    last = []
    for bb in range(B):
        t = int(rng.integers(0, N))
        path = _root_path(par[bb], t)
        acc[bb, :len(path)] = path
        na[bb] = len(path)
        last.append(t)
    S = G.gdn_commit(k, v, a, b, S0, acc, na)
    o_plain = G.gdn_tree(q, k, v, a, b, S0, par)
    o_solve = G.gdn_tree_solve(q, k, v, a, b, S0, par)
    for bb in range(B):
        t = last[bb]
        for h in range(H):
            np.testing.assert_allclose(S[bb, h].T @ q[bb, t, h], o_plain[bb, t, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S[bb, h].T @ q[bb, t, h], o_solve[bb, t, h], rtol=1e-9, atol=1e-10)


def test_commit_beta_zero_is_pure_decay():
    (q, k, v, a, b, S0), par = _inputs(N=9, tree="chain")
    b[:] = 0.0
    B = q.shape[0]
    acc = np.tile(np.arange(9), (B, 1))
    na = np.array([9, 4][:B])
    S = G.gdn_commit(k, v, a, b, S0, acc, na)
    for bb in range(B):
        for h in range(q.shape[2]):
            gamma = np.prod(a[bb, :na[bb], h])
            np.testing.assert_allclose(S[bb, h], gamma * S0[bb, h], rtol=1e-13, atol=1e-15)


def test_commit_orthonormal_keys_recall_every_value():
    """alpha = 1, beta = 1 and orthonormal keys along the accepted chain: each
    write replaces the value stored under its key and leaves the others, so
    S^T k_i = v_i for every accepted node i."""
    (q, k, v, a, b, S0), par = _inputs(B=1, N=5, H=2, Dk=8, Dv=6, tree="chain")
    rng = np.random.default_rng(11)
    for h in range(2):
        Qm, _ = np.linalg.qr(rng.standard_normal((8, 5)))
        k[0, :, h] = Qm.T
    a[:] = 1.0
    b[:] = 1.0
    S = G.gdn_commit(k, v, a, b, S0, np.arange(5)[None], np.array([5]))
    for h in range(2):
        for i in range(5):
            np.testing.assert_allclose(S[0, h].T @ k[0, i, h], v[0, i, h], rtol=1e-12, atol=1e-12)
