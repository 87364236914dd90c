"""Oracle: Gated DeltaNet over a draft tree, with no state written back.

Follows the DFlash-TfM summary (page "gist.science/nl/paper/2607.06763"),
section "3. Rollback-vrije Boom-verificatie voor GDN".  The recurrence it
states is, for a node t with parent p(t),

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{p(t)} + beta_t k_t v_t^T,

with S_{p(t)} = S_0 (the committed state) when t hangs under the last
accepted token.  Each node's output is o_t = S_t^T q_t.  The states are kept
only inside this function: nothing is returned but the outputs, which is the
"no speculative state update" contract of the same section.

Readings: S has shape [Dk, Dv]; alpha and beta are one scalar per
(sequence, node, head); there is no output scaling or normalisation.

``gdn_tree`` is the plain definition (the recurrence along every root path,
memoised per node because nodes come in topological order).
``gdn_tree_solve`` follows the section's method in its order: the tree is
already topologically sorted; build the ancestor interaction matrices X and Y;
solve the unit lower-triangular system (I + X) U = beta V, together with its
companion system for the committed-state term; form the outputs.  It is
checked against ``gdn_tree`` by the tests.
"""
from __future__ import annotations

import numpy as np


def gdn_tree(q, k, v, alpha, beta, S0, parent):
    """q, k [B, N, H, Dk]; v [B, N, H, Dv]; alpha, beta [B, N, H];
    S0 [B, H, Dk, Dv]; parent [B, N] with parent[t] < t.
    Returns o [B, N, H, Dv] float64."""
    q, k, v, alpha, beta, S0 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, S0))
    parent = np.asarray(parent)
    B, N, H, Dk = q.shape
    Dv = v.shape[-1]
    out = np.empty((B, N, H, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            states = []
            for t in range(N):
                p = int(parent[b, t])
                assert -1 <= p < t, "nodes must be topologically ordered"
                Sp = S0[b, h] if p < 0 else states[p]
                kt, vt = k[b, t, h], v[b, t, h]
                a, be = alpha[b, t, h], beta[b, t, h]
                St = a * (Sp - be * np.outer(kt, kt @ Sp)) + be * np.outer(kt, vt)
                states.append(St)
                out[b, t, h] = St.T @ q[b, t, h]
    return out


def _path(parent_b, t):
    P = []
    cur = t
    while cur != -1:
        P.append(cur)
        cur = int(parent_b[cur])
    return P  # t first, root-side last


def gdn_tree_solve(q, k, v, alpha, beta, S0, parent):
    """Same outputs as gdn_tree, by the masked triangular solve:

      gamma_t = product of alpha over the root path of t (t included);
      X[t, i] = beta_t (gamma_t / gamma_i) k_t . k_i   for i a strict ancestor
      Y[t, i] = (gamma_t / gamma_i) q_t . k_i          for i ancestor-or-self
      (I + X) Ut = beta V,   (I + X) W = beta gamma K,   U = Ut - W S0
      O = gamma (Q S0) + Y U
    """
    q, k, v, alpha, beta, S0 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, S0))
    parent = np.asarray(parent)
    B, N, H, Dk = q.shape
    Dv = v.shape[-1]
    out = np.empty((B, N, H, Dv), dtype=np.float64)
    for b in range(B):
        paths = [_path(parent[b], t) for t in range(N)]
        for h in range(H):
            a = alpha[b, :, h]
            be = beta[b, :, h]
            # decay ratio gamma_t / gamma_i: product of alpha over the path
            # segment strictly below i down to t
            ratio = np.zeros((N, N))
            gamma = np.empty(N)
            for t in range(N):
                P = paths[t]
                gamma[t] = np.prod(a[P])
                prod = 1.0
                for i in P:  # walk from t towards the root
                    ratio[t, i] = prod
                    prod *= a[i]
            Kh, Qh, Vh = k[b, :, h], q[b, :, h], v[b, :, h]
            strict = np.zeros((N, N), dtype=bool)
            incl = np.zeros((N, N), dtype=bool)
            for t in range(N):
                for i in paths[t]:
                    incl[t, i] = True
                    if i != t:
                        strict[t, i] = True
            X = np.where(strict, be[:, None] * ratio * (Kh @ Kh.T), 0.0)
            Y = np.where(incl, ratio * (Qh @ Kh.T), 0.0)
            A = np.eye(N) + X
            Ut = np.linalg.solve(A, be[:, None] * Vh)
            W = np.linalg.solve(A, (be * gamma)[:, None] * Kh)
            U = Ut - W @ S0[b, h]
            out[b, :, h] = gamma[:, None] * (Qh @ S0[b, h]) + Y @ U
    return out


def gdn_commit(k, v, alpha, beta, S0, accepted_nodes, num_accepted):
    """The committed state after the walk: the same recurrence, run as a chain
    over the accepted nodes in order (each the child of the one before, the
    first a child of the last accepted token), starting from S0.  With no
    accepted node the state stays S0.  This is the deferred commit of the
    same section: the state is published only once the accepted branch is
    known.

    k [B, N, H, Dk]; v [B, N, H, Dv]; alpha, beta [B, N, H]; S0 [B, H, Dk, Dv];
    accepted_nodes [B, N] (first num_accepted[b] entries valid);
    num_accepted [B].  Returns S [B, H, Dk, Dv] float64."""
    k, v, alpha, beta, S0 = (np.asarray(x, dtype=np.float64) for x in (k, v, alpha, beta, S0))
    acc = np.asarray(accepted_nodes)
    na = np.asarray(num_accepted)
    B, N, H, Dk = k.shape
    S = S0.copy()
    for b in range(B):
        for h in range(H):
            St = S0[b, h].copy()
            for s in range(int(na[b])):
                t = int(acc[b, s])
                kt, vt = k[b, t, h], v[b, t, h]
                a, be = alpha[b, t, h], beta[b, t, h]
                St = a * (St - be * np.outer(kt, kt @ St)) + be * np.outer(kt, vt)
            S[b, h] = St
    return S
