"""tree_gdn_verify on the GPU against the oracle recurrence, within the
stated tolerance (2e-2 of the output RMS for bf16 inputs, 1e-4 for fp32)."""
import numpy as np
import pytest
import torch

from helpers import np64, rel_err, say, tol_for
from oracle import gdn as OG
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run(lib, x, out_dtype=None):
    parent = torch.from_numpy(x.trees.parent).to(DEV)
    m = lib.tree_mask_build(parent, torch.full((x.B,), 100, dtype=torch.int32, device=DEV))
    S0_before = x.S0.clone()
    out = lib.tree_gdn_verify(x.q, x.k, x.v, x.alpha, x.beta, x.S0, m["anc"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(S0_before, x.S0)  # no state written
    return out


def run_checked(lib, x):
    """fp32 output for the tolerance check; for bf16 inputs also the bf16
    output, which must be exactly the round-to-nearest-even of the fp32 one."""
    out32 = run(lib, x, torch.float32)
    if x.q.dtype == torch.bfloat16:
        out16 = run(lib, x)
        assert out16.dtype == torch.bfloat16
        assert torch.equal(out16, out32.to(torch.bfloat16))
    return out32


def check(lib, x, tag):
    say(f"gdn {tag} B={x.B} N={x.N} H={x.H} dtype={x.q.dtype}")
    out = run_checked(lib, x)
    ref = OG.gdn_tree(np64(x.q), np64(x.k), np64(x.v), np64(x.alpha), np64(x.beta), np64(x.S0),
                      x.trees.parent)
    err = rel_err(np64(out), ref)
    say(f"   err={err:.3e}")
    assert err <= tol_for(x.q.dtype), err


def test_c5_full(lib):
    x = W.gdn_inputs(5, B=16, N=32, H=16, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16,
                     device=DEV)
    check(lib, x, "c5")


def test_step_batch_two_per_cu(lib):
    """The verify step's GDN shape: 32 sequences x 16 heads = 512 workgroups,
    more than the CUs, so two share a CU (the launch the benchmark times);
    the trees are the step's spine-first trees."""
    x = W.gdn_inputs(3, B=32, N=32, H=16, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16,
                     device=DEV)
    check(lib, x, "step batch")


@pytest.mark.parametrize("tree,N", [("spine_first", 48), ("random_parent", 64)])
def test_more_heads_than_cus_past_32_nodes(lib, tree, N):
    """32 sequences x 16 heads = 512 workgroups at 33-64 nodes: the
    block-triangular kernel then runs two workgroups per CU (its 128-register
    build), a launch the smaller test grids do not reach."""
    x = W.gdn_inputs(56, B=32, N=N, H=16, Dk=128, Dv=128, tree=tree, dtype=torch.bfloat16, device=DEV,
                     s0_std=0.5)
    check(lib, x, f"{tree} of {N}, 512 workgroups")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tree,N", [("chain", 64), ("star", 17), ("random_parent", 64),
                                    ("random_parent", 1), ("leaf_sibling", 32), ("spine_first", 40),
                                    ("random_parent", 65), ("spine_first", 100), ("chain", 128),
                                    ("random_parent", 128), ("spine_first", 128), ("star", 128)])
def test_trees(lib, dtype, tree, N):
    x = W.gdn_inputs(51, B=3, N=N, H=4, Dk=128, Dv=128, tree=tree, dtype=dtype, device=DEV)
    check(lib, x, tree)


@pytest.mark.parametrize("N", [2, 15, 16, 17, 31, 33, 48, 49, 63])
def test_chain_depths_per_node_tile(lib, N):
    """bf16 chains over the padded node counts of the dense kernel (16, 32)
    and of the block-triangular kernel from 33 nodes (64), across the switch
    between them, with depths just below, at and above a power of two: the
    dense kernel's gate products take ceil(log2 depth) doubling rounds and
    its solve as many steps.  The state is large enough that its low bf16
    part matters."""
    x = W.gdn_inputs(52, B=2, N=N, H=3, Dk=128, Dv=128, tree="chain", dtype=torch.bfloat16,
                     device=DEV, s0_std=0.5)
    check(lib, x, f"chain of {N}")


@pytest.mark.parametrize("tree", ["chain", "random_parent"])
@pytest.mark.parametrize("N", [96, 97])
def test_past_64_padding_boundary(lib, tree, N):
    """bf16 inputs on both sides of the past-64 kernel's padding step (96
    nodes in six 16-node tiles, 97 in eight): chains fill every diagonal
    block and reach the deepest block row of the back-substitution; random
    trees mix short and long paths.  The state is large enough that its low
    bf16 part matters."""
    x = W.gdn_inputs(55, B=2, N=N, H=3, Dk=128, Dv=128, tree=tree, dtype=torch.bfloat16, device=DEV,
                     s0_std=0.5)
    check(lib, x, f"{tree} of {N}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N", [64, 128])
def test_strong_state_and_gates(lib, dtype, N):
    """Larger committed state and gates spread over (0, 1] on deep random trees
    (gate products far below 1, so the gate ratios of distant ancestors matter)."""
    x = W.gdn_inputs(52, B=2, N=N, H=3, Dk=128, Dv=128, tree="random_parent", dtype=dtype,
                     device=DEV, s0_std=1.0)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    x.alpha.uniform_(0.05, 1.0, generator=gen)
    check(lib, x, "strong")


def test_deterministic(lib):
    x = W.gdn_inputs(53, B=4, N=32, H=4, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16,
                     device=DEV)
    a = run(lib, x)
    b = run(lib, x)
    assert torch.equal(a, b)


def _gate_nodes(parent_b):
    """A root (parent -1) with children, an interior node (parent >= 0, with
    children) and a leaf, the deepest of each kind."""
    N = len(parent_b)
    kids = np.zeros(N, dtype=int)
    for t in range(N):
        if parent_b[t] >= 0:
            kids[parent_b[t]] += 1
    depth = np.zeros(N, dtype=int)
    for t in range(N):
        depth[t] = 1 if parent_b[t] < 0 else depth[parent_b[t]] + 1
    roots = [t for t in range(N) if parent_b[t] < 0 and kids[t] > 0]
    inner = [t for t in range(N) if parent_b[t] >= 0 and kids[t] > 0]
    leaves = [t for t in range(N) if kids[t] == 0 and parent_b[t] >= 0]
    pick = lambda s: max(s, key=lambda t: (depth[t], t))
    return pick(roots), pick(inner), pick(leaves)


def _root_path(parent_b, t):
    path = []
    while t >= 0:
        path.append(t)
        t = int(parent_b[t])
    return path[::-1]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("where,N", [("root", 40), ("interior", 40), ("leaf", 40), ("all", 40),
                                     ("underflow", 40), ("all", 128), ("underflow", 128)])
def test_zero_and_underflowing_gates(lib, dtype, where, N):
    """Gates exactly 0 (a gate exp(g) that underflowed) at a root, an interior
    node and a leaf, and gates of 1e-30 along deep paths so that the gate
    products underflow fp32: every output stays finite and within tolerance
    of the recurrence, and the commit over a path through those nodes agrees
    with the oracle too (DFlash-TfM summary, section 3: the state follows the
    recurrence whatever the gate)."""
    x = W.gdn_inputs(54, B=3, N=N, H=4, Dk=128, Dv=128, tree="spine_first", dtype=dtype,
                     device=DEV, s0_std=0.5, max_depth=8 if N <= 64 else 24)
    alpha = x.alpha.cpu().numpy()
    acc = np.full((x.B, x.N), -1, dtype=np.int32)
    na = np.zeros(x.B, dtype=np.int32)
    for b in range(x.B):
        par = x.trees.parent[b]
        root, inner, leaf = _gate_nodes(par)
        if where == "underflow":
            # three tiny gates on the leaf's path (product 1e-90), heads 0 and 2
            for t in _root_path(par, leaf)[-3:]:
                alpha[b, t, 0::2] = 1e-30
            alpha[b, ::5, 1] = 1e-30
            target = leaf
        else:
            chosen = {"root": [root], "interior": [inner], "leaf": [leaf],
                      "all": [root, inner, leaf]}[where]
            for t in chosen:
                alpha[b, t, :] = 0.0
            # one head keeps one nonzero gate per chosen node: mixed heads
            alpha[b, chosen[0], 3] = 0.5
            # the commit follows the deepest path through the first chosen node
            through = [t for t in range(x.N) if chosen[0] in _root_path(par, t)]
            target = max(through, key=lambda t: (len(_root_path(par, t)), t))
        path = _root_path(par, target)
        acc[b, :len(path)] = path
        na[b] = len(path)
    x.alpha.copy_(torch.from_numpy(alpha).to(DEV))
    say(f"gdn gates {where} dtype={dtype}")
    out = run_checked(lib, x)
    assert torch.isfinite(out).all()
    ref = OG.gdn_tree(np64(x.q), np64(x.k), np64(x.v), np64(x.alpha), np64(x.beta), np64(x.S0),
                      x.trees.parent)
    err = rel_err(np64(out), ref)
    say(f"   verify err={err:.3e}")
    assert err <= tol_for(dtype), err
    S = lib.tree_gdn_commit(x.k, x.v, x.alpha, x.beta, x.S0, torch.from_numpy(acc).to(DEV),
                            torch.from_numpy(na).to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    refS = OG.gdn_commit(np64(x.k), np64(x.v), np64(x.alpha), np64(x.beta), np64(x.S0), acc, na)
    serr = rel_err(np64(S), refS)
    say(f"   commit err={serr:.3e}")
    assert serr <= 1e-4, serr
