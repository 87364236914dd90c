"""The allocation-free walk (tree_walk_accept_noalloc, static device scratch)
against tree_walk_accept with a caller workspace: accepted tokens, nodes and
counts bit for bit, on two calls in a row, the second with a smaller input
(so the scratch holds the first call's rows when the second runs), and
against the oracle walk."""
import numpy as np
import pytest
import torch

from helpers import np64, say
from oracle import walk as OW
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(config, B, N, V, dtype, tree):
    trees = W.make_trees(config, tree, B, N, V)
    x = W.walk_inputs(config, trees, V, dtype, device=DEV, plant=12.0)
    return trees, x.logits


def test_noalloc_walk_matches_workspace_walk(lib):
    cases = [(4, 64, 64, 262144, torch.bfloat16, "ddtree"),   # 4160 rows
             (1, 3, 17, 1000, torch.float32, "random_parent")]  # then 54 rows
    for config, B, N, V, dtype, tree in cases:
        say(f"noalloc walk B={B} N={N} V={V} dtype={dtype}")
        trees, logits = _case(config, B, N, V, dtype, tree)
        tok = torch.from_numpy(trees.tokens).to(DEV)
        par = torch.from_numpy(trees.parent).to(DEV)
        got = lib.tree_walk_accept_noalloc(tok, par, logits)
        ref = lib.tree_walk_accept(tok, par, logits)
        torch.cuda.synchronize()
        for k in ("accepted_tokens", "accepted_nodes", "num_accepted"):
            assert torch.equal(got[k], ref[k]), k
        want = OW.tree_walk(trees.tokens, trees.parent, np64(logits))
        assert np.array_equal(got["accepted_tokens"].cpu().numpy(), want["accepted_tokens"])
        assert np.array_equal(got["num_accepted"].cpu().numpy(), want["num_accepted"])
        say(f"   accepted {got['num_accepted'].cpu().tolist()[:8]}")


def test_noalloc_walk_rejects_oversized(lib):
    B, N = lib.WALK_NOALLOC_MAX_ROWS // 33 + 1, 32
    tok = torch.zeros(B, N, dtype=torch.int32, device=DEV)
    par = torch.full((B, N), -1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(B, N + 1, 1, dtype=torch.float32, device=DEV)
    with pytest.raises(lib.TVError) as e:
        lib.tree_walk_accept_noalloc(tok, par, logits)
    assert e.value.code == lib.TV_ERR_SCRATCH
