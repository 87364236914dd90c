"""Draft-tree construction on the GPU against the oracle: candidate tokens
bit-exact and log-probabilities within 1e-5 + 1e-6 |lp| (fp32 log-sum-exp
over up to 262144 entries), tree structure and float32 scores bit-exact on
given candidates (both sides add in float32, one rounding per node)."""
import numpy as np
import pytest
import torch

from helpers import say
from oracle import mask as OM
from oracle import treebuild as OT
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check_topk(lib, x, K):
    got = lib.tree_draft_topk(x, K)
    torch.cuda.synchronize()
    tok, lp = OT.draft_topk(x.double().cpu().numpy(), K)
    assert np.array_equal(got["cand_tokens"].cpu().numpy(), tok)
    g = got["cand_logprob"].cpu().numpy().astype(np.float64)
    err = np.abs(g - lp) - (1e-5 + 1e-6 * np.abs(lp))
    assert err.max() <= 0, float(err.max())
    return got


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,L,V,K", [(3, 4, 1000, 8), (2, 2, 1001, 16), (1, 3, 7, 7), (2, 16, 4096, 1)])
def test_topk(lib, dtype, B, L, V, K):
    say(f"topk B={B} L={L} V={V} K={K} {dtype}")
    _check_topk(lib, W.draft_logits(70, B, L, V, dtype, device=DEV), K)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_topk_ties(lib, dtype):
    """Coarse logits (multiples of 1/2 in [-3, 3]): many equal values, which
    go to the lower token id."""
    x = (torch.round(W.draft_logits(71, 2, 3, 2000, torch.float32, sigma=1.5) * 2) / 2).clamp(-3, 3)
    say(f"topk ties {dtype}")
    _check_topk(lib, x.to(dtype).to(DEV), 16)


def test_topk_full_vocabulary(lib):
    """Rows of the DDTree workload's vocabulary (262144), bf16, sigma 8."""
    x = W.draft_logits(72, 2, 8, 262144, torch.bfloat16, device=DEV, on_device=True)
    say("topk V=262144")
    _check_topk(lib, x, 8)


def _check_build(lib, tok, lp, N, w):
    got = lib.tree_build(torch.from_numpy(tok).to(DEV), torch.from_numpy(lp).to(DEV), N, w)
    torch.cuda.synchronize()
    ref = OT.tree_build(tok, lp, N, w)
    for k in ("tokens", "parent", "depth", "num_nodes"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k
    assert np.array_equal(got["score"].cpu().numpy(), ref["score"])
    return got


@pytest.mark.parametrize("L,K,N,w", [(8, 8, 64, 1), (8, 8, 128, 1), (4, 3, 128, 1), (2, 2, 10, 1),
                                     (8, 8, 64, 4), (6, 5, 100, 7), (16, 16, 128, 16), (1, 16, 16, 3),
                                     (8, 8, 1, 1), (3, 16, 128, 128)])
@pytest.mark.parametrize("ties", [False, True])
def test_build(lib, L, K, N, w, ties):
    tok, lp = W.draft_candidates(73 + L, 5, L, K, ties=ties)
    say(f"build L={L} K={K} N={N} w={w} ties={ties}")
    _check_build(lib, tok, lp, N, w)


def test_end_to_end_ddtree_batch(lib):
    """The DDTree workload's construction at full size: 64 sequences, 8 depths
    of 262144-entry bf16 draft logits, top 8, budget 64.  Candidates are
    compared exactly (tokens) and within tolerance (log-probabilities).  bf16
    logits lie on a coarse grid, so different paths can have equal cumulative
    values; which of them fills the last places is decided by the last bit of
    each side's own float32 log-probabilities.  What is unique is compared:
    the sorted cumulative values of the tree (recomputed along each GPU path
    from the oracle's float64 log-probabilities) against the oracle tree's,
    within 1e-4; and the GPU tree is checked to be valid: parents first,
    depths consistent, every node the candidate of its depth, better
    siblings and parents in the tree."""
    B, L, V, K, N = 64, 8, 262144, 8, 64
    x = W.draft_logits(4, B, L, V, torch.bfloat16, device=DEV, on_device=True)
    say("tree construction, DDTree batch")
    cand = lib.tree_draft_topk(x, K)
    tree = lib.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 1)
    torch.cuda.synchronize()
    tok, lp = OT.draft_topk(x.double().cpu().numpy(), K)
    assert np.array_equal(cand["cand_tokens"].cpu().numpy(), tok)
    ref = OT.tree_build(tok, lp.astype(np.float32), N, 1)
    g = {k: tree[k].cpu().numpy() for k in ("tokens", "parent", "depth", "num_nodes")}
    assert np.array_equal(g["num_nodes"], ref["num_nodes"])
    same = 0
    for b in range(B):
        rank_of = [{int(t): r for r, t in enumerate(tok[b, d])} for d in range(L)]

        def path_value(par, dep, toks, t):
            v, ranks = 0.0, []
            while t >= 0:
                r = rank_of[dep[t] - 1][int(toks[t])]
                v += lp[b, dep[t] - 1, r]
                ranks.append(r)
                t = par[t]
            return v, tuple(ranks[::-1])

        par, dep, toks = g["parent"][b], g["depth"][b], g["tokens"][b]
        vals, paths = [], set()
        for t in range(N):
            assert par[t] < t and dep[t] == (1 if par[t] < 0 else dep[par[t]] + 1)
            assert int(toks[t]) in rank_of[dep[t] - 1]
            v, pth = path_value(par, dep, toks, t)
            vals.append(v)
            paths.add(pth)
        for pth in paths:  # closed under parents and better siblings
            assert pth[:-1] in paths or len(pth) == 1
            assert pth[-1] == 0 or pth[:-1] + (pth[-1] - 1,) in paths
        rvals = [path_value(ref["parent"][b], ref["depth"][b], ref["tokens"][b], t)[0] for t in range(N)]
        assert np.abs(np.sort(vals) - np.sort(rvals)).max() <= 1e-4
        same += int(np.array_equal(toks, ref["tokens"][b]) and np.array_equal(par, ref["parent"][b]))
    say(f"   trees identical to the oracle's in {same} of {B} sequences")
    m = OM.tree_mask(g["parent"], np.full(B, 100), g["depth"])
    assert np.all(m["status"] == 0)
