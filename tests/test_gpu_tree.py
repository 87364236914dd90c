"""Draft-tree construction on the GPU against the oracle: candidate tokens
bit-exact, log-probabilities equal to the oracle's float64 log-softmax
rounded to float32 (the library rounds its float64 log-sum-exp once), tree
structure and float32 scores bit-exact on given candidates (both sides add in
float32, one rounding per node) and end to end from the draft logits."""
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
    g = got["cand_logprob"].cpu().numpy()
    want = lp.astype(np.float32)
    bad = np.flatnonzero(g.ravel() != want.ravel())
    assert bad.size == 0, (bad[:8], g.ravel()[bad[:8]], lp.ravel()[bad[:8]])
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


@pytest.mark.parametrize("dtype,V,sigma,K", [
    (torch.bfloat16, 3 * 16384 + 8 * 300, 1.0, 16),  # three whole passes, a ragged one, every element queued
    (torch.bfloat16, 3 * 16384 + 8 * 300, 8.0, 8),
    (torch.float32, 3 * 8192 + 4 * 77, 1.0, 5),
    (torch.bfloat16, 3 * 16384 + 8 * 300 + 3, 1.0, 3),  # rows not 16-byte multiples: element by element
])
def test_topk_passes_and_queue_load(lib, dtype, V, sigma, K):
    """Rows of several passes of 4 chunks a thread, a partial pass and a tail;
    sigma 1 puts every element within the fp64 band, so each pass fills the
    wave's queue to its bound."""
    say(f"topk passes V={V} sigma={sigma} K={K} {dtype}")
    _check_topk(lib, W.draft_logits(74, 2, 2, V, dtype, sigma=sigma, device=DEV), K)


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
    of 262144-entry bf16 draft logits, top 8, budget 64, one candidate per
    round and 8 per round.  bf16 logits lie on a coarse grid, so different
    paths often tie on their float32 cumulative values; with candidates and
    log-probabilities bit-exact, every tie is decided the same way on both
    sides and the trees must be identical node for node."""
    B, L, V, K, N = 64, 8, 262144, 8, 64
    x = W.draft_logits(4, B, L, V, torch.bfloat16, device=DEV, on_device=True)
    say("tree construction, DDTree batch")
    cand = lib.tree_draft_topk(x, K)
    torch.cuda.synchronize()
    tok, lp = OT.draft_topk(x.double().cpu().numpy(), K)
    assert np.array_equal(cand["cand_tokens"].cpu().numpy(), tok)
    assert np.array_equal(cand["cand_logprob"].cpu().numpy(), lp.astype(np.float32))
    for w in (1, 8):
        tree = lib.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, w)
        torch.cuda.synchronize()
        ref = OT.tree_build(tok, lp.astype(np.float32), N, w)
        g = {k: tree[k].cpu().numpy() for k in ("tokens", "parent", "depth", "num_nodes", "score")}
        for k in ("tokens", "parent", "depth", "num_nodes"):
            assert np.array_equal(g[k], ref[k]), (w, k)
        assert np.array_equal(g["score"], ref["score"]), w
    m = OM.tree_mask(g["parent"], np.full(B, 100), g["depth"])
    assert np.all(m["status"] == 0)
