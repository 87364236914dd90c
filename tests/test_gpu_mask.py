"""tree_mask_build on the GPU against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

from helpers import anc_u64, say
from oracle import mask as OM
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run_and_compare(lib, parent, ctx, depth_in=None, dense=True):
    B, N = parent.shape
    say(f"mask B={B} N={N} depth_in={depth_in is not None}")
    p = torch.from_numpy(np.ascontiguousarray(parent, dtype=np.int32)).to(DEV)
    c = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(DEV)
    d = None if depth_in is None else torch.from_numpy(np.asarray(depth_in, dtype=np.int32)).to(DEV)
    out = lib.tree_mask_build(p, c, d, dense_bias=dense)
    torch.cuda.synchronize()
    ref = OM.tree_mask(parent, ctx, depth_in)
    assert np.array_equal(out["status"].cpu().numpy(), ref["status"])
    assert np.array_equal(anc_u64(out["anc"]), ref["anc"])
    assert np.array_equal(out["depth"].cpu().numpy(), ref["depth"])
    assert np.array_equal(out["pos"].cpu().numpy(), ref["pos"])
    if dense:
        assert np.array_equal(out["dense_bias"].cpu().numpy(), OM.node_bias(ref["vis"]))
    return out


@pytest.mark.parametrize("kind,B,N,vocab", [("random_parent", 1, 16, 1000), ("leaf_sibling", 8, 32, 1000),
                                            ("spine_first", 32, 32, 1000), ("ddtree", 64, 64, 4096),
                                            ("random_parent", 16, 64, 1000), ("chain", 2, 64, 10),
                                            ("star", 3, 64, 10), ("random_parent", 5, 1, 10),
                                            ("random_parent", 7, 33, 10), ("random_parent", 4, 128, 1000),
                                            ("chain", 2, 128, 10), ("star", 2, 100, 10),
                                            ("ddtree", 8, 128, 4096), ("random_parent", 3, 65, 10),
                                            ("chain", 1, 65, 10)])
def test_trees(lib, kind, B, N, vocab):
    tb = W.make_trees(40, kind, B, N, vocab, max_depth=8)
    ctx = np.random.default_rng(1).integers(1, 40000, size=B)
    run_and_compare(lib, tb.parent, ctx, tb.depth)
    run_and_compare(lib, tb.parent, ctx, None, dense=False)


def test_status_codes(lib):
    parent = np.array([[-1, 0, 0, 1], [-1, 1, 0, 1], [-1, 0, 3, 1], [-2, 0, 0, 1],
                       [-1, 0, 0, 1], [-1, 0, 0, 1], [-1, 0, 0, 1]])
    depth = np.array([[1, 2, 2, 3]] * 4 + [[1, 2, 2, 2], [1, 2, 2, 3], [1, 1, 2, 3]])
    ctx = np.array([5, 5, 5, 5, 5, 0, 0])
    out = run_and_compare(lib, parent, ctx, depth)
    assert out["status"].cpu().tolist() == [0, 1, 1, 1, 2, 3, 2]


def test_worked_example(lib):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ddtree_worked_example.json")))
    out = run_and_compare(lib, np.array([g["parents"]]), [100], np.array([g["depths"]]))
    assert out["depth"][0].cpu().tolist() == g["depths"]
