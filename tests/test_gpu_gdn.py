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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tree,N", [("chain", 64), ("star", 17), ("random_parent", 64),
                                    ("random_parent", 1), ("leaf_sibling", 32), ("spine_first", 40)])
def test_trees(lib, dtype, tree, N):
    x = W.gdn_inputs(51, B=3, N=N, H=4, Dk=128, Dv=128, tree=tree, dtype=dtype, device=DEV)
    check(lib, x, tree)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_strong_state_and_gates(lib, dtype):
    """Larger committed state and gates spread over (0, 1] on deep random trees
    (gate products far below 1, so the gate ratios of distant ancestors matter)."""
    x = W.gdn_inputs(52, B=2, N=64, H=3, Dk=128, Dv=128, tree="random_parent", dtype=dtype,
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
