"""The five verify workloads (shapes only) and reduced variants of them.

c1  tiny fp32: B=1, N=16 random-parent tree, Hq=8, Hkv=2, D=64, ctx 512,
    logits [17, 1000] fp32.
c2  B=8 bf16 leaf-sibling trees (spine of depth 8, 4 candidates per spine
    position, N=32), Hq=16, Hkv=8, D=256, ctx 4096.
c3  B=32 bf16 random spine-first trees (N=32, max depth 8), ctx uniform in
    [1024, 32768], Hq=16, Hkv=8, D=256; one layer with a 512-token sliding
    window and one global layer.
c4  B=64 bf16 DDTree trees (top-8 per depth, budget 64, max depth 8),
    Hq=64, Hkv=8, D=128, ctx 32768, logits [64, 65, 262144] bf16.
c5  Gated DeltaNet tree verify: B=16, H=16, Dk=Dv=128, N=32 spine-first trees
    of max depth 8, bf16 q/k/v, fp32 alpha/beta/state.
"""
from __future__ import annotations

import torch

ATTN = {
    1: dict(B=1, N=16, Hq=8, Hkv=2, D=64, ctx_lo=512, ctx_hi=512, tree="random_parent",
            dtype=torch.float32, windows=(0,), vocab=1000),
    2: dict(B=8, N=32, Hq=16, Hkv=8, D=256, ctx_lo=4096, ctx_hi=4096, tree="leaf_sibling",
            dtype=torch.bfloat16, windows=(0,), vocab=262144),
    3: dict(B=32, N=32, Hq=16, Hkv=8, D=256, ctx_lo=1024, ctx_hi=32768, tree="spine_first",
            dtype=torch.bfloat16, windows=(512, 0), vocab=262144),
    4: dict(B=64, N=64, Hq=64, Hkv=8, D=128, ctx_lo=32768, ctx_hi=32768, tree="ddtree",
            dtype=torch.bfloat16, windows=(0,), vocab=262144),
}

GDN = {
    5: dict(B=16, N=32, H=16, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16),
}

# vocabulary of the target logits per workload (c1 and c4 state theirs; the
# others borrow c4's 262144-entry vocabulary where a walk is run on them)
VOCAB = {1: 1000, 2: 262144, 3: 262144, 4: 262144, 5: 262144}


def reduced(config: int, **override) -> dict:
    """A copy of an attention workload's shape with fields overridden."""
    d = dict(ATTN[config])
    d.update(override)
    return d
