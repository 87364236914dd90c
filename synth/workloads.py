"""Seeded synthetic workloads shaped like the pages' verify steps.

Only input generation lives here (random tensors, paging, trees, planted
logits); none of the verify arithmetic does.  Every tensor comes from a PCG64
stream keyed by (workload id, tensor tag, sequence index), or, for the bulk
paged KV and logits of the large workloads, from a seeded ``torch.Generator``
on the device (the same bytes are then copied back for the oracle).

Floating-point tensors are drawn in fp32; bf16 workloads round them to nearest
even with torch's CPU conversion.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from . import trees as T

BLOCK = 16  # tokens per KV page

# tensor tags for the PCG64 streams
TAG_TREE, TAG_CTX, TAG_PERM, TAG_Q, TAG_KN, TAG_VN, TAG_KC, TAG_VC, TAG_LOGIT, TAG_PLANT = range(10)
TAG_GQ, TAG_GK, TAG_GV, TAG_GA, TAG_GB, TAG_GS = range(20, 26)
TAG_ACC = 30
TAG_DRAFT, TAG_CAND = 40, 41


@dataclasses.dataclass
class TreeBatch:
    parent: np.ndarray            # int32 [B, N]
    tokens: np.ndarray            # int32 [B, N]
    depth: Optional[np.ndarray]   # int32 [B, N] when the construction fixes it


@dataclasses.dataclass
class AttnInputs:
    """One attention layer of a tree-verify step.  Tensors are torch tensors
    on ``device``; dtype is torch.float32 or torch.bfloat16."""
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    window: int
    scale: float
    trees: TreeBatch
    ctx_len: torch.Tensor        # int32 [B]
    block_table: torch.Tensor    # int32 [B, max_blocks], -1 past the end
    num_blocks: int
    q: torch.Tensor              # [B, N, Hq, D]
    k_node: torch.Tensor         # [B, N, Hkv, D]
    v_node: torch.Tensor         # [B, N, Hkv, D]
    k_cache: torch.Tensor        # [num_blocks, Hkv, BLOCK, D]
    v_cache: torch.Tensor        # [num_blocks, Hkv, BLOCK, D]

    @property
    def max_ctx_len(self) -> int:
        return int(self.block_table.shape[1]) * BLOCK


@dataclasses.dataclass
class WalkInputs:
    trees: TreeBatch
    logits: torch.Tensor          # [B, N+1, V]


@dataclasses.dataclass
class GdnInputs:
    B: int
    N: int
    H: int
    Dk: int
    Dv: int
    trees: TreeBatch
    q: torch.Tensor               # [B, N, H, Dk] (bf16 or fp32)
    k: torch.Tensor               # [B, N, H, Dk]
    v: torch.Tensor               # [B, N, H, Dv]
    alpha: torch.Tensor           # fp32 [B, N, H]
    beta: torch.Tensor            # fp32 [B, N, H]
    S0: torch.Tensor              # fp32 [B, H, Dk, Dv]


# ---------------------------------------------------------------- trees

def make_trees(config: int, kind: str, B: int, N: int, vocab: int, *, max_depth: int = 8,
               width: int = 4, top_k: int = 8, sigma: float = 8.0, tag: int = TAG_TREE) -> TreeBatch:
    par, tok, dep = [], [], []
    for b in range(B):
        r = T.rng_for(config, tag, b)
        if kind == "random_parent":
            p, t, d = T.random_parent_tree(r, N, vocab)
        elif kind == "chain":
            p, t, d = T.chain_tree(r, N, vocab)
        elif kind == "star":
            p, t, d = T.star_tree(r, N, vocab)
        elif kind == "leaf_sibling":
            assert N % width == 0
            p, t, d = T.leaf_sibling_tree(r, N // width, width, vocab)
        elif kind == "spine_first":
            p, t, d = T.spine_first_tree(r, N, min(max_depth, N), vocab)
        elif kind == "ddtree":
            p, t, d = T.ddtree(r, vocab, top_k, N, max_depth, sigma)
            if len(p) < N:  # heap exhausted before the budget (tiny vocab/top_k)
                raise ValueError("ddtree produced fewer nodes than the budget")
        else:
            raise ValueError(kind)
        par.append(p)
        tok.append(t)
        dep.append(d)
    depth = None if any(d is None for d in dep) else np.stack(dep).astype(np.int32)
    return TreeBatch(np.stack(par).astype(np.int32), np.stack(tok).astype(np.int32), depth)


# ---------------------------------------------------------------- helpers

def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def _normal(config: int, tag: int, b: int, shape, dtype: torch.dtype, std: float = 1.0) -> torch.Tensor:
    r = T.rng_for(config, tag, b)
    return _round(r.standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)


def _device_normal(seed: int, shape, dtype: torch.dtype, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    # fill in slabs so that the fp32 staging stays small
    flat = out.view(-1)
    step = 1 << 26
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def paging(config: int, ctx_len: np.ndarray, tag: int = TAG_PERM):
    """Block table over a randomly permuted pool of exactly sum(ceil(ctx/16))
    pages; unused table entries are -1."""
    nblk = [(int(c) + BLOCK - 1) // BLOCK for c in ctx_len]
    pool = int(sum(nblk))
    max_blocks = max(nblk) if nblk else 0
    perm = T.rng_for(config, tag, 0).permutation(pool).astype(np.int32)
    table = np.full((len(ctx_len), max(max_blocks, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, pool


# ---------------------------------------------------------------- attention

def attn_inputs(config: int, *, B: int, N: int, Hq: int, Hkv: int, D: int,
                ctx_lo: int, ctx_hi: int, tree: str, dtype: torch.dtype, window: int = 0,
                layer: int = 0, vocab: int = 1000, max_depth: int = 8, width: int = 4,
                trees: Optional[TreeBatch] = None, ctx_len: Optional[np.ndarray] = None,
                device="cpu", kv_on_device: bool = False) -> AttnInputs:
    """Inputs of one attention layer.  ``layer`` selects an independent KV
    pool and Q (layers of one step share the trees and context lengths)."""
    if trees is None:
        trees = make_trees(config, tree, B, N, vocab, max_depth=max_depth, width=width)
    if ctx_len is None:
        r = T.rng_for(config, TAG_CTX, 0)
        ctx_len = r.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.int32)
    table, pool = paging(config, ctx_len)
    lt = 100 * layer
    q = torch.stack([_normal(config, TAG_Q + lt, b, (N, Hq, D), dtype) for b in range(B)])
    kn = torch.stack([_normal(config, TAG_KN + lt, b, (N, Hkv, D), dtype) for b in range(B)])
    vn = torch.stack([_normal(config, TAG_VN + lt, b, (N, Hkv, D), dtype) for b in range(B)])
    shape = (pool, Hkv, BLOCK, D)
    if kv_on_device:
        kc = _device_normal(config * 1000 + 2 * layer + 1, shape, dtype, device)
        vc = _device_normal(config * 1000 + 2 * layer + 2, shape, dtype, device)
    else:
        kc = _normal(config, TAG_KC + lt, 0, shape, dtype).to(device)
        vc = _normal(config, TAG_VC + lt, 0, shape, dtype).to(device)
    return AttnInputs(
        B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, window=int(window), scale=1.0 / math.sqrt(D),
        trees=trees, ctx_len=torch.from_numpy(ctx_len).to(device),
        block_table=torch.from_numpy(table).to(device), num_blocks=pool,
        q=q.to(device), k_node=kn.to(device), v_node=vn.to(device), k_cache=kc, v_cache=vc)


# ---------------------------------------------------------------- walk

def walk_inputs(config: int, trees: TreeBatch, vocab: int, dtype: torch.dtype, *,
                device="cpu", on_device: bool = False, plant: float = 0.0,
                plant_len: Optional[int] = None) -> WalkInputs:
    """Target logits [B, N+1, vocab] ~ N(0, 1).  With ``plant`` > 0 a random
    root-to-leaf path of the tree is planted: the row of the last accepted
    token and of each path node gets ``plant`` added at the token of the next
    path node, so that a greedy walk follows the path for ``plant_len`` steps
    (default: the whole path)."""
    B, N = trees.parent.shape
    if on_device:
        logits = _device_normal(config * 1000 + 999, (B, N + 1, vocab), dtype, device)
    else:
        logits = torch.stack([_normal(config, TAG_LOGIT, b, (N + 1, vocab), dtype) for b in range(B)])
    if plant > 0.0:
        for b in range(B):
            r = T.rng_for(config, TAG_PLANT, b)
            par = trees.parent[b]
            # choose a leaf uniformly and plant its root path
            is_parent = np.zeros(N, dtype=bool)
            for p in par:
                if p >= 0:
                    is_parent[p] = True
            leaves = np.flatnonzero(~is_parent)
            leaf = int(leaves[r.integers(0, len(leaves))])
            path = []
            cur = leaf
            while cur >= 0:
                path.append(cur)
                cur = int(par[cur])
            path.reverse()
            steps = len(path) if plant_len is None else min(plant_len, len(path))
            row = 0
            for i in range(steps):
                node = path[i]
                tok = int(trees.tokens[b, node])
                if 0 <= tok < vocab:
                    logits[b, row, tok] += plant
                row = 1 + node
    return WalkInputs(trees=trees, logits=logits.to(device) if not on_device else logits)


# ---------------------------------------------------------------- GDN

def gdn_inputs(config: int, *, B: int, N: int, H: int, Dk: int, Dv: int, tree: str,
               dtype: torch.dtype, max_depth: int = 8, trees: Optional[TreeBatch] = None,
               s0_std: float = 0.02, device="cpu") -> GdnInputs:
    """q, k ~ N(0,1) L2-normalised over the head dimension in fp32, then
    rounded to ``dtype``; v ~ N(0,1); alpha ~ U(0.9, 1.0); beta ~ U(0, 1);
    S0 ~ s0_std * N(0, 1) in fp32."""
    if trees is None:
        trees = make_trees(config, tree, B, N, 1000, max_depth=max_depth)
    qs, ks, vs, als, bes, ss = [], [], [], [], [], []
    for b in range(B):
        rq = T.rng_for(config, TAG_GQ, b).standard_normal((N, H, Dk), dtype=np.float32)
        rk = T.rng_for(config, TAG_GK, b).standard_normal((N, H, Dk), dtype=np.float32)
        rq /= np.linalg.norm(rq, axis=-1, keepdims=True)
        rk /= np.linalg.norm(rk, axis=-1, keepdims=True)
        qs.append(_round(rq, dtype))
        ks.append(_round(rk, dtype))
        vs.append(_normal(config, TAG_GV, b, (N, H, Dv), dtype))
        als.append(torch.from_numpy(T.rng_for(config, TAG_GA, b).uniform(0.9, 1.0, (N, H)).astype(np.float32)))
        bes.append(torch.from_numpy(T.rng_for(config, TAG_GB, b).uniform(0.0, 1.0, (N, H)).astype(np.float32)))
        ss.append(_normal(config, TAG_GS, b, (H, Dk, Dv), torch.float32, std=s0_std))
    st = lambda xs: torch.stack(xs).to(device)
    return GdnInputs(B=B, N=N, H=H, Dk=Dk, Dv=Dv, trees=trees, q=st(qs), k=st(ks), v=st(vs),
                     alpha=st(als), beta=st(bes), S0=st(ss))


# ---------------------------------------------------------------- accepted paths

def accepted_paths(config: int, parent: np.ndarray, *, tag: int = TAG_ACC, p_none: float = 0.15):
    """A walk-shaped outcome per sequence: the root path of a random node (root
    side first), or no accepted node with probability p_none.  Returns
    accepted_nodes int32 [B, N] (-1 past the count) and num_accepted int32 [B]."""
    B, N = parent.shape
    acc = np.full((B, N), -1, dtype=np.int32)
    na = np.zeros(B, dtype=np.int32)
    for b in range(B):
        r = T.rng_for(config, tag, b)
        if r.random() < p_none:
            continue
        t = int(r.integers(0, N))
        path = []
        while t >= 0:
            path.append(t)
            t = int(parent[b, t])
        path.reverse()
        acc[b, :len(path)] = path
        na[b] = len(path)
    return acc, na


# ---------------------------------------------------------------- draft distributions

def draft_logits(config: int, B: int, L: int, V: int, dtype: torch.dtype, *, sigma: float = 8.0,
                 device="cpu", on_device: bool = False) -> torch.Tensor:
    """Draft logits [B, L, V] of a factorised drafter: sigma * N(0, 1) per
    entry (the DDTree workload's recipe).  On the device the bulk comes from a
    seeded torch generator; otherwise from the per-sequence NumPy streams."""
    if on_device:
        out = _device_normal(config * 1000 + TAG_DRAFT, (B, L, V), torch.float32, device)
        return (out * sigma).to(dtype)
    xs = [_normal(config, TAG_DRAFT, b, (L, V), torch.float32, std=sigma) for b in range(B)]
    return torch.stack(xs).to(dtype).to(device)


def draft_candidates(config: int, B: int, L: int, K: int, *, ties: bool = False, scale: float = 1.5):
    """Per-depth candidates as a top-k step hands them over: distinct token ids
    [B, L, K] (int32) and log-probabilities [B, L, K] (float32, decreasing per
    depth, all negative).  With ties the values are multiples of 1/4, so that
    equal cumulative values occur."""
    tok = np.empty((B, L, K), dtype=np.int32)
    lp = np.empty((B, L, K), dtype=np.float32)
    for b in range(B):
        r = T.rng_for(config, TAG_CAND, b)
        tok[b] = r.permutation(100000)[:L * K].reshape(L, K)
        v = -np.sort(r.exponential(scale, size=(L, K)), axis=1)
        if ties:
            v = -np.ceil(-v * 4) / 4
        lp[b] = v.astype(np.float32)
    return tok, lp
