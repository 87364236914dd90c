"""Benchmark of one tree-verify step on one MI355X.

A step is one pass of the whole verify path over one batch: tree_mask_build,
tree_verify_attn for a 512-token sliding-window layer and for a global layer,
tree_walk_accept and tree_gdn_verify.  The batch is the mixed workload: 32
sequences with context lengths uniform in [1024, 32768], random spine-first
trees of N = 32 nodes (max depth 8), Hq = 16, Hkv = 8, D = 256, bf16, paged
KV in 16-token pages under a random block table.  That workload states no
vocabulary or GDN shape, so the walk runs over [32, 33, 262144] bf16 logits
(the DDTree workload's vocabulary) and the GDN layer uses H = 16,
Dk = Dv = 128 over the same trees.

Prints one JSON line: verified tree nodes per second (B * N per step), the
roofline of the dominant kernel (the global-layer attention: context K/V bytes
over its event-timed duration against 8 TB/s) and the CPU oracle on a bounded
sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-curve", action="store_true",
                    help="skip the cost curve over tree sizes and the tree-construction timing "
                         "(the curve's attention calls share kernel names with the step's, which "
                         "muddles a kernel trace of the step)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2)
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per global-layer attention call (rocprofv3 --pmc)")
    ap.add_argument("--attn-only", type=int, default=0, choices=[0, 2, 4],
                    help="instead of the verify step, time tree_verify_attn alone on the full-size "
                         "shapes of this attention workload (2: batch 8 leaf-sibling trees, "
                         "4: DDTree-shaped batch 64) and print one JSON line for that kernel")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this many MiB "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


ATTN_SRC = os.path.join(ROOT, "tree_verify_attention_amd", "csrc", "tv_attn.hip")


def source_digest(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha1(f.read()).hexdigest()


def measured_traffic(path: str):
    """HBM bytes per global-layer call from counter runs, if they were taken
    on the attention source as it is now (else None)."""
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha1") != source_digest(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


class Step:
    """Inputs resident in HBM, preallocated outputs and workspaces."""

    def __init__(self, dev):
        import tree_verify_attention_amd as tv
        from synth import configs as CF
        from synth import workloads as W
        self.tv = tv
        tv.load()
        c = dict(CF.ATTN[3])
        wins = c.pop("windows")
        c.pop("vocab")
        self.B, self.N = c["B"], c["N"]
        self.layers = []
        trees = None
        ctx = None
        for li, w in enumerate(wins):
            x = W.attn_inputs(3, device=dev, kv_on_device=True, layer=li, window=w,
                              trees=trees, ctx_len=ctx, **c)
            trees, ctx = x.trees, x.ctx_len.cpu().numpy()
            self.layers.append(x)
        self.trees = trees
        self.parent = torch.from_numpy(trees.parent).to(dev)
        self.tokens = torch.from_numpy(trees.tokens).to(dev)
        self.ctx_len = self.layers[0].ctx_len
        self.V = 262144
        self.logits = W.walk_inputs(3, trees, self.V, torch.bfloat16, device=dev, on_device=True).logits
        g = CF.GDN[5]
        self.gdn = W.gdn_inputs(3, B=self.B, N=self.N, H=g["H"], Dk=g["Dk"], Dv=g["Dv"], tree="spine_first",
                                dtype=torch.bfloat16, trees=trees, device=dev)
        B, N = self.B, self.N
        self.mask_out = dict(anc=torch.empty(B, N, tv.anc_words(N), dtype=torch.int64, device=dev),
                             depth=torch.empty(B, N, dtype=torch.int32, device=dev),
                             pos=torch.empty(B, N, dtype=torch.int32, device=dev),
                             status=torch.empty(B, dtype=torch.int32, device=dev), dense_bias=None)
        self.attn_out = [torch.empty_like(x.q) for x in self.layers]
        self.attn_ws = []
        for x in self.layers:
            n = tv.tree_verify_attn_workspace_size(B, N, x.Hq, x.Hkv, x.D, x.max_ctx_len, x.window)
            self.attn_ws.append(torch.empty(max(n, 1), dtype=torch.uint8, device=dev))
        self.walk_out = dict(accepted_tokens=torch.empty(B, N + 1, dtype=torch.int32, device=dev),
                             accepted_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
                             num_accepted=torch.empty(B, dtype=torch.int32, device=dev))
        self.walk_ws = torch.empty(tv.tree_walk_accept_workspace_size(B, N), dtype=torch.uint8, device=dev)
        self.gdn_out = torch.empty(B, N, g["H"], g["Dv"], dtype=torch.bfloat16, device=dev)

    def kv_bytes(self, li):
        x = self.layers[li]
        ctx = x.ctx_len.cpu().numpy().astype(np.int64)
        per_tok = 2 * x.Hkv * x.D * x.k_cache.element_size()
        if x.window > 0:
            # the union of keys the nodes can see: the last window - 1 positions
            seen = np.minimum(ctx, x.window - 1)
        else:
            seen = ctx
        return int(seen.sum() * per_tok)

    def run(self, events=None):
        tv = self.tv
        ev = events or {}

        def mark(name, i):
            if name in ev:
                ev[name][i].record()

        mark("mask", 0)
        tv.tree_mask_build(self.parent, self.ctx_len, out=self.mask_out)
        mark("mask", 1)
        m = self.mask_out
        for li, x in enumerate(self.layers):
            nm = f"attn{li}"
            mark(nm, 0)
            tv.tree_verify_attn(x.q, x.k_node, x.v_node, x.k_cache, x.v_cache, x.block_table, x.ctx_len,
                                x.max_ctx_len, m["anc"], m["pos"], x.window, x.scale,
                                out=self.attn_out[li], workspace=self.attn_ws[li])
            mark(nm, 1)
        mark("walk", 0)
        tv.tree_walk_accept(self.tokens, self.parent, self.logits, out=self.walk_out, workspace=self.walk_ws)
        mark("walk", 1)
        g = self.gdn
        mark("gdn", 0)
        tv.tree_gdn_verify(g.q, g.k, g.v, g.alpha, g.beta, g.S0, m["anc"], out=self.gdn_out)
        mark("gdn", 1)


def next_rows(step: Step, dev, reps: int) -> dict:
    """The commits after the walk, outside the timed step: the GDN state
    advanced over walk-shaped accepted paths (root paths of random nodes), and
    the same paths' keys and values of the global layer copied into a small
    pool of two fresh pages per sequence (the step's own caches stay as they
    are).  Event-timed averages over `reps` calls."""
    tv = step.tv
    from synth import workloads as W
    acc, na = W.accepted_paths(3, step.trees.parent)
    acc_t = torch.from_numpy(acc).to(dev)
    na_t = torch.from_numpy(na).to(dev)
    g = step.gdn
    S_out = torch.empty_like(g.S0)
    x = step.layers[1]
    B = step.B
    ctx = x.ctx_len.cpu().numpy().astype(np.int64)
    width = int((ctx.max() + step.N + 15) // 16 + 1)
    table = np.full((B, width), -1, dtype=np.int32)
    for b in range(B):
        table[b, ctx[b] // 16] = 2 * b
        table[b, ctx[b] // 16 + 1] = 2 * b + 1
    table_t = torch.from_numpy(table).to(dev)
    pool_k = torch.zeros(2 * B, x.Hkv, 16, x.D, dtype=x.k_node.dtype, device=dev)
    pool_v = torch.zeros_like(pool_k)

    def timed(fn):
        for _ in range(3):
            fn()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) / reps

    gms = timed(lambda: tv.tree_gdn_commit(g.k, g.v, g.alpha, g.beta, g.S0, acc_t, na_t, out=S_out))
    kms = timed(lambda: tv.tree_kv_commit(x.k_node, x.v_node, acc_t, na_t, x.ctx_len, table_t, pool_k, pool_v))
    gbytes = 2 * g.S0.numel() * 4  # the state read and written once
    kbytes = int(na.sum()) * 2 * x.Hkv * x.D * x.k_node.element_size() * 2  # rows read and written
    return {"accepted_per_seq_mean": round(float(na.mean()), 2),
            "gdn_commit": {"ms": round(gms, 4), "bytes": gbytes, "GBps": round(gbytes / (gms * 1e-3) / 1e9, 1),
                           "frac_of_8TBps": round(gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "kv_commit": {"ms": round(kms, 4), "bytes": kbytes}}


def tree_construction(step: Step, dev, reps: int) -> dict:
    """Draft-tree construction at the DDTree workload's shape, outside the
    step: 64 sequences x 8 depths of 262144-entry bf16 draft logits (sigma 8,
    seeded on the device), top 8 per depth, then best-first growth to 64
    nodes (one candidate per round, and 8 per round).  Event-timed averages."""
    tv = step.tv
    from synth import workloads as W
    B, L, V, K, N = 64, 8, 262144, 8, 64
    x = W.draft_logits(4, B, L, V, torch.bfloat16, device=dev, on_device=True)
    cand = tv.tree_draft_topk(x, K)
    tree = tv.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 1)

    def timed(fn):
        for _ in range(3):
            fn()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) / reps

    tk = timed(lambda: tv.tree_draft_topk(x, K, out=cand))
    b1 = timed(lambda: tv.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 1, out=tree))
    b8 = timed(lambda: tv.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 8, out=tree))
    nbytes = x.numel() * x.element_size()
    del x
    return {"workload": "B=64, 8 depths x 262144 bf16 draft logits, top 8, budget 64",
            "topk_ms": round(tk, 4), "topk_GBps": round(nbytes / (tk * 1e-3) / 1e9, 1),
            "topk_frac_of_8TBps": round(nbytes / (tk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "build_ms_w1": round(b1, 4), "build_ms_w8": round(b8, 4)}


CURVE_NODES = (1, 2, 4, 8, 16, 32, 64, 128)


def cost_curve(step: Step, dev, reps: int) -> dict:
    """Verify cost against tree size on the mixed batch: the same 32 sequences,
    context lengths, paged caches and head shapes, with spine-first trees of
    N nodes (depth <= 8) and fresh seeded queries and node keys/values for
    each N.  Per N: event-timed mask + window-layer + global-layer attention
    (the verify calls of that workload), averaged over `reps` passes; the
    least-squares slope gives the cost per extra candidate."""
    tv = step.tv
    from synth import workloads as W
    B = step.B
    res = {"N": [], "ms": [], "mask_ms": [], "window_ms": [], "global_ms": []}
    for N in CURVE_NODES:
        trees = W.make_trees(3, "spine_first", B, N, 1000, max_depth=min(8, N), tag=1000 + N)
        parent = torch.from_numpy(trees.parent).to(dev)
        mo = dict(anc=torch.empty(B, N, tv.anc_words(N), dtype=torch.int64, device=dev),
                  depth=torch.empty(B, N, dtype=torch.int32, device=dev),
                  pos=torch.empty(B, N, dtype=torch.int32, device=dev),
                  status=torch.empty(B, dtype=torch.int32, device=dev), dense_bias=None)
        calls = []
        for li, x in enumerate(step.layers):
            seed = 7000 + 10 * N + 3 * li
            q = W._device_normal(seed, (B, N, x.Hq, x.D), x.q.dtype, dev)
            kn = W._device_normal(seed + 1, (B, N, x.Hkv, x.D), x.q.dtype, dev)
            vn = W._device_normal(seed + 2, (B, N, x.Hkv, x.D), x.q.dtype, dev)
            ws = torch.empty(max(1, tv.tree_verify_attn_workspace_size(B, N, x.Hq, x.Hkv, x.D, x.max_ctx_len,
                                                                       x.window)), dtype=torch.uint8, device=dev)
            o = torch.empty_like(q)
            calls.append((x, q, kn, vn, ws, o))
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]

        def once(e=None):
            if e: e[0].record()
            tv.tree_mask_build(parent, step.ctx_len, out=mo)
            if e: e[1].record()
            for li, (x, q, kn, vn, ws, o) in enumerate(calls):
                tv.tree_verify_attn(q, kn, vn, x.k_cache, x.v_cache, x.block_table, x.ctx_len, x.max_ctx_len,
                                    mo["anc"], mo["pos"], x.window, x.scale, out=o, workspace=ws)
                if e: e[2 + li].record()
        for _ in range(10):
            once()
        torch.cuda.synchronize()
        for i in range(reps):
            once(ev[i])
        torch.cuda.synchronize()
        # mask, window layer, global layer
        parts = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(3)] for e in ev]).mean(axis=0)
        res["N"].append(N)
        res["mask_ms"].append(round(float(parts[0]), 4))
        res["window_ms"].append(round(float(parts[1]), 4))
        res["global_ms"].append(round(float(parts[2]), 4))
        res["ms"].append(round(float(parts.sum()), 4))
        del calls
    n = np.array(res["N"], dtype=np.float64)
    t = np.array(res["ms"])
    small = n <= 32
    res["ms_per_candidate_N_le_32"] = round(float(np.polyfit(n[small], t[small], 1)[0]), 5)
    res["ms_per_candidate_all"] = round(float(np.polyfit(n, t, 1)[0]), 5)
    res["workload"] = ("mixed batch (B=32, ctx U[1024,32768], Hq=16, Hkv=8, D=256, bf16) with "
                       "spine-first trees of N nodes; mask + W=512 layer + global layer")
    return res


def cpu_baseline(step: Step, nseq: int):
    """The oracle on the first `nseq` sequences of the same step (mask, both
    attention layers, walk, GDN), timed on this host's cores."""
    from oracle import attn as OA, gdn as OG, mask as OM, walk as OW
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    b_idx = list(range(nseq))
    par = step.trees.parent[b_idx]
    toks = step.trees.tokens[b_idx]
    # bring the sample's inputs to the host (outside the timed region)
    host = []
    for x in step.layers:
        G = x.Hq // x.Hkv
        per = []
        for b in b_idx:
            ctx = int(x.ctx_len[b])
            pages = x.block_table[b, :(ctx + 15) // 16].long()
            kc = x.k_cache[pages].double().cpu().numpy()   # [pages, Hkv, 16, D]
            vc = x.v_cache[pages].double().cpu().numpy()
            table = np.arange(len(pages), dtype=np.int64)
            per.append((ctx, kc, vc, table, x.q[b].double().cpu().numpy(), x.k_node[b].double().cpu().numpy(),
                        x.v_node[b].double().cpu().numpy()))
        host.append((x, G, per))
    logits = step.logits[b_idx].double().cpu().numpy()
    g = step.gdn
    gin = [t[b_idx].double().cpu().numpy() for t in (g.q, g.k, g.v, g.alpha, g.beta, g.S0)]
    ctx_np = step.ctx_len.cpu().numpy()[b_idx]

    t0 = time.perf_counter()
    m = OM.tree_mask(par, ctx_np)
    for x, G, per in host:
        for i, (ctx, kc, vc, table, q, kn, vn) in enumerate(per):
            OA.tree_attn(q[None], kn[None], vn[None], kc, vc, table[None], np.array([ctx]),
                         m["vis"][i:i + 1], m["pos"][i:i + 1], x.window, x.scale)
    OW.tree_walk(toks, par, logits)
    OG.gdn_tree(*gin, par)
    dt = time.perf_counter() - t0
    nodes = nseq * step.N
    return dict(value=nodes / dt, unit="nodes/s", cores=int(threads), kind="oracle",
                sample=f"first {nseq} of {step.B} sequences of the step (all {step.N} nodes; mask, "
                       f"window and global attention, walk over 262144-entry rows, GDN), "
                       f"{dt:.1f} s on {len(os.sched_getaffinity(0))} host cores")


def attn_only(args, dev) -> dict:
    """tree_verify_attn alone on one full-size attention workload, inputs
    resident in HBM: K warm calls timed with events on the current stream."""
    import tree_verify_attention_amd as tv
    from synth import configs as CF
    from synth import workloads as W
    c = CF.reduced(args.attn_only)
    c.pop("windows")
    c.pop("vocab")
    x = W.attn_inputs(args.attn_only, device=dev, kv_on_device=True, **c)
    m = tv.tree_mask_build(torch.from_numpy(x.trees.parent).to(dev), x.ctx_len)
    out = torch.empty_like(x.q)
    n = tv.tree_verify_attn_workspace_size(x.B, x.N, x.Hq, x.Hkv, x.D, x.max_ctx_len, 0)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    call = lambda: tv.tree_verify_attn(x.q, x.k_node, x.v_node, x.k_cache, x.v_cache, x.block_table,
                                       x.ctx_len, x.max_ctx_len, m["anc"], m["pos"], 0, x.scale,
                                       out=out, workspace=ws)
    for _ in range(args.warmup):
        call()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        call()
    z.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(z) / args.steps
    ctx = x.ctx_len.cpu().numpy().astype(np.int64)
    kv = int(ctx.sum()) * 2 * x.Hkv * x.D * x.k_cache.element_size()
    # QK^T and P.V over the context keys: 2 products x 2 flops per multiply-add
    flops = 4.0 * float(ctx.sum()) * x.Hq * x.N * x.D
    return {"attn_only_config": args.attn_only, "B": x.B, "N": x.N, "Hq": x.Hq, "Hkv": x.Hkv, "D": x.D,
            "sum_ctx": int(ctx.sum()), "steps": args.steps, "warmup": args.warmup, "ms_per_call": round(ms, 4),
            "kv_GBps": round(kv / (ms * 1e-3) / 1e9, 1), "kv_frac_of_8TBps": round(kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_mfma_2500TFLOPs": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.attn_only:
        print(json.dumps(attn_only(args, dev)), flush=True)
        return
    step = Step(dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    names = ["mask", "attn0", "attn1", "walk", "gdn"]
    per_call = {n: 0.0 for n in names}
    # timed region: exactly K steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step.run()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # per-call durations: the same steps again with events around each call
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    for i in range(args.steps):
        step.run(evs[i])
    torch.cuda.synchronize()
    for e in evs:
        for n in names:
            per_call[n] += e[n][0].elapsed_time(e[n][1]) / args.steps

    nodes_per_s = step.B * step.N / (ms_per_step * 1e-3)
    kv_global = step.kv_bytes(1)
    kv_window = step.kv_bytes(0)
    achieved = kv_global / (per_call["attn1"] * 1e-3) / 1e9
    traffic = measured_traffic(args.traffic)
    out = {
        "metric": "verified tree nodes/sec + KV-stream HBM GB/s (% of peak), 1x MI355X",
        "value": round(nodes_per_s, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixed batch: B=32, N=32 spine-first trees (depth<=8), ctx U[1024,32768], "
                               "Hq=16, Hkv=8, D=256, bf16, 16-token pages; W=512 layer + global layer; "
                               "walk over [32,33,262144] bf16 logits; GDN H=16 Dk=Dv=128",
                   "global_batch": step.B, "nodes_per_tree": step.N,
                   "sum_ctx": int(step.ctx_len.sum().item()), "parallelism": "single GPU"},
        "kv_stream": {"global_layer_GBps": round(achieved, 1),
                      "global_layer_frac_of_8TBps": round(achieved / HBM_PEAK_GBS, 4),
                      "window_layer_GBps": round(kv_window / (per_call["attn0"] * 1e-3) / 1e9, 1),
                      "pair_GBps": round((kv_global + kv_window) / ((per_call["attn0"] + per_call["attn1"]) * 1e-3) / 1e9, 1)},
        "calls_ms": {n: round(v, 4) for n, v in per_call.items()},
        "roofline": {"kernel": "tree_verify_attn on the global layer: attn_stream_kernel + "
                               "attn_merge_stream_kernel (one call, event-timed)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": kv_global,
                     "bytes_per_unit": "8192 B of K+V per (context token, sequence): 2 x Hkv 8 x D 256 x 2 B",
                     "call_ms": round(per_call["attn1"], 4)},
    }
    out["next_rows"] = next_rows(step, dev, args.steps)
    if not args.no_curve:
        out["next_rows"]["cost_curve"] = cost_curve(step, dev, min(args.steps, 20))
        out["next_rows"]["tree_construction"] = tree_construction(step, dev, min(args.steps, 20))
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = n
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(step, args.cpu_sample_seqs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
