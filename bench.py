"""Benchmark of the tree-verify path on one MI355X.

Headline step: one pass of every step of the verify path over the mixed
workload (32 sequences with context lengths uniform in [1024, 32768], random
spine-first trees of N = 32 nodes of max depth 8, Hq = 16, Hkv = 8, D = 256,
bf16, paged KV in 16-token pages under a random block table):
tree_mask_build, tree_verify_attn for a 512-token sliding-window layer and for
a global layer, tree_walk_accept over [32, 33, 262144] bf16 logits (the DDTree
workload's vocabulary; the mixed workload names none) and tree_gdn_verify with
H = 16, Dk = Dv = 128 over the same trees.  `value` is verified tree nodes per
second (B * N per step) over K back-to-back steps with inputs resident in HBM.

`configs` times each of the five workloads as its own step (c1: mask +
attention + walk; c2: mask + attention; c3: mask + window layer + global layer;
c4: mask + attention + walk; c5: mask + GDN), every call separately: a 1 GiB
buffer is written and a 512 MiB one read before each repetition (outside the
timed region, so that L2 and the 256 MB last-level cache hold none of the
call's inputs and no dirty lines), and the
median, 10th and 90th percentile of the event-timed durations are reported,
with each workload's roofline.  `stream_ceiling` is the read rate a plain
streaming kernel reaches on the device, printed beside the vendor's 8 TB/s.
`cpu_baseline` is the oracle on a bounded sample of the headline step on the
host's cores, and with one thread.
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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of the MI355X


def log(msg: str):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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
    ap.add_argument("--cpu-sample-seqs", type=int, default=16,
                    help="sequences of the headline step the oracle runs on all host cores")
    ap.add_argument("--cpu-1t-seqs", type=int, default=8,
                    help="sequences of the headline step the oracle runs on one thread")
    ap.add_argument("--reps", type=int, default=50, help="timed repetitions per call in `configs`")
    ap.add_argument("--rep-warmup", type=int, default=10, help="untimed repetitions per call in `configs`")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB written before each repetition in `configs` (0: no flush)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload timing")
    ap.add_argument("--config", type=int, default=0, choices=[0, 1, 2, 3, 4, 5],
                    help="time only this workload's step (as in `configs`) and print its JSON line "
                         "(for per-workload kernel traces)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per global-layer attention call (rocprofv3 --pmc)")
    ap.add_argument("--attn-only", type=int, default=0, choices=[0, 2, 4],
                    help="instead of the verify step, time tree_verify_attn alone on the full-size "
                         "shapes of this attention workload (2: batch 8 leaf-sibling trees, "
                         "4: DDTree-shaped batch 64) and print one JSON line for that kernel")
    ap.add_argument("--tree-only", action="store_true",
                    help="time only draft-tree construction (top-k and growth) at the DDTree shape, "
                         "--steps calls each, and print one JSON line")
    ap.add_argument("--gdn-only", type=int, default=0,
                    help="instead of the verify step, time tree_gdn_verify alone on the verify-cost "
                         "curve's GDN shape (B=32, H=16, Dk=Dv=128, bf16, spine-first trees) with this "
                         "many nodes, warm calls, and print one JSON line for that kernel")
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


def tree_construction(step: Step, dev, reps: int, flush_mib: int = 1024) -> dict:
    """Draft-tree construction at the DDTree workload's shape, outside the
    step: 64 sequences x 8 depths of 262144-entry bf16 draft logits (sigma 8,
    seeded on the device), top 8 per depth, then best-first growth to 64
    nodes (one candidate per round, and 8 per round).  Event-timed averages
    of back-to-back calls; the top-k also cold (the logits nearly fit the
    last-level cache): a flush before each call, median and p10/p90."""
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
    cold = time_calls([("topk", lambda: tv.tree_draft_topk(x, K, out=cand))], reps, 2,
                      Flusher(dev, flush_mib))["topk"]
    b1 = timed(lambda: tv.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 1, out=tree))
    b8 = timed(lambda: tv.tree_build(cand["cand_tokens"], cand["cand_logprob"], N, 8, out=tree))
    nbytes = x.numel() * x.element_size()
    del x
    return {"workload": "B=64, 8 depths x 262144 bf16 draft logits, top 8, budget 64",
            "topk_ms": round(tk, 4), "topk_GBps": round(nbytes / (tk * 1e-3) / 1e9, 1),
            "topk_frac_of_8TBps": round(nbytes / (tk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "topk_cold": {**cold, "flush_mib": flush_mib,
                          "GBps": round(nbytes / (cold["median_ms"] * 1e-3) / 1e9, 1)},
            "build_ms_w1": round(b1, 4), "build_ms_w8": round(b8, 4)}


CURVE_NODES = (1, 2, 4, 8, 16, 32, 64, 128)


def cost_curve(step: Step, dev, reps: int) -> dict:
    """Verify cost against tree size on the mixed batch: the same 32 sequences,
    context lengths, paged caches and head shapes, with spine-first trees of
    N nodes (depth <= 8) and fresh seeded queries and node keys/values for
    each N.  Per N: event-timed mask + window-layer + global-layer attention
    (the verify calls of that workload), averaged over `reps` passes; the
    least-squares slope gives the cost per extra candidate.  The GDN layer's
    tree_gdn_verify over the same trees is timed alongside (gdn_ms)."""
    tv = step.tv
    from synth import workloads as W
    B = step.B
    res = {"N": [], "ms": [], "mask_ms": [], "window_ms": [], "global_ms": [], "gdn_ms": []}
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
        # the GDN layer (H = 16, Dk = Dv = 128, bf16) over the same trees
        g = W.gdn_inputs(3, B=B, N=N, H=16, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16,
                         trees=trees, device=dev)
        gout = torch.empty_like(g.v)
        gcall = lambda: tv.tree_gdn_verify(g.q, g.k, g.v, g.alpha, g.beta, g.S0, mo["anc"], out=gout)
        for _ in range(10):
            gcall()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            gcall()
        z.record()
        torch.cuda.synchronize()
        res["gdn_ms"].append(round(a.elapsed_time(z) / reps, 4))
        del g, gout
    n = np.array(res["N"], dtype=np.float64)
    t = np.array(res["ms"])
    small = n <= 32
    res["ms_per_candidate_N_le_32"] = round(float(np.polyfit(n[small], t[small], 1)[0]), 5)
    res["ms_per_candidate_all"] = round(float(np.polyfit(n, t, 1)[0]), 5)
    res["workload"] = ("mixed batch (B=32, ctx U[1024,32768], Hq=16, Hkv=8, D=256, bf16) with "
                       "spine-first trees of N nodes; ms = mask + W=512 layer + global layer; gdn_ms = "
                       "tree_gdn_verify with H=16, Dk=Dv=128, bf16, over the same trees (warm calls)")
    return res


def _probe_lib():
    import ctypes
    from tree_verify_attention_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.tv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.tv_probe_stream_read.restype = ctypes.c_int
    return lib


class Flusher:
    """Run before each timed repetition, on the same stream and outside the
    timed events: write a 1 GiB (by default) buffer, then read another half
    as large.  The write evicts the call's inputs from L2 and the 256 MB
    last-level cache; the read replaces the write's dirty lines with clean
    ones, so that the timed call does not pay for writing them back."""

    def __init__(self, dev, mib: int):
        import ctypes
        self.buf = torch.empty(max(mib, 0) << 20, dtype=torch.uint8, device=dev) if mib > 0 else None
        if self.buf is not None:
            self.rd = torch.empty(max(mib, 0) << 19, dtype=torch.uint8, device=dev).fill_(5)
            self.sink = torch.empty(1 << 14, dtype=torch.int32, device=dev)
            self.lib = _probe_lib()
            self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            self.args = (ctypes.c_void_p(self.rd.data_ptr()), self.rd.numel(), ctypes.c_void_p(self.sink.data_ptr()),
                         1 << 14, self.stream)
        self.k = 0

    def __call__(self):
        if self.buf is not None:
            self.k ^= 1
            self.buf.fill_(self.k)
            assert self.lib.tv_probe_stream_read(*self.args) == 0


def time_calls(calls, reps: int, warmup: int, flush: Flusher) -> dict:
    """calls: [(name, fn)] issued in order as one step.  Each repetition
    flushes before every call and brackets the call with events on the
    current stream.  Returns median, p10, p90 and mean per call in ms."""
    for _ in range(warmup):
        for _, fn in calls:
            flush()
            fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(reps)]
    for r in range(reps):
        for c, (_, fn) in enumerate(calls):
            flush()
            ev[r][c][0].record()
            fn()
            ev[r][c][1].record()
    torch.cuda.synchronize()
    out = {}
    for c, (name, _) in enumerate(calls):
        t = np.array([ev[r][c][0].elapsed_time(ev[r][c][1]) for r in range(reps)])
        out[name] = {"median_ms": round(float(np.median(t)), 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
                     "p90_ms": round(float(np.percentile(t, 90)), 5), "mean_ms": round(float(t.mean()), 5)}
    return out


def _kv_bytes(x, window: int) -> int:
    """Algorithmic context K+V bytes of one attention call: the union of the
    context positions the nodes can see (all of them without a window; the
    last window - 1 with one), 2 * Hkv * D elements each."""
    ctx = x.ctx_len.cpu().numpy().astype(np.int64)
    seen = np.minimum(ctx, window - 1) if window > 0 else ctx
    return int(seen.sum()) * 2 * x.Hkv * x.D * x.k_cache.element_size()


def _attn_flops(x) -> float:
    """QK^T and P.V over the context keys: 4 flops per (key, query row, dim)."""
    return 4.0 * float(x.ctx_len.cpu().numpy().astype(np.int64).sum()) * x.Hq * x.N * x.D


def _gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def _hbm_roof(kernel, nbytes, ms, ceiling):
    a = _gbps(nbytes, ms)
    r = {"kernel": kernel, "bound": "hbm", "algorithmic_bytes": int(nbytes), "achieved": round(a, 1),
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4)}
    if ceiling:
        r["frac_of_measured_ceiling"] = round(a / ceiling, 4)
    return r


def _mask_call(tv, parent, ctx_len, B, N, dev):
    mo = dict(anc=torch.empty(B, N, tv.anc_words(N), dtype=torch.int64, device=dev),
              depth=torch.empty(B, N, dtype=torch.int32, device=dev),
              pos=torch.empty(B, N, dtype=torch.int32, device=dev),
              status=torch.empty(B, dtype=torch.int32, device=dev), dense_bias=None)
    tv.tree_mask_build(parent, ctx_len, out=mo)
    return mo, (lambda: tv.tree_mask_build(parent, ctx_len, out=mo))


def _attn_call(tv, x, mo, window, dev):
    out = torch.empty_like(x.q)
    n = tv.tree_verify_attn_workspace_size(x.B, x.N, x.Hq, x.Hkv, x.D, x.max_ctx_len, window)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    return lambda: tv.tree_verify_attn(x.q, x.k_node, x.v_node, x.k_cache, x.v_cache, x.block_table,
                                       x.ctx_len, x.max_ctx_len, mo["anc"], mo["pos"], window, x.scale,
                                       out=out, workspace=ws)


def _walk_call(tv, trees, logits, dev):
    B, N = trees.parent.shape
    tok = torch.from_numpy(trees.tokens).to(dev)
    par = torch.from_numpy(trees.parent).to(dev)
    wo = dict(accepted_tokens=torch.empty(B, N + 1, dtype=torch.int32, device=dev),
              accepted_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
              num_accepted=torch.empty(B, dtype=torch.int32, device=dev))
    ws = torch.empty(tv.tree_walk_accept_workspace_size(B, N), dtype=torch.uint8, device=dev)
    return lambda: tv.tree_walk_accept(tok, par, logits, out=wo, workspace=ws)


def _summary(name, workload, B, N, calls, timing):
    step = sum(timing[c]["median_ms"] for c, _ in calls)
    return {"workload": workload, "B": B, "N": N, "calls": timing, "step_ms": round(step, 5),
            "nodes_per_s": round(B * N / (step * 1e-3), 1)}


def per_config(step, dev, args, ceiling, only: int = 0) -> dict:
    """Each workload as its own step, timed call by call (see time_calls);
    `only` > 0 times that workload alone (`step` may then be None unless it
    is workload 3, whose inputs are the headline step's)."""
    import tree_verify_attention_amd as tv
    from synth import configs as CF
    from synth import workloads as W
    flush = Flusher(dev, args.flush_mib)
    reps, warm = args.reps, args.rep_warmup
    res = {}

    def attn_cfg(cid, kv_on_device):
        c = dict(CF.ATTN[cid])
        wins = c.pop("windows")
        vocab = c.pop("vocab")
        x = W.attn_inputs(cid, device=dev, kv_on_device=kv_on_device, vocab=vocab, **c)
        return x, wins, vocab

    # c1: tiny fp32 step (launch-bound)
    if only in (0, 1):
        x, wins, vocab = attn_cfg(1, False)
        par = torch.from_numpy(x.trees.parent).to(dev)
        mo, mask = _mask_call(tv, par, x.ctx_len, x.B, x.N, dev)
        logits = W.walk_inputs(1, x.trees, vocab, torch.float32, device=dev).logits
        calls = [("mask", mask), ("attn", _attn_call(tv, x, mo, 0, dev)), ("walk", _walk_call(tv, x.trees, logits, dev))]
        t = time_calls(calls, reps, warm, flush)
        r = _summary("c1", "B=1, N=16 random-parent tree, Hq=8, Hkv=2, D=64, ctx 512, fp32; logits [1,17,1000] fp32",
                     x.B, x.N, calls, t)
        kv = _kv_bytes(x, 0)
        r["roofline"] = {"bound": "launch", "note": f"{kv} B of context K+V and a 68 KB logits row set: the "
                         "calls are launch-latency bound", "attn_achieved_GBps": round(_gbps(kv, t["attn"]["median_ms"]), 1)}
        res["c1"] = r
        del x, logits, calls

    # c2: leaf-sibling batch, HBM-bound
    if only in (0, 2):
        x, wins, vocab = attn_cfg(2, True)
        par = torch.from_numpy(x.trees.parent).to(dev)
        mo, mask = _mask_call(tv, par, x.ctx_len, x.B, x.N, dev)
        calls = [("mask", mask), ("attn", _attn_call(tv, x, mo, 0, dev))]
        t = time_calls(calls, reps, warm, flush)
        r = _summary("c2", "B=8, N=32 leaf-sibling trees, Hq=16, Hkv=8, D=256, ctx 4096, bf16", x.B, x.N, calls, t)
        r["roofline"] = _hbm_roof("tree_verify_attn", _kv_bytes(x, 0), t["attn"]["median_ms"], ceiling)
        res["c2"] = r
        del x, calls
        torch.cuda.empty_cache()

    # c3: the headline step's layers, mask + window layer + global layer
    if only in (0, 3):
        xw, xg = step.layers
        mo, mask = _mask_call(tv, step.parent, step.ctx_len, step.B, step.N, dev)
        calls = [("mask", mask), ("attn_window", _attn_call(tv, xw, mo, xw.window, dev)),
                 ("attn_global", _attn_call(tv, xg, mo, xg.window, dev))]
        t = time_calls(calls, reps, warm, flush)
        r = _summary("c3", "B=32, N=32 spine-first trees, ctx U[1024,32768], Hq=16, Hkv=8, D=256, bf16; "
                     "W=512 layer + global layer", step.B, step.N, calls, t)
        bw, bg = _kv_bytes(xw, xw.window), _kv_bytes(xg, 0)
        tw, tg = t["attn_window"]["median_ms"], t["attn_global"]["median_ms"]
        r["roofline"] = {"pair": _hbm_roof("tree_verify_attn, window + global layer", bw + bg, tw + tg, ceiling),
                         "window": _hbm_roof("tree_verify_attn, W=512", bw, tw, ceiling),
                         "global": _hbm_roof("tree_verify_attn, global", bg, tg, ceiling)}
        res["c3"] = r
        del calls

    # c4: DDTree batch, MFMA-bound attention and a 2.18 GB walk
    if only in (0, 4):
        x, wins, vocab = attn_cfg(4, True)
        par = torch.from_numpy(x.trees.parent).to(dev)
        mo, mask = _mask_call(tv, par, x.ctx_len, x.B, x.N, dev)
        logits = W.walk_inputs(4, x.trees, vocab, torch.bfloat16, device=dev, on_device=True).logits
        calls = [("mask", mask), ("attn", _attn_call(tv, x, mo, 0, dev)), ("walk", _walk_call(tv, x.trees, logits, dev))]
        t = time_calls(calls, reps, warm, flush)
        r = _summary("c4", "B=64, N=64 DDTree trees, Hq=64, Hkv=8, D=128, ctx 32768, bf16; logits [64,65,262144] bf16",
                     x.B, x.N, calls, t)
        fl = _attn_flops(x)
        ta = t["attn"]["median_ms"]
        tfl = fl / (ta * 1e-3) / 1e12
        r["roofline"] = {"attn": {"kernel": "tree_verify_attn (wide-tile)", "bound": "mfma", "algorithmic_flops": fl,
                                  "achieved": round(tfl, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tfl / BF16_MFMA_PEAK_TFLOPS, 4),
                                  "kv_GBps": round(_gbps(_kv_bytes(x, 0), ta), 1)},
                         "walk": _hbm_roof("tree_walk_accept", logits.numel() * logits.element_size(),
                                           t["walk"]["median_ms"], ceiling)}
        res["c4"] = r
        del x, logits, calls
        torch.cuda.empty_cache()

    # c5: GDN tree verify
    if only in (0, 5):
        g = dict(CF.GDN[5])
        gx = W.gdn_inputs(5, device=dev, **g)
        par = torch.from_numpy(gx.trees.parent).to(dev)
        ctx = torch.full((gx.B,), 1, dtype=torch.int32, device=dev)
        mo, mask = _mask_call(tv, par, ctx, gx.B, gx.N, dev)
        gout = torch.empty_like(gx.v)
        calls = [("mask", mask),
                 ("gdn", lambda: tv.tree_gdn_verify(gx.q, gx.k, gx.v, gx.alpha, gx.beta, gx.S0, mo["anc"], out=gout))]
        t = time_calls(calls, reps, warm, flush)
        r = _summary("c5", "B=16, H=16, Dk=Dv=128, N=32 spine-first trees, bf16 q/k/v, fp32 gates and state",
                     gx.B, gx.N, calls, t)
        gbytes = sum(z.numel() * z.element_size() for z in (gx.q, gx.k, gx.v, gx.alpha, gx.beta, gx.S0, gout, mo["anc"]))
        r["roofline"] = _hbm_roof("tree_gdn_verify", gbytes, t["gdn"]["median_ms"], ceiling)
        res["c5"] = r

    res["protocol"] = (f"per call: {warm} untimed then {reps} timed repetitions, each after writing "
                       f"{args.flush_mib} MiB and reading {args.flush_mib // 2} MiB on the same stream "
                       f"(outside the events); median, p10, p90 of the event-timed durations; "
                       f"step_ms = sum of the calls' medians")
    return res


def stream_ceiling(dev) -> dict:
    """The read rate of a plain streaming kernel over 4 GiB (best of a few
    grid sizes, 10 timed passes each)."""
    import ctypes
    lib = _probe_lib()
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = None
    for grid in (1024, 2048, 4096, 8192, 16384):
        call = lambda: lib.tv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), n,
                                                ctypes.c_void_p(sink.data_ptr()), grid, stream)
        for _ in range(2):
            assert call() == 0
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            call()
        z.record()
        torch.cuda.synchronize()
        gb = _gbps(n, a.elapsed_time(z) / 10)
        if best is None or gb > best[0]:
            best = (gb, grid)
    del buf
    return {"GBps": round(best[0], 1), "grid": best[1], "bytes": n, "frac_of_8TBps": round(best[0] / HBM_PEAK_GBS, 4),
            "kernel": "16-byte non-temporal loads, 8 in flight per lane, grid-stride, 256 threads per workgroup"}


def _oracle_sample(step: Step, nseq: int):
    """Host copies of the first nseq sequences of the headline step."""
    b_idx = list(range(nseq))
    host = []
    for x in step.layers:
        per = []
        for b in b_idx:
            ctx = int(x.ctx_len[b])
            pages = x.block_table[b, :(ctx + 15) // 16].long()
            kc = x.k_cache[pages].float().cpu().numpy()   # [pages, Hkv, 16, D], exact
            vc = x.v_cache[pages].float().cpu().numpy()
            table = np.arange(len(pages), dtype=np.int64)
            per.append((ctx, kc, vc, table, x.q[b].double().cpu().numpy(), x.k_node[b].double().cpu().numpy(),
                        x.v_node[b].double().cpu().numpy()))
        host.append((x, per))
    g = step.gdn
    return dict(par=step.trees.parent[b_idx], toks=step.trees.tokens[b_idx],
                ctx=step.ctx_len.cpu().numpy()[b_idx], host=host,
                logits=step.logits[b_idx].double().cpu().numpy(),
                gin=[t[b_idx].double().cpu().numpy() for t in (g.q, g.k, g.v, g.alpha, g.beta, g.S0)])


def _oracle_step(sm) -> float:
    """The oracle over the sample: mask, both attention layers, walk, GDN."""
    from oracle import attn as OA, gdn as OG, mask as OM, walk as OW
    t0 = time.perf_counter()
    m = OM.tree_mask(sm["par"], sm["ctx"])
    for x, per in sm["host"]:
        for i, (ctx, kc, vc, table, q, kn, vn) in enumerate(per):
            OA.tree_attn(q[None], kn[None], vn[None], kc, vc, table[None], np.array([ctx]),
                         m["vis"][i:i + 1], m["pos"][i:i + 1], x.window, x.scale)
    OW.tree_walk(sm["toks"], sm["par"], sm["logits"])
    OG.gdn_tree(*sm["gin"], sm["par"])
    return time.perf_counter() - t0


def cpu_baseline(step: Step, nseq: int, nseq_1t: int) -> dict:
    """The oracle (unchanged) on the first sequences of the headline step, on
    all host cores and on one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    host_cores = len(os.sched_getaffinity(0))
    sm = _oracle_sample(step, nseq)
    dt = _oracle_step(sm)
    what = (f"sequences of the headline step ({step.N} nodes each; mask, window and global attention, "
            f"walk over 262144-entry rows, GDN)")
    res = dict(value=round(nseq * step.N / dt, 2), unit="nodes/s", cores=int(threads), kind="oracle",
               sample=f"first {nseq} of {step.B} {what}: {dt:.1f} s on {threads} BLAS threads "
                      f"({host_cores} host cores)")
    if threadpool_limits is not None and 0 < nseq_1t <= nseq:
        n1 = nseq_1t
        sm1 = dict(par=sm["par"][:n1], toks=sm["toks"][:n1], ctx=sm["ctx"][:n1], logits=sm["logits"][:n1],
                   host=[(x, per[:n1]) for x, per in sm["host"]], gin=[t[:n1] for t in sm["gin"]])
        with threadpool_limits(limits=1):
            dt1 = _oracle_step(sm1)
        res["single_thread"] = dict(value=round(nseq_1t * step.N / dt1, 2), unit="nodes/s", cores=1,
                                    sample=f"first {nseq_1t} of {step.B} {what}: {dt1:.1f} s on one thread")
    return res


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


def gdn_only(args, dev) -> dict:
    """tree_gdn_verify alone, inputs resident in HBM, on the verify-cost
    curve's GDN shape with `args.gdn_only` nodes: K warm calls timed with
    events on the current stream."""
    import tree_verify_attention_amd as tv
    from synth import workloads as W
    B, N = 32, args.gdn_only
    trees = W.make_trees(3, "spine_first", B, N, 1000, max_depth=min(8, N), tag=1000 + N)
    g = W.gdn_inputs(3, B=B, N=N, H=16, Dk=128, Dv=128, tree="spine_first", dtype=torch.bfloat16,
                     trees=trees, device=dev)
    m = tv.tree_mask_build(torch.from_numpy(trees.parent).to(dev), torch.full((B,), 1, dtype=torch.int32,
                                                                            device=dev))
    out = torch.empty_like(g.v)
    call = lambda: tv.tree_gdn_verify(g.q, g.k, g.v, g.alpha, g.beta, g.S0, m["anc"], out=out)
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
    nbytes = sum(t.numel() * t.element_size() for t in (g.q, g.k, g.v, g.alpha, g.beta, g.S0, out, m["anc"]))
    return {"gdn_only_nodes": N, "B": B, "H": 16, "Dk": 128, "Dv": 128, "steps": args.steps,
            "warmup": args.warmup, "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def copy_probe(mib: int, dev) -> int:
    """Three plain device copies of `mib` MiB: the reference for scaling the
    HBM byte counters of a profiled run.  Returns the bytes per copy."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return n


def tree_only(args, dev) -> dict:
    """Draft-tree construction alone (tree_draft_topk, then tree_build with
    w = 1 and 8), on the DDTree workload's shape, inputs resident in HBM."""
    import types
    import tree_verify_attention_amd as tv
    tv.load()
    out = {"tree_only": True, **tree_construction(types.SimpleNamespace(tv=tv), dev, args.steps, args.flush_mib)}
    if args.copy_probe_mib > 0:
        out["copy_probe_bytes"] = copy_probe(args.copy_probe_mib, dev)
    return out


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
    if args.gdn_only:
        print(json.dumps(gdn_only(args, dev)), flush=True)
        return
    if args.tree_only:
        print(json.dumps(tree_only(args, dev)), flush=True)
        return
    if args.config:
        step = Step(dev) if args.config == 3 else None
        res = per_config(step, dev, args, None, only=args.config)
        print(json.dumps({"config_only": args.config, **res}), flush=True)
        return
    log("building the headline step's inputs")
    step = Step(dev)
    torch.cuda.synchronize()
    log("timing the headline step")
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
    log("streaming-read ceiling")
    ceiling = stream_ceiling(dev)
    out["stream_ceiling"] = ceiling
    out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceiling["GBps"], 4)
    if not args.no_configs:
        log("per-workload steps c1..c5")
        out["configs"] = per_config(step, dev, args, ceiling["GBps"])
    log("commits, cost curve, tree construction")
    out["next_rows"] = next_rows(step, dev, args.steps)
    if not args.no_curve:
        out["next_rows"]["cost_curve"] = cost_curve(step, dev, min(args.steps, 20))
        out["next_rows"]["tree_construction"] = tree_construction(step, dev, min(args.steps, 20), args.flush_mib)
    if args.copy_probe_mib > 0:
        out["copy_probe_bytes"] = copy_probe(args.copy_probe_mib, dev)
    if not args.no_cpu_baseline:
        log("oracle on the host")
        out["cpu_baseline"] = cpu_baseline(step, args.cpu_sample_seqs, args.cpu_1t_seqs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
