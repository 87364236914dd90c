"""Python binding of the MI355X tree-verification library (libtreeverify.so).

Thin ctypes marshalling over the C ABI declared in ``include/tree_verify.h``:
the functions here have the same names as the C entry points, check tensor
devices, dtypes, shapes and contiguity, allocate outputs and workspaces with
torch when the caller does not pass them, and call the library on torch's
current HIP stream.  Every step of the computation runs in the library's
kernels; there is no fallback, and a missing library raises at once.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeverify.so")

TV_OK, TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE, TV_ERR_LAUNCH, TV_ERR_SCRATCH = range(7)
TV_F32, TV_BF16 = 0, 1
TV_TREE_OK, TV_TREE_BAD_PARENT, TV_TREE_BAD_DEPTH, TV_TREE_BAD_CTX = range(4)
MAX_NODES = 128      # mask, attention, walk, KV commit
GDN_MAX_NODES = 128  # the Gated DeltaNet calls


def anc_words(n: int) -> int:
    """64-bit words of one node's ancestor set (node j: bit j % 64 of word j // 64)."""
    return (n + 63) // 64
BLOCK_SIZE = 16

EXPORTS = (
    "tree_mask_build", "tree_verify_attn_workspace_size", "tree_verify_attn",
    "tree_gdn_verify", "tree_walk_accept_workspace_size", "tree_walk_accept",
    "tree_gdn_commit", "tree_kv_commit", "tree_draft_topk", "tree_build", "tv_status_string",
    "tree_walk_accept_noalloc",
)
WALK_NOALLOC_MAX_ROWS = 262144  # B * (N + 1) at most for tree_walk_accept_noalloc

_lib = None


class TVError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: status {code} ({status_string(code)})")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m tree_verify_attention_amd.build")
    lib = ctypes.CDLL(path)
    P, I, S, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.tree_mask_build.argtypes = [P, P, P, I, I, P, P, P, P, P, P]
    lib.tree_mask_build.restype = S
    lib.tree_verify_attn_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.tree_verify_attn_workspace_size.restype = Z
    lib.tree_verify_attn.argtypes = [P, P, P, P, P, P, I, I, P, I, P, P, I, I, I, I, I, I, I, F, S,
                                     S, P, P, Z, P]
    lib.tree_verify_attn.restype = S
    lib.tree_gdn_verify.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, S, S, P, P]
    lib.tree_gdn_verify.restype = S
    lib.tree_walk_accept_workspace_size.argtypes = [I, I]
    lib.tree_walk_accept_workspace_size.restype = Z
    lib.tree_walk_accept.argtypes = [P, P, P, I, I, I, S, P, P, P, P, Z, P]
    lib.tree_walk_accept.restype = S
    lib.tree_walk_accept_noalloc.argtypes = [P, P, P, I, I, I, S, P, P, P, P]
    lib.tree_walk_accept_noalloc.restype = S
    lib.tree_gdn_commit.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, S, P, P]
    lib.tree_gdn_commit.restype = S
    lib.tree_kv_commit.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, S, P, P, P]
    lib.tree_kv_commit.restype = S
    lib.tree_draft_topk.argtypes = [P, I, I, I, I, S, P, P, P]
    lib.tree_draft_topk.restype = S
    lib.tree_build.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P]
    lib.tree_build.restype = S
    lib.tv_status_string.argtypes = [S]
    lib.tv_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().tv_status_string(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, code):
    if code != TV_OK:
        raise TVError(fn, code)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return TV_F32
    if dt == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"unsupported dtype {dt}")


# ---------------------------------------------------------------- mask

def tree_mask_build(parent: torch.Tensor, ctx_len: torch.Tensor, depth_in: Optional[torch.Tensor] = None,
                    dense_bias: bool = False, out: Optional[dict] = None) -> dict:
    """Ancestor words [B, N, anc_words(N)] (int64 tensor holding the uint64 bits), depths, position
    ids, per-sequence status and optionally the N x N additive bias."""
    lib = load()
    dev = parent.device
    B, N = parent.shape
    _need(parent, "parent", torch.int32, dev)
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    if depth_in is not None:
        _need(depth_in, "depth_in", torch.int32, dev, (B, N))
    if out is None:
        out = dict(anc=torch.empty(B, N, anc_words(N), dtype=torch.int64, device=dev),
                   depth=torch.empty(B, N, dtype=torch.int32, device=dev),
                   pos=torch.empty(B, N, dtype=torch.int32, device=dev),
                   status=torch.empty(B, dtype=torch.int32, device=dev),
                   dense_bias=torch.empty(B, N, N, dtype=torch.float32, device=dev) if dense_bias else None)
    code = lib.tree_mask_build(_ptr(parent), _ptr(depth_in), _ptr(ctx_len), B, N, _ptr(out["anc"]),
                               _ptr(out["depth"]), _ptr(out["pos"]), _ptr(out.get("dense_bias")),
                               _ptr(out["status"]), _stream(dev))
    _check("tree_mask_build", code)
    return out


# ---------------------------------------------------------------- attention

def tree_verify_attn_workspace_size(B, N, Hq, Hkv, D, max_ctx_len, window) -> int:
    return int(load().tree_verify_attn_workspace_size(B, N, Hq, Hkv, D, max_ctx_len, window))


def tree_verify_attn(q, k_node, v_node, k_cache, v_cache, block_table, ctx_len, max_ctx_len: int,
                     anc, pos, window: int, scale: float, out=None, workspace=None,
                     out_dtype=None) -> torch.Tensor:
    """Tree-masked attention; returns out [B, N, Hq, D] in out_dtype (default:
    q's dtype; float32 is allowed for bf16 inputs)."""
    lib = load()
    dev = q.device
    B, N, Hq, D = q.shape
    Hkv = k_node.shape[2]
    dt = q.dtype
    _need(q, "q", dt, dev)
    _need(k_node, "k_node", dt, dev, (B, N, Hkv, D))
    _need(v_node, "v_node", dt, dev, (B, N, Hkv, D))
    nb = k_cache.shape[0]
    _need(k_cache, "k_cache", dt, dev, (nb, Hkv, BLOCK_SIZE, D))
    _need(v_cache, "v_cache", dt, dev, (nb, Hkv, BLOCK_SIZE, D))
    _need(block_table, "block_table", torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(anc, "anc", torch.int64, dev, (B, N, anc_words(N)))
    _need(pos, "pos", torch.int32, dev, (B, N))
    odt = out.dtype if out is not None else (out_dtype or dt)
    if out is None:
        out = torch.empty(B, N, Hq, D, dtype=odt, device=dev)
    _need(out, "out", odt, dev, (B, N, Hq, D))
    ws_bytes = tree_verify_attn_workspace_size(B, N, Hq, Hkv, D, max_ctx_len, window)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib.tree_verify_attn(_ptr(q), _ptr(k_node), _ptr(v_node), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_table), block_table.shape[1], nb, _ptr(ctx_len),
                                int(max_ctx_len), _ptr(anc), _ptr(pos), B, N, Hq, Hkv, D, BLOCK_SIZE,
                                int(window), float(scale), _dtype_code(dt), _dtype_code(odt), _ptr(out),
                                _ptr(workspace),
                                ws_have, _stream(dev))
    _check("tree_verify_attn", code)
    return out


# ---------------------------------------------------------------- GDN

def tree_gdn_verify(q, k, v, alpha, beta, S0, anc, out=None, out_dtype=None) -> torch.Tensor:
    """Gated DeltaNet tree outputs [B, N, H, Dv] in out_dtype (default: q's
    dtype; float32 is allowed for bf16 inputs); S0 is only read."""
    lib = load()
    dev = q.device
    B, N, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", dt, dev)
    _need(k, "k", dt, dev, (B, N, H, Dk))
    _need(v, "v", dt, dev, (B, N, H, Dv))
    _need(alpha, "alpha", torch.float32, dev, (B, N, H))
    _need(beta, "beta", torch.float32, dev, (B, N, H))
    _need(S0, "S0", torch.float32, dev, (B, H, Dk, Dv))
    _need(anc, "anc", torch.int64, dev, (B, N, anc_words(N)))
    odt = out.dtype if out is not None else (out_dtype or dt)
    if out is None:
        out = torch.empty(B, N, H, Dv, dtype=odt, device=dev)
    _need(out, "out", odt, dev, (B, N, H, Dv))
    code = lib.tree_gdn_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(anc),
                               B, N, H, Dk, Dv, _dtype_code(dt), _dtype_code(odt), _ptr(out),
                               _stream(dev))
    _check("tree_gdn_verify", code)
    return out


# ---------------------------------------------------------------- walk

def tree_walk_accept_workspace_size(B, N) -> int:
    return int(load().tree_walk_accept_workspace_size(B, N))


def tree_walk_accept(tokens, parent, logits, out=None, workspace=None) -> dict:
    """Greedy tree walk: accepted_tokens [B, N+1], accepted_nodes [B, N],
    num_accepted [B] (int32)."""
    lib = load()
    dev = tokens.device
    B, N = tokens.shape
    V = logits.shape[-1]
    _need(tokens, "tokens", torch.int32, dev)
    _need(parent, "parent", torch.int32, dev, (B, N))
    _need(logits, "logits", logits.dtype, dev, (B, N + 1, V))
    if out is None:
        out = dict(accepted_tokens=torch.empty(B, N + 1, dtype=torch.int32, device=dev),
                   accepted_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
                   num_accepted=torch.empty(B, dtype=torch.int32, device=dev))
    ws_bytes = tree_walk_accept_workspace_size(B, N)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    code = lib.tree_walk_accept(_ptr(tokens), _ptr(parent), _ptr(logits), B, N, V,
                                _dtype_code(logits.dtype), _ptr(out["accepted_tokens"]),
                                _ptr(out["accepted_nodes"]), _ptr(out["num_accepted"]),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(dev))
    _check("tree_walk_accept", code)
    return out


def tree_walk_accept_noalloc(tokens, parent, logits, out=None) -> dict:
    """tree_walk_accept with the library's static scratch instead of a
    workspace (B * (N + 1) <= WALK_NOALLOC_MAX_ROWS); the library allocates
    nothing.  Outputs are allocated here only when `out` is not given."""
    lib = load()
    dev = tokens.device
    B, N = tokens.shape
    V = logits.shape[-1]
    _need(tokens, "tokens", torch.int32, dev)
    _need(parent, "parent", torch.int32, dev, (B, N))
    _need(logits, "logits", logits.dtype, dev, (B, N + 1, V))
    if out is None:
        out = dict(accepted_tokens=torch.empty(B, N + 1, dtype=torch.int32, device=dev),
                   accepted_nodes=torch.empty(B, N, dtype=torch.int32, device=dev),
                   num_accepted=torch.empty(B, dtype=torch.int32, device=dev))
    code = lib.tree_walk_accept_noalloc(_ptr(tokens), _ptr(parent), _ptr(logits), B, N, V,
                                        _dtype_code(logits.dtype), _ptr(out["accepted_tokens"]),
                                        _ptr(out["accepted_nodes"]), _ptr(out["num_accepted"]),
                                        _stream(dev))
    _check("tree_walk_accept_noalloc", code)
    return out


# ---------------------------------------------------------------- commits

def tree_gdn_commit(k, v, alpha, beta, S0, accepted_nodes, num_accepted, out=None) -> torch.Tensor:
    """The committed GDN state [B, H, Dk, Dv] (float32) after the walk; out
    may be S0 itself (in place)."""
    lib = load()
    dev = k.device
    B, N, H, Dk = k.shape
    Dv = v.shape[-1]
    dt = k.dtype
    _need(k, "k", dt, dev)
    _need(v, "v", dt, dev, (B, N, H, Dv))
    _need(alpha, "alpha", torch.float32, dev, (B, N, H))
    _need(beta, "beta", torch.float32, dev, (B, N, H))
    _need(S0, "S0", torch.float32, dev, (B, H, Dk, Dv))
    _need(accepted_nodes, "accepted_nodes", torch.int32, dev, (B, N))
    _need(num_accepted, "num_accepted", torch.int32, dev, (B,))
    if out is None:
        out = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, (B, H, Dk, Dv))
    code = lib.tree_gdn_commit(_ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                               _ptr(accepted_nodes), _ptr(num_accepted), B, N, H, Dk, Dv,
                               _dtype_code(dt), _ptr(out), _stream(dev))
    _check("tree_gdn_commit", code)
    return out


def tree_kv_commit(k_node, v_node, accepted_nodes, num_accepted, ctx_len, block_table, k_cache,
                   v_cache) -> None:
    """Copy the accepted nodes' key/value rows into positions ctx_len + s of
    the paged caches (in place)."""
    lib = load()
    dev = k_node.device
    B, N, Hkv, D = k_node.shape
    dt = k_node.dtype
    _need(k_node, "k_node", dt, dev)
    _need(v_node, "v_node", dt, dev, (B, N, Hkv, D))
    _need(accepted_nodes, "accepted_nodes", torch.int32, dev, (B, N))
    _need(num_accepted, "num_accepted", torch.int32, dev, (B,))
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(block_table, "block_table", torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    nb = k_cache.shape[0]
    _need(k_cache, "k_cache", dt, dev, (nb, Hkv, BLOCK_SIZE, D))
    _need(v_cache, "v_cache", dt, dev, (nb, Hkv, BLOCK_SIZE, D))
    code = lib.tree_kv_commit(_ptr(k_node), _ptr(v_node), _ptr(accepted_nodes), _ptr(num_accepted),
                              _ptr(ctx_len), _ptr(block_table), block_table.shape[1], nb, B, N, Hkv,
                              D, BLOCK_SIZE, _dtype_code(dt), _ptr(k_cache), _ptr(v_cache),
                              _stream(dev))
    _check("tree_kv_commit", code)


# ---------------------------------------------------------------- tree construction

TREE_MAX_TOPK = 16
TREE_MAX_DEPTH = 16


def tree_draft_topk(logits: torch.Tensor, K: int, out: Optional[dict] = None) -> dict:
    """Per (sequence, depth) the K largest draft logits' tokens (ties to the
    lower id) and their log-softmax values: logits [B, L, V] bf16 or fp32 ->
    cand_tokens int32 [B, L, K], cand_logprob float32 [B, L, K]."""
    lib = load()
    dev = logits.device
    B, L, V = logits.shape
    _need(logits, "logits", logits.dtype, dev, (B, L, V))
    if out is None:
        out = dict(cand_tokens=torch.empty(B, L, K, dtype=torch.int32, device=dev),
                   cand_logprob=torch.empty(B, L, K, dtype=torch.float32, device=dev))
    code = lib.tree_draft_topk(_ptr(logits), B, L, V, int(K), _dtype_code(logits.dtype),
                               _ptr(out["cand_tokens"]), _ptr(out["cand_logprob"]), _stream(dev))
    _check("tree_draft_topk", code)
    return out


def tree_build(cand_tokens: torch.Tensor, cand_logprob: torch.Tensor, N: int, w: int = 1,
               out: Optional[dict] = None, with_score: bool = True) -> dict:
    """Best-first growth of the draft tree (budget N, w candidates per round):
    tokens, parent, depth int32 [B, N], score float32 [B, N] (optional),
    num_nodes int32 [B], in the layout tree_mask_build takes."""
    lib = load()
    dev = cand_tokens.device
    B, L, K = cand_tokens.shape
    _need(cand_tokens, "cand_tokens", torch.int32, dev, (B, L, K))
    _need(cand_logprob, "cand_logprob", torch.float32, dev, (B, L, K))
    if out is None:
        out = dict(tokens=torch.empty(B, N, dtype=torch.int32, device=dev),
                   parent=torch.empty(B, N, dtype=torch.int32, device=dev),
                   depth=torch.empty(B, N, dtype=torch.int32, device=dev),
                   score=torch.empty(B, N, dtype=torch.float32, device=dev) if with_score else None,
                   num_nodes=torch.empty(B, dtype=torch.int32, device=dev))
    code = lib.tree_build(_ptr(cand_tokens), _ptr(cand_logprob), B, L, K, int(N), int(w),
                          _ptr(out["tokens"]), _ptr(out["parent"]), _ptr(out["depth"]),
                          _ptr(out.get("score")), _ptr(out["num_nodes"]), _stream(dev))
    _check("tree_build", code)
    return out
