"""The commits after the walk on the GPU against the oracle: the GDN state
advanced over the accepted nodes (fp32 state; max |gpu - ref| / RMS(ref)
<= 1e-4, the fp32 bound, since every input is exact in the oracle's fp64)
and the accepted path's keys and values in the paged cache (bit-exact)."""
import numpy as np
import pytest
import torch

from helpers import np64, rel_err, say
from oracle import gdn as OG
from oracle import kvcommit as OK
from synth import configs as CF
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_STATE = 1e-4


def _gdn(config, **kw):
    x = W.gdn_inputs(config, device=DEV, **kw)
    acc, na = W.accepted_paths(config, x.trees.parent)
    return x, acc, na


def _gdn_check(lib, x, acc, na, tag, in_place=False):
    say(f"gdn commit {tag} B={x.B} N={x.N} H={x.H} dtype={x.k.dtype} accepted={na.tolist()}")
    acc_t = torch.from_numpy(acc).to(DEV)
    na_t = torch.from_numpy(na).to(DEV)
    S0_host = np64(x.S0)
    if in_place:
        S = x.S0.clone()
        lib.tree_gdn_commit(x.k, x.v, x.alpha, x.beta, S, acc_t, na_t, out=S)
    else:
        S = lib.tree_gdn_commit(x.k, x.v, x.alpha, x.beta, x.S0, acc_t, na_t)
    torch.cuda.synchronize()
    ref = OG.gdn_commit(np64(x.k), np64(x.v), np64(x.alpha), np64(x.beta), S0_host, acc, na)
    err = rel_err(np64(S), ref)
    say(f"   err={err:.3e}")
    assert err <= TOL_STATE, err
    got = S.cpu().numpy()
    for b in range(x.B):          # no accepted node: the state is S0 bit for bit
        if na[b] == 0:
            assert np.array_equal(got[b], x.S0[b].cpu().numpy())
    return S



@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_commit_c5_shapes(lib, dtype):
    c = dict(CF.GDN[5])
    c["dtype"] = dtype
    x, acc, na = _gdn(5, **c)
    _gdn_check(lib, x, acc, na, "c5")


def test_gdn_commit_in_place(lib):
    c = dict(CF.GDN[5])
    c.update(B=4)
    x, acc, na = _gdn(5, **c)
    _gdn_check(lib, x, acc, na, "in place", in_place=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N", [64, 128])
def test_gdn_commit_deep_chain_strong_state(lib, dtype, N):
    """A chain of N nodes fully accepted (more than one staged chunk at 128),
    gates down to 0.05, S0 ~ N(0, 1)."""
    x, _, _ = _gdn(52, B=3, N=N, H=4, Dk=128, Dv=128, tree="chain", dtype=dtype, s0_std=1.0)
    g = torch.Generator().manual_seed(5)
    x.alpha.copy_(torch.rand(x.alpha.shape, generator=g).mul(0.95).add(0.05).to(DEV))
    acc = np.tile(np.arange(N, dtype=np.int32), (3, 1))
    na = np.array([N, 1, N // 2 + 1], dtype=np.int32)
    _gdn_check(lib, x, acc, na, f"deep chain N={N}")


def test_gdn_commit_matches_verify_output(lib):
    """The committed state reproduces the verify pass's output at the last
    accepted node: S^T q_t = o_t (two entry points against each other)."""
    c = dict(CF.GDN[5])
    c.update(B=6, dtype=torch.float32)
    x, acc, na = _gdn(53, **c)
    parent = torch.from_numpy(x.trees.parent).to(DEV)
    m = lib.tree_mask_build(parent, torch.full((x.B,), 50, dtype=torch.int32, device=DEV))
    o = lib.tree_gdn_verify(x.q, x.k, x.v, x.alpha, x.beta, x.S0, m["anc"])
    S = lib.tree_gdn_commit(x.k, x.v, x.alpha, x.beta, x.S0, torch.from_numpy(acc).to(DEV),
                            torch.from_numpy(na).to(DEV))
    torch.cuda.synchronize()
    for b in range(x.B):
        if na[b] == 0:
            continue
        t = int(acc[b, na[b] - 1])
        lhs = np.einsum("hkv,hk->hv", np64(S[b]), np64(x.q[b, t]))
        ref = np64(o[b, t])
        assert rel_err(lhs, ref) <= 1e-4


# ---------------------------------------------------------------- KV commit

def _kv_case(config, B, N, Hkv, D, dtype, ctx, extra_pages=8):
    x = W.attn_inputs(config, B=B, N=N, Hq=Hkv, Hkv=Hkv, D=D, ctx_lo=0, ctx_hi=0, tree="random_parent",
                      dtype=dtype, device=DEV, ctx_len=np.asarray(ctx, dtype=np.int32))
    # a table and pool with room for ctx + N positions per sequence
    need = [(c + N + 15) // 16 for c in ctx]
    pool = sum(need) + extra_pages
    perm = np.random.default_rng(config).permutation(pool).astype(np.int32)
    table = np.full((B, max(need)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    g = torch.Generator(device=DEV).manual_seed(config)
    kc = torch.randn(pool, Hkv, 16, D, generator=g, device=DEV).to(dtype)
    vc = torch.randn(pool, Hkv, 16, D, generator=g, device=DEV).to(dtype)
    acc, na = W.accepted_paths(config, x.trees.parent)
    return x, table, kc, vc, acc, na


def _kv_check(lib, x, table, kc, vc, acc, na, ctx, tag):
    say(f"kv commit {tag} B={x.B} N={x.N} Hkv={x.Hkv} D={x.D} dtype={x.k_node.dtype} ctx={list(ctx)} "
        f"accepted={na.tolist()}")
    ref_k, ref_v = OK.kv_commit(kc.cpu().float().numpy(), vc.cpu().float().numpy(),
                                x.k_node.cpu().float().numpy(), x.v_node.cpu().float().numpy(),
                                acc, na, np.asarray(ctx), table)
    lib.tree_kv_commit(x.k_node, x.v_node, torch.from_numpy(acc).to(DEV), torch.from_numpy(na).to(DEV),
                       torch.as_tensor(np.asarray(ctx, dtype=np.int32), device=DEV),
                       torch.from_numpy(table).to(DEV), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().float().numpy(), ref_k)
    assert np.array_equal(vc.cpu().float().numpy(), ref_v)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 256), (torch.bfloat16, 128), (torch.float32, 64)])
def test_kv_commit(lib, dtype, D):
    ctx = [0, 1, 15, 16, 17, 1000]
    x, table, kc, vc, acc, na = _kv_case(60 + D, B=6, N=32, Hkv=8 if D > 64 else 2, D=D, dtype=dtype, ctx=ctx)
    _kv_check(lib, x, table, kc, vc, acc, na, ctx, "mixed ctx")


def test_kv_commit_skips_pages_outside(lib):
    ctx = [31, 40]
    x, table, kc, vc, acc, na = _kv_case(71, B=2, N=16, Hkv=2, D=64, dtype=torch.float32, ctx=ctx)
    acc[:] = np.arange(16)
    na[:] = 16
    table[0, 1] = kc.shape[0] + 5        # positions 16..31 of sequence 0: outside the pool
    table[1, 2] = -7
    _kv_check(lib, x, table, kc, vc, acc, na, ctx, "pages outside")


def test_kv_commit_128_node_chain(lib):
    """A 128-node tree whose whole chain is accepted: positions ctx .. ctx + 127
    over nine pages."""
    ctx = [5, 300]
    x, table, kc, vc, acc, na = _kv_case(72, B=2, N=128, Hkv=2, D=128, dtype=torch.bfloat16, ctx=ctx)
    acc[:] = np.arange(128)
    na[:] = [128, 77]
    _kv_check(lib, x, table, kc, vc, acc, na, ctx, "128 nodes")
