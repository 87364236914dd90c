"""Pins for the accepted-path KV commit oracle (positions ctx_len + s of the
accepted nodes, serve-integration spec layout contract): checked through the
attention oracle's own page gather, which is a separate path."""
import numpy as np

from oracle import attn as OA
from oracle import kvcommit as KC


def _case(seed=0, B=3, N=12, Hkv=2, D=8, ctx=(5, 16, 31), nblocks=20, mb=4):
    rng = np.random.default_rng(seed)
    kc = rng.standard_normal((nblocks, Hkv, 16, D)).astype(np.float32)
    vc = rng.standard_normal((nblocks, Hkv, 16, D)).astype(np.float32)
    kn = rng.standard_normal((B, N, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, N, Hkv, D)).astype(np.float32)
    perm = rng.permutation(nblocks)[:B * mb].reshape(B, mb).astype(np.int32)
    acc = np.full((B, N), -1, dtype=np.int32)
    na = np.array([0, 5, 12][:B], dtype=np.int32)
    for b in range(B):
        acc[b, :na[b]] = rng.choice(N, size=na[b], replace=False)
    return kc, vc, kn, vn, acc, na, np.array(ctx, dtype=np.int32), perm


def test_no_accept_leaves_cache():
    kc, vc, kn, vn, acc, na, ctx, bt = _case()
    na[:] = 0
    k2, v2 = KC.kv_commit(kc, vc, kn, vn, acc, na, ctx, bt)
    np.testing.assert_array_equal(k2, kc)
    np.testing.assert_array_equal(v2, vc)


def test_committed_positions_read_back_through_the_page_gather():
    kc, vc, kn, vn, acc, na, ctx, bt = _case()
    k2, v2 = KC.kv_commit(kc, vc, kn, vn, acc, na, ctx, bt)
    for b in range(len(na)):
        for g in range(kc.shape[1]):
            K_old, V_old = OA.context_kv(kc, vc, bt[b], g, int(ctx[b]))
            K_new, V_new = OA.context_kv(k2, v2, bt[b], g, int(ctx[b]) + int(na[b]))
            np.testing.assert_array_equal(K_new[:ctx[b]], K_old)   # the context is untouched
            np.testing.assert_array_equal(V_new[:ctx[b]], V_old)
            for s in range(na[b]):
                np.testing.assert_array_equal(K_new[ctx[b] + s], kn[b, acc[b, s], g])
                np.testing.assert_array_equal(V_new[ctx[b] + s], vn[b, acc[b, s], g])
    # pages no sequence owns are untouched
    owned = set(bt.ravel().tolist())
    for p in range(kc.shape[0]):
        if p not in owned:
            np.testing.assert_array_equal(k2[p], kc[p])


def test_page_outside_the_pool_is_not_written():
    kc, vc, kn, vn, acc, na, ctx, bt = _case()
    bt[2, 1] = kc.shape[0] + 3          # positions 16..31 of sequence 2 point outside
    k2, v2 = KC.kv_commit(kc, vc, kn, vn, acc, na, ctx, bt)
    K_new, _ = OA.context_kv(k2, v2, bt[2], 0, 16)   # pages 0 only
    # sequence 2 has ctx 31: accepted positions 31..42 fall in pages 1 and 2;
    # page 1 (positions 31) is outside the pool, so only positions 32.. land
    assert np.array_equal(k2[bt[2, 2], 0, 0], kn[2, acc[2, 1], 0])
    np.testing.assert_array_equal(K_new, OA.context_kv(kc, vc, bt[2], 0, 16)[0])
