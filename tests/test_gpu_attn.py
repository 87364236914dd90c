"""tree_verify_attn on the GPU against the oracle, within the stated
tolerance (max |gpu - ref| / RMS(ref): 2e-2 for bf16, 1e-4 for fp32)."""
import numpy as np
import pytest
import torch

from helpers import np64, rel_err, say, tol_for
from oracle import attn as OA
from oracle import mask as OM
from synth import configs as CF
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu_attn(lib, x, window=None, mask=None, out_dtype=None):
    w = x.window if window is None else window
    if mask is None:
        parent = torch.from_numpy(x.trees.parent).to(DEV)
        mask = lib.tree_mask_build(parent, x.ctx_len)
    out = lib.tree_verify_attn(x.q, x.k_node, x.v_node, x.k_cache, x.v_cache, x.block_table,
                               x.ctx_len, x.max_ctx_len, mask["anc"], mask["pos"], w, x.scale,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, mask


def gpu_attn_checked(lib, x, window):
    """fp32 output for the tolerance check; for bf16 inputs also the bf16
    output, which must be exactly the round-to-nearest-even of the fp32 one."""
    out32, mask = gpu_attn(lib, x, window, out_dtype=torch.float32)
    if x.q.dtype == torch.bfloat16:
        out16, _ = gpu_attn(lib, x, window, mask)
        assert out16.dtype == torch.bfloat16
        assert torch.equal(out16, out32.to(torch.bfloat16))
    return out32


def oracle_full(x, window):
    m = OM.tree_mask(x.trees.parent, x.ctx_len.cpu().numpy())
    return OA.tree_attn(np64(x.q), np64(x.k_node), np64(x.v_node), np64(x.k_cache), np64(x.v_cache),
                        x.block_table.cpu().numpy(), x.ctx_len.cpu().numpy(), m["vis"], m["pos"],
                        window, x.scale)


def make(config, device=DEV, **over):
    c = CF.reduced(config, **over)
    win = c.pop("windows")
    c.pop("vocab")
    return W.attn_inputs(config, device=device, **c), win


def check_full(lib, x, window, tag):
    say(f"attn {tag} B={x.B} N={x.N} Hq={x.Hq} Hkv={x.Hkv} D={x.D} W={window} "
        f"ctx={x.ctx_len.cpu().tolist()}")
    out = gpu_attn_checked(lib, x, window)
    ref = oracle_full(x, window)
    err = rel_err(np64(out), ref)
    say(f"   err={err:.3e}")
    assert err <= tol_for(x.q.dtype), err
    return err


def test_c1_full(lib):
    x, wins = make(1)
    check_full(lib, x, wins[0], "c1")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_dims_and_dtypes(lib, dtype, D):
    x, _ = make(1, B=2, N=20, Hq=4, Hkv=2, D=D, ctx_lo=700, ctx_hi=2500, dtype=dtype)
    for w in (0, 300):
        check_full(lib, x, w, f"dims {dtype} D={D}")


def test_c2_reduced(lib):
    x, _ = make(2, B=2, ctx_lo=2000, ctx_hi=3100)
    check_full(lib, x, 0, "c2-reduced")


@pytest.mark.parametrize("window", [512, 0])
def test_c3_reduced(lib, window):
    x, _ = make(3, B=3, ctx_lo=600, ctx_hi=5000)
    check_full(lib, x, window, "c3-reduced")


def test_c4_reduced(lib):
    x, _ = make(4, B=2, ctx_lo=1500, ctx_hi=2100, tree="ddtree")
    check_full(lib, x, 0, "c4-reduced")


@pytest.mark.parametrize("window", [1, 2, 5, 9, 16, 100])
def test_windows(lib, window):
    x, _ = make(3, B=2, N=24, ctx_lo=150, ctx_hi=300, Hq=4, Hkv=2, D=64, tree="random_parent",
                dtype=torch.float32)
    check_full(lib, x, window, "window")


def test_window_one_is_own_value(lib):
    x, _ = make(1, B=2, N=16, ctx_lo=40, ctx_hi=90)
    out, _ = gpu_attn(lib, x, 1)
    G = x.Hq // x.Hkv
    for h in range(x.Hq):
        assert torch.equal(out[:, :, h].cpu(), x.v_node[:, :, h // G].cpu())


@pytest.mark.parametrize("tree,N", [("chain", 64), ("star", 64), ("random_parent", 1),
                                    ("random_parent", 63), ("random_parent", 33)])
def test_tree_shapes(lib, tree, N):
    x, _ = make(1, B=2, N=N, Hq=4, Hkv=1, D=64, ctx_lo=17, ctx_hi=150, tree=tree, dtype=torch.bfloat16)
    check_full(lib, x, 0, f"tree {tree}")
    check_full(lib, x, 20, f"tree {tree}")


def test_short_and_empty_context(lib):
    """ctx 0 (nodes only), 1, 15, 16, 17: ragged page tails."""
    trees = W.make_trees(50, "random_parent", 5, 12, 100)
    x, _ = make(1, B=5, N=12, Hq=4, Hkv=2, D=64, trees=trees,
                ctx_len=np.array([0, 1, 15, 16, 17], dtype=np.int32))
    check_full(lib, x, 0, "short ctx")
    check_full(lib, x, 3, "short ctx")


def test_gqa_group_of_one_and_many(lib):
    for Hq, Hkv in ((8, 8), (16, 1)):
        x, _ = make(1, B=1, N=9, Hq=Hq, Hkv=Hkv, D=128, ctx_lo=300, ctx_hi=300, dtype=torch.bfloat16)
        check_full(lib, x, 0, f"gqa {Hq}/{Hkv}")


def test_deterministic(lib):
    x, _ = make(3, B=2, ctx_lo=3000, ctx_hi=4000)
    a, m = gpu_attn(lib, x, 0)
    b, _ = gpu_attn(lib, x, 0, m)
    assert torch.equal(a, b)


def _unit_check(lib, x, window, units, tag, chunk=8):
    """The whole layer on the GPU in the benchmark's launch configuration,
    then every node and query head of the listed (sequence, kv head) units
    against the oracle, fetching only the pages those units read.  The bar is
    the tolerance over all compared rows together (max |gpu - ref| over their
    RMS); progress is printed per chunk of units."""
    out = gpu_attn_checked(lib, x, window)
    m = OM.tree_mask(x.trees.parent, x.ctx_len.cpu().numpy())
    G = x.Hq // x.Hkv
    max_abs, sq, n = 0.0, 0.0, 0
    for c0 in range(0, len(units), chunk):
        part = units[c0:c0 + chunk]
        for (b, g) in part:
            ctx = int(x.ctx_len[b])
            pages = x.block_table[b, :(ctx + 15) // 16].long()
            kc = x.k_cache[pages, g].reshape(-1, x.D)[:ctx].double().cpu().numpy()
            vc = x.v_cache[pages, g].reshape(-1, x.D)[:ctx].double().cpu().numpy()
            ref = OA.tree_attn_group(np64(x.q[b, :, g * G:(g + 1) * G]), kc, vc, np64(x.k_node[b, :, g]),
                                     np64(x.v_node[b, :, g]), m["vis"][b], m["pos"][b], window, x.scale)
            got = np64(out[b, :, g * G:(g + 1) * G])
            assert np.isfinite(got).all()
            max_abs = max(max_abs, float(np.abs(got - ref).max()))
            sq += float((ref ** 2).sum())
            n += ref.size
        say(f"   {tag}: units {c0 + len(part)}/{len(units)} max|err|/rms so far "
            f"{max_abs / np.sqrt(sq / n):.3e}")
    err = max_abs / np.sqrt(sq / n)
    say(f"   {tag}: err={err:.3e} over {len(units)} units")
    assert err <= tol_for(x.q.dtype), err
    return err


def _all_units(x):
    return [(b, g) for b in range(x.B) for g in range(x.Hkv)]


@pytest.mark.parametrize("window", [512, 0])
def test_c3_full_size_all_outputs(lib, window):
    """The mixed batch at full size (B=32, ctx in [1024, 32768], both layers),
    in the launch configuration the benchmark times: every output element is
    compared with the oracle (stream shares, segment boundaries and partial
    merges included)."""
    x, _ = make(3, kv_on_device=True)
    say(f"attn c3 full W={window} ctx sum={int(x.ctx_len.sum())}")
    _unit_check(lib, x, window, _all_units(x), f"c3 W={window}")


def test_c2_full_size_all_outputs(lib):
    x, _ = make(2, kv_on_device=True)
    say("attn c2 full")
    _unit_check(lib, x, 0, _all_units(x), "c2")


def test_stream_shares_within_the_page_cache(lib):
    """A global layer large enough that two stream workgroups per CU would
    each take more key tiles (about 516 of 32 keys) than the page cache covers
    (1024 pages of 16 keys): the plan grows the grid instead, so no segment
    reads the block table per refill.  The workspace size query reveals the
    grid; sampled units spread over the batch and both ends of the kv heads
    are compared with the oracle (segment boundaries and merges included)."""
    B, N, Hq, Hkv, D, ctx = 32, 16, 16, 8, 64, 33000
    x = W.attn_inputs(3, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, ctx_lo=ctx, ctx_hi=ctx, tree="spine_first",
                      dtype=torch.bfloat16, device=DEV, kv_on_device=True)
    rows = (Hq // Hkv) * N
    units = B * Hkv
    ws = lib.tree_verify_attn_workspace_size(B, N, Hq, Hkv, D, ctx, 0)
    wg = ws // (rows * (D * 4 + 8)) - units + 1
    tiles = units * ((ctx + 31) // 32 + (N + 31) // 32)
    say(f"attn stream cap: {tiles} tiles over {wg} workgroups")
    assert -(-tiles // wg) <= 512
    sample = [(b, g) for b in (0, 7, 13, 20, 31) for g in (0, 3, 7)]
    _unit_check(lib, x, 0, sample, "stream cap")


def test_c4_full_size_all_outputs(lib):
    """The DDTree batch at full size: every output element, i.e. all 64 nodes
    x 8 query heads (both 256-row groups of the wide-tile kernel) of all 512
    (sequence, kv head) units, over every XCD slot of the unit numbering."""
    x, _ = make(4, kv_on_device=True)
    say("attn c4 full")
    _unit_check(lib, x, 0, _all_units(x), "c4", chunk=64)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_wide_query_tiles(lib, D):
    """More than 64 query rows per kv head (G * N = 160): the row tiles of a
    workgroup end inside the tile; ragged contexts from empty to several
    splits; no window, a window inside a stage and one past the context."""
    trees = W.make_trees(51, "random_parent", 6, 40, 100)
    x, _ = make(1, B=6, N=40, Hq=8, Hkv=2, D=D, trees=trees, dtype=torch.bfloat16,
                ctx_len=np.array([0, 1, 17, 63, 700, 5000], dtype=np.int32))
    for w in (0, 37, 6000):
        check_full(lib, x, w, f"wide D={D}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tree,N,G,D", [("chain", 128, 1, 64), ("random_parent", 100, 2, 128),
                                        ("ddtree", 128, 4, 128), ("random_parent", 65, 1, 256)])
def test_trees_past_one_word(lib, dtype, tree, N, G, D):
    """Trees of 65 to 128 nodes: ancestor sets in two words, node keys over
    several tiles (and, for bf16, 64-key stages); windows that cut into the
    node keys of deep chains."""
    trees = W.make_trees(52, tree, 3, N, 4096 if tree == "ddtree" else 100)
    x, _ = make(1, B=3, N=N, Hq=2 * G, Hkv=2, D=D, trees=trees, dtype=dtype,
                ctx_len=np.array([0, 40, 900], dtype=np.int32))
    for w in (0, 20, 70):
        check_full(lib, x, w, f"{tree} N={N} G={G} D={D} {dtype}")


def test_c4_shape_at_128_nodes(lib):
    """The DDTree batch's head shape (G = 8, D = 128) with 128-node trees:
    1024 query rows per kv head."""
    x, _ = make(4, B=2, N=128, ctx_lo=1500, ctx_hi=2100, tree="ddtree")
    check_full(lib, x, 0, "c4-shape N=128")


def _nsplit_host(x, window, rows_per_wg=64, min_split=2048, target_wg=4096, tile=32):
    """Splits the library plans for a split-layout launch, recomputed on the
    host from the documented planning rule (at least 2048 keys per split,
    about 4096 workgroups): used only to assert that a case reaches several
    splits."""
    rows = (x.Hq // x.Hkv) * x.N
    rg = -(-rows // rows_per_wg)
    rng = min(x.max_ctx_len, window) if window > 0 else x.max_ctx_len
    want = max(1, min(-(-target_wg // (x.B * x.Hkv * rg)), max(1, -(-rng // min_split))))
    st = max(tile, -(-(-(-rng // want)) // tile) * tile)
    return -(-rng // st) if rng > 0 else 1


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("window,D", [(2049, 256), (4096, 128), (8192, 256)])
def test_split_layout_several_splits(lib, dtype, window, D):
    """Sliding windows wider than one split (serve-integration spec, "2. Verify:
    tree attention mask": the per-layer window): the split kernel writes fp32
    partials per split, hands the second team's state over in LDS, and the
    merge kernel combines them.  G * N = 64 rows per kv head; contexts up to
    12k, one shorter than the window and one empty."""
    trees = W.make_trees(56, "spine_first", 3, 32, 1000)
    x, _ = make(3, B=3, N=32, Hq=4, Hkv=2, D=D, trees=trees, dtype=dtype,
                ctx_len=np.array([12000, 3000, 0], dtype=np.int32))
    ws = lib.tree_verify_attn_workspace_size(x.B, x.N, x.Hq, x.Hkv, x.D, x.max_ctx_len, window)
    assert ws > 0, "partials in use"
    assert _nsplit_host(x, window) >= 2
    check_full(lib, x, window, f"split W={window} D={D} {dtype}")


def test_split_layout_fp32_many_rows(lib):
    """fp32 with G * N > 64 (two row groups of the split kernel) over contexts
    longer than one split, global and windowed."""
    trees = W.make_trees(57, "random_parent", 3, 20, 1000)
    x, _ = make(1, B=3, N=20, Hq=8, Hkv=2, D=128, trees=trees, dtype=torch.float32,
                ctx_len=np.array([5000, 2100, 17], dtype=np.int32))
    for window in (0, 4500):
        ws = lib.tree_verify_attn_workspace_size(x.B, x.N, x.Hq, x.Hkv, x.D, x.max_ctx_len, window)
        assert ws > 0, "partials in use"
        assert _nsplit_host(x, window) >= 2
        check_full(lib, x, window, f"fp32 rows=80 W={window}")
