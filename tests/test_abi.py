"""The C-ABI library loads, exports every function the header declares, and
rejects bad arguments on the host before launching anything (no GPU needed:
every call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

import tree_verify_attention_amd as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_verify.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tv.LIB_PATH):
        pytest.fail("libtreeverify.so is not built (run python -m tree_verify_attention_amd.build)")
    return tv.load()


def test_header_lists_the_entry_points():
    fns = header_functions()
    assert fns == sorted(tv.EXPORTS), fns


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(7):
        assert tv.status_string(code)
    assert tv.status_string(99) == "unknown status"


def test_mask_validation(lib):
    f = lib.tree_mask_build
    assert f(None, None, FAKE, 1, 4, FAKE, FAKE, FAKE, None, FAKE, None) == tv.TV_ERR_NULL
    assert f(FAKE, None, FAKE, 1, 4, None, FAKE, FAKE, None, FAKE, None) == tv.TV_ERR_NULL
    assert f(FAKE, None, FAKE, 0, 4, FAKE, FAKE, FAKE, None, FAKE, None) == tv.TV_ERR_SHAPE
    assert f(FAKE, None, FAKE, 1, 0, FAKE, FAKE, FAKE, None, FAKE, None) == tv.TV_ERR_SHAPE
    assert f(FAKE, None, FAKE, 1, 129, FAKE, FAKE, FAKE, None, FAKE, None) == tv.TV_ERR_UNSUPPORTED


def _attn(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, maxb=256, nblk=100, ctx=FAKE,
             maxctx=4096, anc=FAKE, pos=FAKE, B=2, N=32, Hq=16, Hkv=8, D=256, bs=16, W=0,
             scale=0.0625, dt=tv.TV_BF16, odt=tv.TV_BF16, out=FAKE, ws=None, wsb=0)
    a.update(kw)
    return lib.tree_verify_attn(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["maxb"],
                                a["nblk"], a["ctx"], a["maxctx"], a["anc"], a["pos"], a["B"], a["N"],
                                a["Hq"], a["Hkv"], a["D"], a["bs"], a["W"], a["scale"], a["dt"],
                                a["odt"], a["out"], a["ws"], a["wsb"], None)


def test_attn_validation(lib):
    assert _attn(lib, q=None) == tv.TV_ERR_NULL
    assert _attn(lib, out=None) == tv.TV_ERR_NULL
    assert _attn(lib, kc=None) == tv.TV_ERR_NULL
    assert _attn(lib, B=0) == tv.TV_ERR_SHAPE
    assert _attn(lib, Hq=12, Hkv=8) == tv.TV_ERR_SHAPE
    assert _attn(lib, maxctx=4097) == tv.TV_ERR_SHAPE          # beyond 16 * max_blocks
    assert _attn(lib, nblk=0) == tv.TV_ERR_SHAPE
    assert _attn(lib, N=129) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, D=96) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, scale=0.0) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, scale=-0.5) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, scale=float("inf")) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, scale=float("nan")) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, bs=32) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, dt=7) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, dt=tv.TV_F32, odt=tv.TV_BF16) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, odt=9) == tv.TV_ERR_UNSUPPORTED
    assert _attn(lib, Hq=512, Hkv=1, N=64) == tv.TV_ERR_UNSUPPORTED   # 32768 rows per kv head
    # a split plan that needs partials and no workspace
    need = lib.tree_verify_attn_workspace_size(2, 32, 16, 8, 256, 4096, 0)
    assert need > 0
    assert _attn(lib) == tv.TV_ERR_WORKSPACE
    assert _attn(lib, ws=FAKE, wsb=need - 1) == tv.TV_ERR_WORKSPACE


def test_attn_workspace_sizes(lib):
    ws = lib.tree_verify_attn_workspace_size
    assert ws(0, 32, 16, 8, 256, 4096, 0) == 0
    assert ws(1, 32, 12, 8, 256, 4096, 0) == 0        # Hq % Hkv != 0
    # a window shorter than one split needs no partials
    assert ws(32, 32, 16, 8, 256, 32768, 512) == 0
    # global layer: fp32 partials (D values + max + sum) of 64 rows per slot,
    # at least one slot per (sequence, kv head)
    big = ws(32, 32, 16, 8, 256, 32768, 0)
    slot = 64 * (256 * 4 + 8)
    assert big > 0 and big % slot == 0 and big // slot >= 32 * 8


def test_gdn_validation(lib):
    f = lib.tree_gdn_verify
    args = [FAKE] * 7 + [4, 32, 16, 128, 128, tv.TV_BF16, tv.TV_F32, FAKE, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == tv.TV_ERR_NULL
    bad = list(args); bad[8] = 0
    assert f(*bad) == tv.TV_ERR_SHAPE
    bad = list(args); bad[10] = 64
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(args); bad[8] = 129
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(args); bad[12] = 3
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(args); bad[12] = tv.TV_F32; bad[13] = tv.TV_BF16
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    # q, k, v, S0 and out must be 16-byte aligned
    for i in (0, 1, 2, 5, 14):
        bad = list(args); bad[i] = ctypes.c_void_p(0x1008)
        assert f(*bad) == tv.TV_ERR_UNSUPPORTED, i


def test_walk_validation(lib):
    f = lib.tree_walk_accept
    need = lib.tree_walk_accept_workspace_size(4, 32)
    assert need == 4 * 33 * 4
    base = [FAKE, FAKE, FAKE, 4, 32, 1000, tv.TV_F32, FAKE, FAKE, FAKE, FAKE, need, None]
    bad = list(base); bad[2] = None
    assert f(*bad) == tv.TV_ERR_NULL
    bad = list(base); bad[5] = 0
    assert f(*bad) == tv.TV_ERR_SHAPE
    bad = list(base); bad[4] = 129
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(base); bad[6] = 5
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(base); bad[11] = need - 1
    assert f(*bad) == tv.TV_ERR_WORKSPACE
    bad = list(base); bad[10] = None
    assert f(*bad) == tv.TV_ERR_WORKSPACE


def test_walk_noalloc_validation(lib):
    """The allocation-free walk checks its arguments like tree_walk_accept and
    rejects inputs larger than its static scratch before any HIP call."""
    f = lib.tree_walk_accept_noalloc
    base = [FAKE, FAKE, FAKE, 4, 32, 1000, tv.TV_F32, FAKE, FAKE, FAKE, None]
    bad = list(base); bad[0] = None
    assert f(*bad) == tv.TV_ERR_NULL
    bad = list(base); bad[9] = None
    assert f(*bad) == tv.TV_ERR_NULL
    bad = list(base); bad[3] = 0
    assert f(*bad) == tv.TV_ERR_SHAPE
    bad = list(base); bad[4] = 129
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    bad = list(base); bad[6] = 5
    assert f(*bad) == tv.TV_ERR_UNSUPPORTED
    # B * (N + 1) one past the scratch's rows, and far past it
    bad = list(base); bad[3] = tv.WALK_NOALLOC_MAX_ROWS // 33 + 1; bad[4] = 32
    assert bad[3] * 33 > tv.WALK_NOALLOC_MAX_ROWS
    assert f(*bad) == tv.TV_ERR_SCRATCH
    bad = list(base); bad[3] = 1 << 30; bad[4] = 128
    assert f(*bad) == tv.TV_ERR_SCRATCH
    assert tv.status_string(tv.TV_ERR_SCRATCH) != "unknown status"


def test_gdn_commit_validation(lib):
    f = lib.tree_gdn_commit
    args = [FAKE] * 7 + [4, 32, 16, 128, 128, tv.TV_BF16, FAKE, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == tv.TV_ERR_NULL
    assert call(a6=None) == tv.TV_ERR_NULL          # num_accepted
    assert call(a13=None) == tv.TV_ERR_NULL         # S_out
    assert call(a7=0) == tv.TV_ERR_SHAPE
    assert call(a8=129) == tv.TV_ERR_UNSUPPORTED
    assert call(a10=64) == tv.TV_ERR_UNSUPPORTED     # Dk
    assert call(a12=5) == tv.TV_ERR_UNSUPPORTED      # dtype
    assert call(a4=ctypes.c_void_p(0x1004)) == tv.TV_ERR_UNSUPPORTED   # S0 not 16-byte aligned


def test_kv_commit_validation(lib):
    f = lib.tree_kv_commit
    args = [FAKE] * 6 + [64, 100, 4, 32, 8, 256, 16, tv.TV_BF16, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=None) == tv.TV_ERR_NULL
    assert call(a15=None) == tv.TV_ERR_NULL         # v_cache
    assert call(a8=0) == tv.TV_ERR_SHAPE
    assert call(a7=0) == tv.TV_ERR_SHAPE            # empty pool
    assert call(a11=96) == tv.TV_ERR_UNSUPPORTED     # D
    assert call(a12=32) == tv.TV_ERR_UNSUPPORTED     # block size
    assert call(a9=129) == tv.TV_ERR_UNSUPPORTED
    assert call(a0=ctypes.c_void_p(0x1008)) == tv.TV_ERR_UNSUPPORTED   # not 16-byte aligned


def test_tree_construction_validation(lib):
    f = lib.tree_draft_topk
    assert f(None, 2, 8, 1000, 8, tv.TV_BF16, FAKE, FAKE, None) == tv.TV_ERR_NULL
    assert f(FAKE, 0, 8, 1000, 8, tv.TV_BF16, FAKE, FAKE, None) == tv.TV_ERR_SHAPE
    assert f(FAKE, 2, 17, 1000, 8, tv.TV_BF16, FAKE, FAKE, None) == tv.TV_ERR_UNSUPPORTED   # depth
    assert f(FAKE, 2, 8, 1000, 17, tv.TV_BF16, FAKE, FAKE, None) == tv.TV_ERR_UNSUPPORTED   # top-k
    assert f(FAKE, 2, 8, 4, 8, tv.TV_BF16, FAKE, FAKE, None) == tv.TV_ERR_UNSUPPORTED       # K > V
    assert f(FAKE, 2, 8, 1000, 8, 9, FAKE, FAKE, None) == tv.TV_ERR_UNSUPPORTED             # dtype
    g = lib.tree_build
    args = [FAKE, FAKE, 4, 8, 8, 64, 1, FAKE, FAKE, FAKE, None, FAKE, None]
    bad = list(args); bad[0] = None
    assert g(*bad) == tv.TV_ERR_NULL
    bad = list(args); bad[11] = None
    assert g(*bad) == tv.TV_ERR_NULL                  # num_nodes
    bad = list(args); bad[6] = 0
    assert g(*bad) == tv.TV_ERR_SHAPE                 # w
    bad = list(args); bad[5] = 129
    assert g(*bad) == tv.TV_ERR_UNSUPPORTED           # N
    bad = list(args); bad[4] = 17
    assert g(*bad) == tv.TV_ERR_UNSUPPORTED           # K
    bad = list(args); bad[3] = 17
    assert g(*bad) == tv.TV_ERR_UNSUPPORTED           # L
