"""CPU-side checks of the C ABI: libvsa.so loads, exports every entry point
that include/vsa.h declares, its host helper matches the oracle, and every
argument error is reported before anything is launched (no GPU needed: each
call below fails validation before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from block_sparse_video_major_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libvsa.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"vsa_permute", "vsa_unpermute", "vsa_pool", "vsa_coarse_topk",
            "vsa_sparse_attn_fwd"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_abi_version_and_status_strings():
    assert L.vsa_abi_version() >> 16 == 3
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.vsa_status_str(code) and L.vsa_status_str(code) != "unknown status"
    assert L.vsa_status_str(42) == "unknown status"


@pytest.mark.parametrize("grid,cube", [((4, 8, 8), (4, 4, 4)), ((16, 32, 64), (4, 4, 4)),
                                       ((2, 4, 6), (2, 2, 2)), ((3, 6, 4), (3, 2, 1)),
                                       ((32, 48, 80), (4, 4, 4))])
def test_host_perm_index_matches_oracle(grid, cube):
    p = L.Problem(1, 1, *grid, *cube, 64)
    got = L.vsa_perm_index(p).numpy()
    assert np.array_equal(got, oracle.perm_index(*grid, *cube))


@pytest.mark.parametrize("grid,cube", [((6, 8, 8), (4, 4, 4)), ((5, 7, 9), (4, 4, 4)),
                                       ((1, 1, 1), (4, 4, 4)), ((3, 5, 2), (2, 2, 2)),
                                       ((21, 30, 52), (4, 4, 4))])
def test_host_perm_index_padded_grid(grid, cube):
    """A grid that does not divide into cubes: Np = ceil-cube count * vol
    positions, -1 at padding, as the oracle's padded layout."""
    p = L.Problem(1, 1, *grid, *cube, 64)
    want = oracle.token_layout(*grid, *cube)
    assert p.padded and p.n_positions == len(want)
    assert p.n_cubes * p.cube_volume == len(want)
    got = L.vsa_perm_index(p).numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("grid,cube", [((16, 32, 64), (4, 4, 4)), ((32, 48, 80), (4, 4, 4)),
                                       ((21, 30, 52), (4, 4, 4)), ((3, 5, 2), (2, 2, 2)), ((4, 4, 4), (4, 4, 4)),
                                       ((2, 9, 3), (1, 1, 1))])
def test_host_hilbert_order_matches_oracle(grid, cube):
    """The library's Hilbert cube table and token order, written in C from
    the same published transform, equal the oracle's."""
    p = L.Problem(1, 1, *grid, *cube, 64, cube_order="hilbert")
    seq = oracle.cube_sequence(*p.cube_grid, "hilbert")
    table = L.vsa_cube_table(p).numpy()
    assert table.tolist() == [(t << 20) | (h << 10) | w for t, h, w in seq]
    assert np.array_equal(L.vsa_perm_index(p).numpy(), oracle.token_layout(*grid, *cube, "hilbert"))
    raster = L.Problem(1, 1, *grid, *cube, 64)
    assert L.vsa_cube_table(raster).tolist() == [(t << 20) | (h << 10) | w
                                                 for t, h, w in oracle.cube_sequence(*p.cube_grid, "raster")]


def test_hilbert_order_needs_its_device_table():
    lib = _raw()
    hp = L.Problem(1, 2, 8, 16, 16, 4, 4, 4, 64, cube_order="hilbert").c_struct()
    assert hp.cube_coords is None
    assert lib.vsa_permute(ctypes.byref(hp), 0, DUMMY, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_fwd(ctypes.byref(hp), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 4, None, None, None,
                                   DUMMY, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_coarse_topk(ctypes.byref(hp), 4, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, None) == \
        L.VSA_ERR_NULL
    # host helpers and size queries do not read the table
    n = ctypes.c_size_t(0)
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(hp), 4, ctypes.byref(n)) == L.VSA_OK
    assert lib.vsa_coarse_bwd_workspace_size(ctypes.byref(hp), ctypes.byref(n)) == L.VSA_OK
    bad = L.Problem(1, 2, 8, 16, 16, 4, 4, 4, 64).c_struct()
    bad.cube_order = 7
    assert lib.vsa_perm_index(ctypes.byref(bad), DUMMY) == L.VSA_ERR_UNSUPPORTED
    wide = L.Problem(1, 1, 4, 4, 4 * 1025, 4, 4, 4, 64, cube_order="hilbert")
    out = np.zeros(wide.n_cubes, np.int32)
    assert lib.vsa_cube_table(ctypes.byref(wide.c_struct()), out.ctypes.data) == L.VSA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        L.Problem(1, 1, 4, 4, 4, cube_order="morton").c_struct()


def test_value_head_size_errors():
    lib = _raw()
    bad = L.Problem(1, 2, 8, 16, 16, 4, 4, 4, 128, head_dim_v=96).c_struct()
    assert lib.vsa_perm_index(ctypes.byref(bad), DUMMY) == L.VSA_ERR_UNSUPPORTED
    hv = ctypes.byref(L.Problem(1, 2, 8, 16, 16, 4, 4, 4, 128, head_dim_v=64).c_struct())
    n = ctypes.c_size_t(0)
    # the backward sizes do not depend on the value head size
    assert lib.vsa_sparse_attn_bwd_workspace_size(hv, 4, ctypes.byref(n)) == L.VSA_OK
    same = ctypes.c_size_t(0)
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(_prob(head_dim=128)), 4, ctypes.byref(same)) == \
        L.VSA_OK and same.value == n.value
    assert lib.vsa_sparse_attn_bwd(hv, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 4, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                   DUMMY, DUMMY, 1, None) == L.VSA_ERR_WORKSPACE
    assert lib.vsa_coarse_bwd_workspace_size(hv, ctypes.byref(n)) == L.VSA_OK
    # the forward validates as usual before any launch
    assert lib.vsa_sparse_attn_fwd(hv, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 0, None, None, None, DUMMY, None,
                                   None) == L.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_fwd(hv, DUMMY, DUMMY, None, DUMMY, DUMMY, 4, None, None, None, DUMMY, None,
                                   None) == L.VSA_ERR_NULL
    p = L.Problem(1, 4, 8, 16, 16, 4, 4, 4, 128, heads_kv=2, head_dim_v=64)
    assert p.v_dim == 64 and p.v_problem().head_dim == 64 and p.v_problem().heads == 2
    assert p.kv_problem().head_dim == 128 and p.kv_problem().head_dim_v == 0


# ----------------------------------------------------------------- errors
DUMMY = 0x1000   # never dereferenced: each call fails validation first


def _raw():
    return L.load()


def _prob(**kw):
    base = dict(batch=1, heads=2, T=8, H=16, W=16, ct=4, ch=4, cw=4, head_dim=64)
    base.update(kw)
    return L.Problem(**base).c_struct()


def _perm(prob, dtype=L.VSA_BF16, src=DUMMY, dst=DUMMY):
    return _raw().vsa_permute(ctypes.byref(prob) if prob is not None else None, dtype, src, dst, None)


def test_permute_errors():
    assert _perm(None) == L.VSA_ERR_NULL
    assert _perm(_prob(ct=0)) == L.VSA_ERR_SHAPE
    assert _perm(_prob(W=0)) == L.VSA_ERR_SHAPE
    assert _perm(_prob(batch=-1)) == L.VSA_ERR_SHAPE
    assert _perm(_prob(head_dim=96)) == L.VSA_ERR_UNSUPPORTED
    assert _perm(_prob(), dtype=7) == L.VSA_ERR_UNSUPPORTED
    assert _perm(_prob(), src=None) == L.VSA_ERR_NULL
    assert _perm(_prob(), dst=None) == L.VSA_ERR_NULL
    assert _raw().vsa_unpermute(ctypes.byref(_prob(ch=-1)), 0, DUMMY, DUMMY, None) == L.VSA_ERR_SHAPE
    assert _raw().vsa_unpermute(ctypes.byref(_prob()), 0, None, DUMMY, None) == L.VSA_ERR_NULL
    assert _perm(_prob(T=1 << 14, H=1 << 14, W=1 << 14, ct=1, ch=1, cw=1)) == L.VSA_ERR_SHAPE


def test_pool_errors():
    lib = _raw()
    assert lib.vsa_pool(ctypes.byref(_prob()), 0, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_pool(ctypes.byref(_prob()), 0, DUMMY, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_pool(ctypes.byref(_prob(cw=0)), 0, DUMMY, DUMMY, None) == L.VSA_ERR_SHAPE
    assert lib.vsa_pool(ctypes.byref(_prob()), 3, DUMMY, DUMMY, None) == L.VSA_ERR_UNSUPPORTED


def test_permute_pool_errors():
    lib = _raw()
    assert lib.vsa_permute_pool(ctypes.byref(_prob()), 0, None, DUMMY, DUMMY, None) == L.VSA_ERR_NULL
    # (x_cube == NULL is the pool on its own, a valid call: not made here)
    assert lib.vsa_permute_pool(ctypes.byref(_prob()), 0, DUMMY, DUMMY, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_pool(ctypes.byref(_prob()), 0, DUMMY, None, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_pool(ctypes.byref(_prob()), 0, None, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_pool(None, 0, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_pool(ctypes.byref(_prob(T=0)), 0, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_SHAPE
    assert lib.vsa_permute_pool(ctypes.byref(_prob()), 2, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_UNSUPPORTED


def test_combine_errors():
    lib = _raw()
    pr = ctypes.byref(_prob())
    assert lib.vsa_combine(None, DUMMY, DUMMY, None, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_combine(pr, None, DUMMY, None, None, DUMMY, None) == L.VSA_ERR_NULL      # no O_f
    assert lib.vsa_combine(pr, DUMMY, DUMMY, None, None, None, None) == L.VSA_ERR_NULL      # no out
    assert lib.vsa_combine(pr, DUMMY, None, DUMMY, None, DUMMY, None) == L.VSA_ERR_NULL     # gate_c without oc
    assert lib.vsa_combine(ctypes.byref(_prob(H=0)), DUMMY, DUMMY, None, None, DUMMY, None) == L.VSA_ERR_SHAPE
    assert lib.vsa_combine(ctypes.byref(_prob(head_dim_v=96)), DUMMY, None, None, None, DUMMY,
                           None) == L.VSA_ERR_UNSUPPORTED


def test_mask_to_lut_errors():
    lib = _raw()
    pr = ctypes.byref(_prob())          # Nc = 32
    assert lib.vsa_mask_to_lut(pr, None, 4, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_mask_to_lut(pr, DUMMY, 4, None, DUMMY, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_mask_to_lut(pr, DUMMY, 4, DUMMY, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_mask_to_lut(pr, DUMMY, 4, DUMMY, DUMMY, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_mask_to_lut(pr, DUMMY, 0, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_TOPK
    assert lib.vsa_mask_to_lut(pr, DUMMY, 33, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_TOPK
    assert lib.vsa_mask_to_lut(ctypes.byref(_prob(heads=0)), DUMMY, 4, DUMMY, DUMMY, DUMMY, None) == L.VSA_ERR_SHAPE


def test_sparse_attn_bwd_workspace_and_errors():
    lib = _raw()
    pr = ctypes.byref(_prob(head_dim=128))     # 8 x 16 x 16 grid, 32 cubes, 2 heads
    n = ctypes.c_size_t(0)
    assert lib.vsa_sparse_attn_bwd_workspace_size(pr, 8, ctypes.byref(n)) == L.VSA_OK
    # per-token records, per-row-block counts, list offsets, list entries (each 256-byte aligned)
    al = lambda x: (x + 255) // 256 * 256
    bh, nc, ntok = 2, 32, 2048
    assert n.value == al(bh * ntok * 8) + al(bh * 2 * nc * 4) + al(bh * (nc + 1) * 4) + al(bh * nc * 8 * 4)
    # a padded 6 x 8 x 8 grid: 8 cubes, per-token records over the 512 padded positions
    pp = ctypes.byref(_prob(T=6, H=8, W=8, head_dim=128))
    assert lib.vsa_sparse_attn_bwd_workspace_size(pp, 4, ctypes.byref(n)) == L.VSA_OK
    assert n.value == al(bh * 512 * 8) + al(bh * 1 * 8 * 4) + al(bh * 9 * 4) + al(bh * 8 * 4 * 4)
    assert lib.vsa_sparse_attn_bwd_workspace_size(pr, 8, None) == L.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_bwd_workspace_size(pr, 0, ctypes.byref(n)) == L.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_bwd_workspace_size(pr, 33, ctypes.byref(n)) == L.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(_prob(ct=2)), 8, ctypes.byref(n)) == \
        L.VSA_ERR_UNSUPPORTED
    big = L.Problem(1, 1, 32, 64, 64, 2, 2, 2, 64)    # vol 8: not handled
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(big.c_struct()), 8, ctypes.byref(n)) == \
        L.VSA_ERR_UNSUPPORTED
    many = L.Problem(1, 1, 64, 64, 144, 4, 4, 4, 64)  # 9216 cubes: above the backward's limit
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(many.c_struct()), 8, ctypes.byref(n)) == \
        L.VSA_ERR_UNSUPPORTED

    def call(q=DUMMY, k=DUMMY, v=DUMMY, lut=DUMMY, valid=DUMMY, maxkv=8, o=DUMMY, lse=DUMMY, do=DUMMY,
             dq=DUMMY, dk=DUMMY, dv=DUMMY, ws=DUMMY, wsb=None, prob=pr):
        return lib.vsa_sparse_attn_bwd(prob, q, k, v, lut, valid, maxkv, o, lse, do, dq, dk, dv, ws,
                                       size if wsb is None else wsb, None)
    assert lib.vsa_sparse_attn_bwd_workspace_size(pr, 8, ctypes.byref(n)) == L.VSA_OK
    size = n.value
    for name in ("q", "k", "v", "lut", "valid", "o", "lse", "do", "dq", "dk", "dv", "ws"):
        assert call(**{name: None}) == L.VSA_ERR_NULL, name
    assert call(wsb=size - 1) == L.VSA_ERR_WORKSPACE
    assert call(maxkv=0) == L.VSA_ERR_TOPK
    assert call(maxkv=33) == L.VSA_ERR_TOPK
    assert call(prob=ctypes.byref(_prob(head_dim=96))) == L.VSA_ERR_UNSUPPORTED
    assert call(prob=None) == L.VSA_ERR_NULL


def test_grouped_heads_must_divide():
    lib = _raw()
    ok = L.Problem(1, 4, 8, 16, 16, 4, 4, 4, 64, heads_kv=2)
    bad = L.Problem(1, 4, 8, 16, 16, 4, 4, 4, 64, heads_kv=3)
    neg = L.Problem(1, 4, 8, 16, 16, 4, 4, 4, 64, heads_kv=-1)
    n = ctypes.c_size_t(0)
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(ok.c_struct()), 4, ctypes.byref(n)) == L.VSA_OK
    for p in (bad, neg):
        assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(p.c_struct()), 4, ctypes.byref(n)) == \
            L.VSA_ERR_SHAPE
        assert lib.vsa_coarse_topk(ctypes.byref(p.c_struct()), 4, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None,
                                   None) == L.VSA_ERR_SHAPE
    assert ok.kv_heads == 2 and ok.kv_problem().heads == 2 and ok.kv_problem().heads_kv == 0


def test_model_layout_entry_points_errors():
    lib = _raw()
    pr = ctypes.byref(_prob())
    assert lib.vsa_permute_bnhd(pr, L.VSA_BF16, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_bnhd(pr, 7, DUMMY, DUMMY, None) == L.VSA_ERR_UNSUPPORTED
    assert lib.vsa_permute_pool_bnhd(pr, L.VSA_BF16, DUMMY, DUMMY, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_permute_pool_bnhd(ctypes.byref(_prob(W=-1)), L.VSA_BF16, DUMMY, DUMMY, DUMMY, None) == \
        L.VSA_ERR_SHAPE
    assert lib.vsa_pool_unpermute_bwd_bnhd(pr, None, None, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_pool_unpermute_bwd_bnhd(pr, DUMMY, None, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_fwd_bnhd(pr, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 0, None, None, None, DUMMY, None,
                                        None) == L.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_fwd_bnhd(pr, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 4, None, DUMMY, None, DUMMY, None,
                                        None) == L.VSA_ERR_NULL


def test_coarse_topk_errors():
    lib = _raw()
    pr = ctypes.byref(_prob())          # Nc = 8*16*16/64 = 32

    def call(k=8, qc=DUMMY, kc=DUMMY, vc=DUMMY, lut=DUMMY, valid=DUMMY, oc=DUMMY, prob=pr):
        return lib.vsa_coarse_topk(prob, k, qc, kc, vc, lut, valid, oc, None)

    assert call(k=0) == L.VSA_ERR_TOPK
    assert call(k=33) == L.VSA_ERR_TOPK
    assert call(qc=None) == L.VSA_ERR_NULL
    assert call(kc=None) == L.VSA_ERR_NULL
    assert call(lut=None) == L.VSA_ERR_NULL
    assert call(valid=None) == L.VSA_ERR_NULL
    assert call(vc=None) == L.VSA_ERR_NULL                  # oc requested without vc
    big = ctypes.byref(_prob(T=64, H=64, W=32))             # Nc = 2048 is fine
    assert call(k=0, prob=big) == L.VSA_ERR_TOPK
    huge = ctypes.byref(_prob(T=64, H=64, W=128))           # Nc = 8192 > 4096
    assert call(prob=huge) == L.VSA_ERR_UNSUPPORTED


def test_sparse_attn_errors():
    lib = _raw()

    def call(prob=None, q=DUMMY, k=DUMMY, v=DUMMY, lut=DUMMY, valid=DUMMY, maxkv=8, oc=None,
             gc=None, gf=None, out=DUMMY, lse=None):
        prob = ctypes.byref(prob or _prob())
        return lib.vsa_sparse_attn_fwd(prob, q, k, v, lut, valid, maxkv, oc, gc, gf, out, lse, None)

    assert call(q=None) == L.VSA_ERR_NULL
    assert call(k=None) == L.VSA_ERR_NULL
    assert call(v=None) == L.VSA_ERR_NULL
    assert call(out=None) == L.VSA_ERR_NULL
    assert call(lut=None) == L.VSA_ERR_NULL
    assert call(valid=None) == L.VSA_ERR_NULL
    assert call(gc=DUMMY) == L.VSA_ERR_NULL                # gate_c needs oc
    assert call(maxkv=0) == L.VSA_ERR_TOPK
    assert call(maxkv=33) == L.VSA_ERR_TOPK
    assert call(prob=_prob(ct=2, ch=2, cw=2)) == L.VSA_ERR_UNSUPPORTED   # cube volume 8
    assert call(prob=_prob(head_dim=32)) == L.VSA_ERR_UNSUPPORTED
    assert call(prob=_prob(H=-4)) == L.VSA_ERR_SHAPE
    # 16-bit cube ids: Nc = 65536 is beyond the fine kernel
    assert call(prob=_prob(T=4, H=4, W=4 * 65536)) == L.VSA_ERR_UNSUPPORTED
    # the per-row (or per-quad) step list must fit beside the tile ring in
    # LDS (Nc = 16384, 16000 cubes per row)
    big = _prob(T=64, H=64, W=256)
    assert call(prob=big, maxkv=16000) == L.VSA_ERR_UNSUPPORTED


def test_sparse_attn_gather_errors():
    """The gathering entry point validates like the others, and refuses the
    shapes its loads do not cover (head size other than 128, cubes not 4
    tokens wide, grids that do not divide into cubes, a value head size of
    its own) before any launch."""
    lib = _raw()

    def call(prob=None, q=DUMMY, k=DUMMY, v=DUMMY, lut=DUMMY, valid=DUMMY, maxkv=8, oc=None,
             gc=None, gf=None, out=DUMMY, lse=None):
        prob = ctypes.byref(prob or _prob(head_dim=128))
        return lib.vsa_sparse_attn_fwd_gather(prob, q, k, v, lut, valid, maxkv, oc, gc, gf, out, lse, None)

    assert call(q=None) == L.VSA_ERR_NULL
    assert call(k=None) == L.VSA_ERR_NULL
    assert call(v=None) == L.VSA_ERR_NULL
    assert call(out=None) == L.VSA_ERR_NULL
    assert call(lut=None) == L.VSA_ERR_NULL
    assert call(valid=None) == L.VSA_ERR_NULL
    assert call(gc=DUMMY) == L.VSA_ERR_NULL
    assert call(maxkv=0) == L.VSA_ERR_TOPK
    assert call(maxkv=33) == L.VSA_ERR_TOPK
    assert call(prob=_prob(head_dim=64)) == L.VSA_ERR_UNSUPPORTED
    assert call(prob=_prob(head_dim=128, ch=8, cw=2)) == L.VSA_ERR_UNSUPPORTED       # 2 tokens wide
    assert call(prob=_prob(head_dim=128, T=8, H=16, W=14)) == L.VSA_ERR_UNSUPPORTED   # padded
    assert call(prob=_prob(head_dim=128, head_dim_v=64)) == L.VSA_ERR_UNSUPPORTED
    assert call(prob=_prob(head_dim=128, H=-4)) == L.VSA_ERR_SHAPE


def test_check_lut_errors():
    lib = _raw()
    pr = ctypes.byref(_prob())
    assert lib.vsa_check_lut(pr, DUMMY, DUMMY, 0, DUMMY, None) == L.VSA_ERR_TOPK
    assert lib.vsa_check_lut(pr, DUMMY, DUMMY, 8, None, None) == L.VSA_ERR_NULL
    assert lib.vsa_check_lut(pr, None, DUMMY, 8, DUMMY, None) == L.VSA_ERR_NULL
    assert lib.vsa_perm_index(ctypes.byref(_prob()), None) == L.VSA_ERR_NULL


def test_python_binding_rejects_wrong_shapes_before_the_library():
    import torch
    p = L.Problem(1, 1, 4, 8, 8, 4, 4, 4, 64)
    cpu = torch.zeros((1, 1, 256, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.vsa_permute(p, L.VSA_BF16, cpu, cpu)                # not device tensors
    with pytest.raises(ValueError):
        L._token_dtype(5)


def test_sparse_attn_bwd_noalloc_errors():
    """The allocation-free backward checks everything on the host before it
    looks up its fixed workspace: wrong arguments and problems whose
    workspace exceeds VSA_NOALLOC_SCRATCH_BYTES (16 MiB) are refused with no
    device work."""
    lib = _raw()
    pr = ctypes.byref(_prob(head_dim=128))

    def call(q=DUMMY, k=DUMMY, v=DUMMY, lut=DUMMY, valid=DUMMY, maxkv=8, o=DUMMY, lse=DUMMY, do=DUMMY,
             dq=DUMMY, dk=DUMMY, dv=DUMMY, prob=pr):
        return lib.vsa_sparse_attn_bwd_noalloc(prob, q, k, v, lut, valid, maxkv, o, lse, do, dq, dk, dv, None)
    for name in ("q", "k", "v", "lut", "valid", "o", "lse", "do", "dq", "dk", "dv"):
        assert call(**{name: None}) == L.VSA_ERR_NULL, name
    assert call(maxkv=0) == L.VSA_ERR_TOPK
    assert call(maxkv=33) == L.VSA_ERR_TOPK
    assert call(prob=ctypes.byref(_prob(head_dim=96))) == L.VSA_ERR_UNSUPPORTED
    assert call(prob=None) == L.VSA_ERR_NULL
    # the 122,880-token layer with 40 heads needs 39 MB of per-token records alone
    large = L.Problem(1, 40, 32, 48, 80, 4, 4, 4, 128)
    n = ctypes.c_size_t(0)
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(large.c_struct()), 192, ctypes.byref(n)) == L.VSA_OK
    assert n.value > 16 << 20
    assert call(prob=ctypes.byref(large.c_struct()), maxkv=192) == L.VSA_ERR_WORKSPACE
    # the 32,768-token layer with 12 heads fits
    wan = L.Problem(1, 12, 16, 32, 64, 4, 4, 4, 128)
    assert lib.vsa_sparse_attn_bwd_workspace_size(ctypes.byref(wan.c_struct()), 154, ctypes.byref(n)) == L.VSA_OK
    assert n.value <= 16 << 20
