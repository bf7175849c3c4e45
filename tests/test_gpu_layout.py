"""GPU checks of the model-layout entry points ([batch, N, heads, d] on the
raster side): vsa_permute_bnhd, vsa_permute_pool_bnhd, vsa_sparse_attn_fwd_bnhd
and vsa_pool_unpermute_bwd_bnhd.

Reordering is index work, so the bar is bit-exactness: the cube-major output
equals the oracle's reorder of the transposed input, and each entry point
writes exactly the bits its [batch, heads, N, d] counterpart writes,
transposed (the arithmetic, pooling order and attention included, is the
same).
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from gpu_helpers import bits, dev, inputs, problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(f"\n[case] {msg}", flush=True)


def _bnhd(t):
    return t.transpose(1, 2).contiguous()


DIMS = [(1, 4, 8, 16, 16, 4, 4, 4, 64), (2, 3, 2, 4, 6, 2, 2, 2, 128), (1, 12, 16, 32, 64, 4, 4, 4, 128)]


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("dtype", [L.VSA_BF16, L.VSA_F32])
def test_permute_and_pool_from_model_layout(dims, dtype):
    B, nh, T, H, W, ct, ch, cw, d = dims
    _log(f"permute(_pool)_bnhd {dims} dtype={dtype}")
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d)
    N, vol = T * H * W, ct * ch * cw
    td = torch.bfloat16 if dtype == L.VSA_BF16 else torch.float32
    g = torch.Generator(device="cuda").manual_seed(91)
    x = torch.randn((B, nh, N, d), generator=g, device="cuda").to(td)
    xb = _bnhd(x)
    cube_a, cube_b, cube_c = (torch.empty_like(x) for _ in range(3))
    xc_a, xc_b = (torch.empty((B, nh, N // vol, d), device="cuda") for _ in range(2))
    L.vsa_permute_pool(p, dtype, x, cube_a, xc_a)
    L.vsa_permute_pool_bnhd(p, dtype, xb, cube_b, xc_b)
    L.vsa_permute_bnhd(p, dtype, xb, cube_c)
    torch.cuda.synchronize()
    pi = oracle.perm_index(T, H, W, ct, ch, cw)
    want = np.take(bits(x), pi, axis=2)
    assert np.array_equal(bits(cube_b), want)
    assert np.array_equal(bits(cube_c), want)
    assert np.array_equal(bits(xc_b), bits(xc_a))


@pytest.mark.parametrize("dims", DIMS[:2] + [(1, 2, 3, 6, 4, 3, 2, 1, 64)])
def test_pool_unpermute_bwd_to_model_layout(dims):
    B, nh, T, H, W, ct, ch, cw, d = dims
    _log(f"pool_unpermute_bwd_bnhd {dims}")
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d)
    N, vol = T * H * W, ct * ch * cw
    g = torch.Generator(device="cuda").manual_seed(92)
    dx = torch.randn((B, nh, N, d), generator=g, device="cuda")
    dxc = torch.randn((B, nh, N // vol, d), generator=g, device="cuda")
    a = torch.empty_like(dx)
    b = torch.empty((B, N, nh, d), device="cuda")
    L.vsa_pool_unpermute_bwd(p, dx, dxc, a)
    L.vsa_pool_unpermute_bwd_bnhd(p, dx, dxc, b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(b), bits(_bnhd(a)))


@pytest.mark.parametrize("name", ["small", "wan"])
def test_sparse_attn_fwd_to_model_layout(name):
    w = wl.WORKLOADS[name]
    _log(f"sparse_attn_fwd_bnhd {name}")
    p = problem(w)
    x = inputs(name)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    q, k, v = (dev(np.take(x[n], pi, axis=2)) for n in ("q", "k", "v"))
    gc, gf = dev(x["gate_c"]), dev(x["gate_f"])
    rng = np.random.default_rng(93)
    lut = np.stack([np.sort(rng.permutation(w.n_cubes)[:w.top_k])
                    for _ in range(w.heads * w.n_cubes)]).reshape(1, w.heads, w.n_cubes, w.top_k).astype(np.int32)
    valid = np.full((1, w.heads, w.n_cubes), w.top_k, np.int32)
    oc = torch.randn((1, w.heads, w.n_cubes, w.head_dim), device="cuda")
    out_a = torch.empty_like(q)
    out_b = torch.empty((1, w.n_tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse_a, lse_b = (torch.empty((1, w.heads, w.n_tokens), device="cuda") for _ in range(2))
    L.vsa_sparse_attn_fwd_raster(p, q, k, v, dev(lut), dev(valid), out_a, oc=oc, gate_c=gc, gate_f=gf, lse=lse_a)
    L.vsa_sparse_attn_fwd_bnhd(p, q, k, v, dev(lut), dev(valid), out_b, oc=oc, gate_c=_bnhd(gc), gate_f=_bnhd(gf),
                               lse=lse_b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_b), bits(_bnhd(out_a)))
    assert np.array_equal(bits(lse_b), bits(lse_a))


def test_pipeline_in_model_layout_matches_bhnd():
    w = wl.SMALL
    _log("VsaForward layout=bnhd")
    from block_sparse_video_major_amd.pipeline import VsaForward
    p = problem(w)
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    out_a = torch.empty_like(q)
    VsaForward(p, w.top_k)(q, k, v, out_a, gc, gf)
    out_b = torch.empty((1, w.n_tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    VsaForward(p, w.top_k, layout="bnhd")(_bnhd(q), _bnhd(k), _bnhd(v), out_b, _bnhd(gc), _bnhd(gf))
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_b), bits(_bnhd(out_a)))
