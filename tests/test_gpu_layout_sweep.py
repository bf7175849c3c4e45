"""Seeded sweep of the reorder and pool passes over random problems: token
grids and cube edges (divisible or padded), raster or Hilbert cube order,
bf16 or fp32, [batch, heads, N, d] or [batch, N, heads, d] on the raster
side.  Bars as for the fixed shapes: reorders bit-exact (zeros at padding),
pools within vol * 2^-24 * max|x|, pool + reorder backward within
2^-22 * (|x| + |y| / n_c).  Inputs are seeded draws; the oracle lays the grid
out itself."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from gpu_helpers import bits, dev, err, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _cases(n=24, seed=151):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        cube = tuple(int(c) for c in rng.integers(1, 5, size=3))
        grid = tuple(int(g) for g in rng.integers(1, 19, size=3))
        out.append(dict(B=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)), grid=grid, cube=cube,
                        d=int(rng.choice([64, 128])), order=("raster", "hilbert")[i % 2],
                        dtype=(L.VSA_BF16, L.VSA_F32)[(i // 2) % 2], bnhd=bool((i // 4) % 2)))
    return out


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"{c['grid']}-{c['cube']}-{c['order']}-{c['dtype']}")
def test_reorder_pool_sweep(c):
    B, nh, d = c["B"], c["heads"], c["d"]
    print(f"\n[case] {c}", flush=True)
    p = L.Problem(B, nh, *c["grid"], *c["cube"], d, cube_order=c["order"])
    pi = oracle.token_layout(*c["grid"], *c["cube"], c["order"])
    real = pi >= 0
    vol = p.cube_volume
    rng = np.random.default_rng(152)
    x = rng.standard_normal((B, nh, p.n_tokens, d)).astype(np.float32)
    if c["dtype"] == L.VSA_BF16:
        xh, td = wl.f32_to_bf16_bits(x), torch.bfloat16
        xv = wl.as_float64(xh)
    else:
        xh, td = x, torch.float32
        xv = x.astype(np.float64)
    xt = dev(xh)
    src = xt.permute(0, 2, 1, 3).contiguous() if c["bnhd"] else xt
    xc = torch.full((B, nh, p.n_positions, d), float("nan"), dtype=td, device="cuda")
    pooled = torch.full((B, nh, p.n_cubes, d), float("nan"), device="cuda")
    if c["bnhd"]:
        L.vsa_permute_pool_bnhd(p, c["dtype"], src, xc, pooled)
    else:
        L.vsa_permute_pool(p, c["dtype"], src, xc, pooled)
    back = torch.full_like(xt, float("nan"))
    L.vsa_unpermute(p, c["dtype"], xc, back)
    dx = rng.standard_normal((B, nh, p.n_positions, d)).astype(np.float32)
    dxc = rng.standard_normal((B, nh, p.n_cubes, d)).astype(np.float32)
    if c["bnhd"]:
        g = torch.full((B, p.n_tokens, nh, d), float("nan"), device="cuda")
        L.vsa_pool_unpermute_bwd_bnhd(p, dev(dx), dev(dxc), g)
    else:
        g = torch.full((B, nh, p.n_tokens, d), float("nan"), device="cuda")
        L.vsa_pool_unpermute_bwd(p, dev(dx), dev(dxc), g)
    torch.cuda.synchronize()
    want = oracle.gather_padded(xv, pi)
    assert np.array_equal(host64(xc), want)
    assert np.array_equal(bits(back), bits(xt))
    assert err(host64(pooled), oracle.pool_real(want, vol, real))[0] <= vol * 2.0 ** -24 * np.abs(xv).max()
    y = oracle.pool_real_bwd(dxc, vol, real)
    gw = oracle.scatter_padded(dx.astype(np.float64) + y, pi, p.n_tokens)
    bound = 2.0 ** -22 * oracle.scatter_padded(np.abs(dx) + np.abs(y), pi, p.n_tokens)
    gh = host64(g)
    if c["bnhd"]:
        gh = gh.transpose(0, 2, 1, 3)
    assert np.all(np.abs(gh - gw) <= bound)
