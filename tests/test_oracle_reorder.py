"""Pins for the oracle's reordering (cube-major order) and cube mean-pool.

The pages fix what the reorder must achieve, not the curve itself: every
fixed-size 1-D block must be one contiguous spatio-temporal region
("VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
GPUs", §Two-Stage Architecture, pre-stage and Stage 1, 4x4x4 cubes of 64
tokens).  The reading taken is cube-major order; these tests characterise it
without re-typing the loop that builds it.
"""
import itertools

import numpy as np
import pytest

import oracle

GRIDS = [
    ((4, 8, 8), (4, 4, 4)),
    ((8, 16, 16), (4, 4, 4)),
    ((2, 4, 6), (2, 2, 2)),
    ((3, 6, 4), (3, 2, 1)),
    ((16, 32, 64), (4, 4, 4)),
]


@pytest.mark.parametrize("grid,cube", GRIDS)
def test_perm_is_bijection(grid, cube):
    pi = oracle.perm_index(*grid, *cube)
    n = grid[0] * grid[1] * grid[2]
    assert pi.shape == (n,)
    assert np.array_equal(np.sort(pi), np.arange(n))


@pytest.mark.parametrize("grid,cube", GRIDS[:4])
def test_each_block_is_one_cube_in_raster_cube_order(grid, cube):
    """Brute-force decode of every raster index back to (t, h, w)."""
    T, H, W = grid
    ct, ch, cw = cube
    vol = ct * ch * cw
    pi = oracle.perm_index(T, H, W, ct, ch, cw)
    coords = {}
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        coords[(t * H + h) * W + w] = (t, h, w)
    prev_cube = None
    for c in range(len(pi) // vol):
        blk = pi[c * vol:(c + 1) * vol]
        cubes = {(coords[r][0] // ct, coords[r][1] // ch, coords[r][2] // cw) for r in blk}
        assert len(cubes) == 1, "a block mixes tokens from two cubes"
        this = cubes.pop()
        if prev_cube is not None:
            assert this > prev_cube, "cubes are not in raster order"
        prev_cube = this
        # inside a cube tokens keep their raster order
        assert np.all(np.diff(blk) > 0)


def test_hand_worked_example():
    # Grid T=2, H=2, W=4 with 2x2x2 cubes: raster index (t*2 + h)*4 + w.
    # Cube 0 holds w in {0,1}: (t,h,w) = 000,001,010,011,100,101,110,111
    # -> 0,1,4,5,8,9,12,13; cube 1 holds w in {2,3} -> 2,3,6,7,10,11,14,15.
    expected = [0, 1, 4, 5, 8, 9, 12, 13, 2, 3, 6, 7, 10, 11, 14, 15]
    assert oracle.perm_index(2, 2, 4, 2, 2, 2).tolist() == expected


@pytest.mark.parametrize("grid,cube", GRIDS[:4])
def test_unpermute_inverts_permute(grid, cube):
    rng = np.random.default_rng(5)
    n = grid[0] * grid[1] * grid[2]
    x = rng.standard_normal((2, 3, n, 8))
    pi = oracle.perm_index(*grid, *cube)
    assert np.array_equal(oracle.unpermute(oracle.permute(x, pi), pi), x)
    assert np.array_equal(oracle.permute(oracle.unpermute(x, pi), pi), x)


def test_permute_moves_rows_as_a_gather():
    pi = oracle.perm_index(2, 2, 4, 2, 2, 2)
    x = np.arange(16, dtype=np.float64)[None, None, :, None] * np.ones((1, 1, 1, 3))
    xp = oracle.permute(x, pi)
    assert xp[0, 0, :, 0].tolist() == pi.tolist()


def test_grid_must_divide():
    with pytest.raises(ValueError):
        oracle.perm_index(4, 8, 6, 4, 4, 4)
    with pytest.raises(ValueError):
        oracle.perm_index(0, 8, 8, 4, 4, 4)


# --------------------------- pooling -------------------------------------

def test_pool_one_hot_rows():
    """A one-hot row at position p contributes 1/vol to cube p // vol only."""
    vol, nc, d = 8, 5, 3
    for p in range(vol * nc):
        x = np.zeros((1, 1, vol * nc, d))
        x[0, 0, p, 1] = 1.0
        xc = oracle.pool(x, vol)
        want = np.zeros((1, 1, nc, d))
        want[0, 0, p // vol, 1] = 1.0 / vol
        assert np.array_equal(xc, want)


def test_pool_mass_conservation_and_constants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 64 * 7, 16))
    xc = oracle.pool(x, 64)
    np.testing.assert_allclose((64 * xc).sum(axis=-2), x.sum(axis=-2), rtol=0, atol=1e-11)
    c = np.full((1, 2, 64 * 3, 4), 2.75)
    assert np.array_equal(oracle.pool(c, 64), np.full((1, 2, 3, 4), 2.75))


def test_pool_rejects_partial_cube():
    with pytest.raises(ValueError):
        oracle.pool(np.zeros((1, 1, 65, 2)), 64)
