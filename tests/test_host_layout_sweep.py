"""Seeded sweep of the library's host helpers against the oracle's layout:
random token grids and cube edges (divisible or padded), both cube orders.
vsa_perm_index and vsa_cube_table are host code, so this runs on the CPU;
the oracle builds its layout from loops over the padded grid
(token_layout) and its own Hilbert transform (cube_sequence)."""
import numpy as np
import pytest

import oracle
from block_sparse_video_major_amd import _lib as L


def _cases(n=60, seed=141):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        cube = tuple(int(c) for c in rng.integers(1, 5, size=3))
        grid = tuple(int(g) for g in rng.integers(1, 23, size=3))
        out.append((grid, cube, "hilbert" if i % 2 else "raster"))
    return out


@pytest.mark.parametrize("grid,cube,order", _cases())
def test_host_layout_matches_oracle(grid, cube, order):
    p = L.Problem(1, 1, *grid, *cube, 64, cube_order=order)
    pi = oracle.token_layout(*grid, *cube, order)
    assert p.n_positions == len(pi) and p.n_cubes * p.cube_volume == len(pi)
    assert np.array_equal(L.vsa_perm_index(p).numpy(), pi)
    seq = oracle.cube_sequence(*p.cube_grid, order)
    assert L.vsa_cube_table(p).tolist() == [(t << 20) | (h << 10) | w for t, h, w in seq]
