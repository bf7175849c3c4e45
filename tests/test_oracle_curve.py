"""Pins for the Hilbert cube order (reading R21; the pages ask for a 3D
space-filling curve that keeps each fixed-size block of the 1-D sequence a
compact region of the video, [VSA-ROCm] §Two-Stage Architecture, Pre-stage).

The curve is pinned by what defines a Hilbert curve, not by retyping the
transform: it visits every cell of the 2^b cube once, each step moves to a
face neighbour, and every aligned 2^j sub-cube is one contiguous stretch of
the walk.  The reading's conventions (start at the origin, end on the t
axis) are pinned too.  The whole layer must not depend on the cube order
once the LUT names the same cubes, so its output and gradients are checked
against the raster order (attention is permutation-equivariant).
"""
import numpy as np
import pytest

import oracle


def _is_unit_step(a, b):
    return sum(abs(x - y) for x, y in zip(a, b)) == 1


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_hilbert_curve_is_a_unit_step_walk_through_the_cube(bits):
    n = 1 << bits
    seq = oracle.cube_sequence(n, n, n, "hilbert")
    assert len(seq) == n ** 3 and len(set(seq)) == n ** 3
    assert all(_is_unit_step(a, b) for a, b in zip(seq, seq[1:]))
    assert seq[0] == (0, 0, 0) and seq[-1] == (n - 1, 0, 0)
    dist = sorted(oracle.hilbert_index(*c, bits) for c in seq)
    assert dist == list(range(n ** 3))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_aligned_subcubes_are_contiguous(bits):
    n = 1 << bits
    seq = oracle.cube_sequence(n, n, n, "hilbert")
    for j in range(1, bits):
        side = 1 << j
        blocks = [(t // side, h // side, w // side) for t, h, w in seq]
        runs = [blocks[i] for i in range(0, len(blocks), side ** 3)]
        for r, b in enumerate(runs):
            assert all(x == b for x in blocks[r * side ** 3:(r + 1) * side ** 3]), (j, r)
        assert len(set(runs)) == len(runs)


@pytest.mark.parametrize("box", [(4, 8, 16), (3, 5, 7), (1, 1, 6), (6, 2, 1)])
def test_truncated_curve_keeps_the_order_of_the_full_curve(box):
    gt, gh, gw = box
    seq = oracle.cube_sequence(gt, gh, gw, "hilbert")
    assert sorted(seq) == sorted((a, b, c) for a in range(gt) for b in range(gh) for c in range(gw))
    n = 1
    while n < max(box):
        n *= 2
    full = [c for c in oracle.cube_sequence(n, n, n, "hilbert")
            if c[0] < gt and c[1] < gh and c[2] < gw]
    assert seq == full


def test_wan_cube_grid_visits_each_4x4x4_block_in_one_stretch():
    """The 32K-token layer's 4 x 8 x 16 cube grid: every aligned block of
    4 x 4 x 4 cubes (16 frames x 16 x 16 tokens) is 64 consecutive cubes
    along the curve, and every step inside a block moves one cube."""
    seq = oracle.cube_sequence(4, 8, 16, "hilbert")
    for r in range(8):
        run = seq[64 * r:64 * (r + 1)]
        assert len({(t // 4, h // 4, w // 4) for t, h, w in run}) == 1
        assert all(_is_unit_step(a, b) for a, b in zip(run, run[1:]))


def test_raster_sequence_is_the_raster_cube_order():
    assert oracle.cube_sequence(2, 3, 2, "raster") == [(a, b, c) for a in range(2) for b in range(3)
                                                         for c in range(2)]
    with pytest.raises(ValueError):
        oracle.cube_sequence(2, 2, 2, "morton")


@pytest.mark.parametrize("grid,cube", [((8, 16, 16), (4, 4, 4)), ((6, 7, 9), (4, 4, 4)), ((4, 6, 2), (2, 2, 1))])
def test_hilbert_token_layout_is_cube_major_along_the_curve(grid, cube):
    T, H, W = grid
    ct, ch, cw = cube
    vol = ct * ch * cw
    pi = oracle.token_layout(T, H, W, ct, ch, cw, "hilbert")
    real = pi[pi >= 0]
    assert sorted(real.tolist()) == list(range(T * H * W))
    seq = oracle.cube_sequence(-(-T // ct), -(-H // ch), -(-W // cw), "hilbert")
    assert len(pi) == len(seq) * vol
    for i, (a, b, c) in enumerate(seq):
        block = pi[i * vol:(i + 1) * vol]
        want = [((a * ct + lt) * H + b * ch + lh) * W + c * cw + lw
                if a * ct + lt < T and b * ch + lh < H and c * cw + lw < W else -1
                for lt in range(ct) for lh in range(ch) for lw in range(cw)]
        assert block.tolist() == want


def _relabel(lut, valid, src, dst):
    """The same key cubes, named in another cube order: cube id i in order
    src is the cube at coordinates src[i]; rows are renamed too."""
    where = {c: i for i, c in enumerate(dst)}
    to = np.array([where[c] for c in src])
    out = np.zeros_like(lut)
    vout = np.zeros_like(valid)
    for idx in np.ndindex(lut.shape[:-2]):
        for i in range(len(src)):
            n = valid[idx + (i,)]
            out[idx + (to[i], slice(0, n))] = np.sort(to[lut[idx + (i, slice(0, n))]])
            vout[idx + (to[i],)] = n
    return out, vout


def _inputs(grid, seed, heads=2, d=8):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    q, k, v = (rng.standard_normal((1, heads, n, d)) for _ in range(3))
    gc, gf = rng.random((1, heads, n, d)), rng.random((1, heads, n, d))
    return q, k, v, gc, gf


@pytest.mark.parametrize("grid,cube,top_k", [((8, 8, 8), (2, 2, 2), 64), ((8, 8, 8), (2, 2, 2), 9),
                                             ((5, 6, 7), (2, 2, 2), 7)])
def test_layer_output_does_not_depend_on_the_cube_order(grid, cube, top_k):
    """Same Top-K sets (continuous random scores: no ties), so the same
    output up to summation order; dense Top-K included."""
    q, k, v, gc, gf = _inputs(grid, 41)
    fr = oracle.vsa_forward(q, k, v, grid, cube, top_k, gate_c=gc, gate_f=gf, cube_order="raster")
    fh = oracle.vsa_forward(q, k, v, grid, cube, top_k, gate_c=gc, gate_f=gf, cube_order="hilbert")
    np.testing.assert_allclose(fh["out"], fr["out"], rtol=1e-12, atol=1e-12)
    gt, gh, gw = (-(-g // c) for g, c in zip(grid, cube))
    src = oracle.cube_sequence(gt, gh, gw, "raster")
    dst = oracle.cube_sequence(gt, gh, gw, "hilbert")
    lut, valid = _relabel(fr["kv_block_idx"], fr["valid_block_num"], src, dst)
    np.testing.assert_array_equal(fh["kv_block_idx"], lut)
    np.testing.assert_array_equal(fh["valid_block_num"], valid)


def test_layer_backward_does_not_depend_on_the_cube_order():
    grid, cube = (4, 8, 8), (2, 2, 2)
    q, k, v, gc, gf = _inputs(grid, 42)
    rng = np.random.default_rng(43)
    n = grid[0] * grid[1] * grid[2]
    dout = rng.standard_normal((1, 2, n, 8))
    nc = 2 * 4 * 4
    lut = rng.integers(0, nc, size=(1, 2, nc, 5)).astype(np.int32)
    valid = rng.integers(1, 6, size=(1, 2, nc)).astype(np.int32)
    src = oracle.cube_sequence(2, 4, 4, "raster")
    dst = oracle.cube_sequence(2, 4, 4, "hilbert")
    lut_h, valid_h = _relabel(lut, valid, src, dst)
    gr = oracle.vsa_backward(q, k, v, grid, cube, lut, valid, dout, gate_c=gc, gate_f=gf)
    gh = oracle.vsa_backward(q, k, v, grid, cube, lut_h, valid_h, dout, gate_c=gc, gate_f=gf,
                             cube_order="hilbert")
    for name in ("dq", "dk", "dv", "dgate_c", "dgate_f"):
        np.testing.assert_allclose(gh[name], gr[name], rtol=1e-11, atol=1e-12, err_msg=name)
