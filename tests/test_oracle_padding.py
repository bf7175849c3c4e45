"""Pins for grids that do not divide into cubes (reading R20: padded up to
whole cubes; padded positions are never keys, pooling averages the real
tokens only, outputs and gradients exist for real tokens only).

Independent references: with every key cube selected and no gates the layer
is dense attention over the real tokens, which torch's
scaled_dot_product_attention computes on the unpadded raster tokens (fp64,
CPU), autograd giving the gradients.  The layout is checked by decoding
every position by hand, the pooling by constant and one-hot cubes and the
adjoint identity."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GRIDS = [((5, 6, 7), (2, 2, 2)), ((3, 4, 9), (2, 4, 4)), ((4, 8, 8), (4, 4, 4))]


@pytest.mark.parametrize("grid,cube", GRIDS)
def test_layout_decodes_by_hand(grid, cube):
    (T, H, W), (ct, ch, cw) = grid, cube
    pi = oracle.token_layout(T, H, W, ct, ch, cw)
    gT, gH, gW = -(-T // ct), -(-H // ch), -(-W // cw)
    assert len(pi) == gT * gH * gW * ct * ch * cw
    real = pi >= 0
    assert sorted(pi[real].tolist()) == list(range(T * H * W))      # every token exactly once
    for p_, r in enumerate(pi):
        c, l = divmod(p_, ct * ch * cw)
        c_t, rem = divmod(c, gH * gW)
        c_h, c_w = divmod(rem, gW)
        l_t, rem = divmod(l, ch * cw)
        l_h, l_w = divmod(rem, cw)
        t, h, w = c_t * ct + l_t, c_h * ch + l_h, c_w * cw + l_w
        want = (t * H + h) * W + w if (t < T and h < H and w < W) else -1
        assert r == want
    if T % ct == 0 and H % ch == 0 and W % cw == 0:
        assert np.array_equal(pi, oracle.perm_index(T, H, W, ct, ch, cw))


def _dense(grid, cube, seed, hq=2, hk=2, d=5):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    q = rng.standard_normal((1, hq, n, d))
    k, v = rng.standard_normal((1, hk, n, d)), rng.standard_normal((1, hk, n, d))
    nc = len(oracle.token_layout(*grid, *cube)) // (cube[0] * cube[1] * cube[2])
    return q, k, v, nc


@pytest.mark.parametrize("grid,cube", GRIDS[:2])
def test_padded_dense_layer_equals_sdpa_on_real_tokens(grid, cube):
    q, k, v, nc = _dense(grid, cube, 121)
    f = oracle.vsa_forward(q, k, v, grid, cube, nc)
    want = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v))).numpy()
    np.testing.assert_allclose(f["out"], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("grid,cube", GRIDS[:2])
def test_padded_dense_layer_backward_equals_sdpa_autograd(grid, cube):
    q, k, v, nc = _dense(grid, cube, 122, hq=4, hk=2)
    lut = np.tile(np.arange(nc, dtype=np.int32), (1, 4, nc, 1))
    valid = np.full((1, 4, nc), nc, np.int32)
    dout = np.random.default_rng(123).standard_normal(q.shape)
    got = oracle.vsa_backward(q, k, v, grid, cube, lut, valid, dout)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    (o * torch.from_numpy(dout)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_pool_averages_the_real_tokens_only():
    grid, cube = (5, 6, 7), (2, 2, 2)
    pi = oracle.token_layout(*grid, *cube)
    real = pi >= 0
    n = 5 * 6 * 7
    x = np.full((1, 1, n, 3), 2.5)
    xp = oracle.gather_padded(x, pi)
    np.testing.assert_allclose(oracle.pool_real(xp, 8, real), 2.5, rtol=0, atol=1e-15)
    # a one-hot token lands at 1 / (its cube's real count)
    one = np.zeros((1, 1, n, 1))
    one[0, 0, n - 1, 0] = 1.0                 # the last token sits in the last, partial cube
    pc = oracle.pool_real(oracle.gather_padded(one, pi), 8, real)
    count = real[-8:].sum()
    assert count < 8 and pc[0, 0, -1, 0] == 1.0 / count and pc[..., :-1, :].sum() == 0


def test_pool_real_bwd_is_the_adjoint_of_pool_real():
    grid, cube = (3, 4, 9), (2, 4, 4)
    pi = oracle.token_layout(*grid, *cube)
    real = pi >= 0
    rng = np.random.default_rng(124)
    x = rng.standard_normal((2, 1, len(pi), 4))
    y = rng.standard_normal((2, 1, len(pi) // 32, 4))
    lhs = (oracle.pool_real(x, 32, real) * y).sum()
    rhs = (x * oracle.pool_real_bwd(y, 32, real)).sum()
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))
