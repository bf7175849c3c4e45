"""Pins for grouped heads in the oracle (reading R19: query head h uses
key/value head h // G).  With every key cube selected and no gates the layer
is dense attention, which torch's scaled_dot_product_attention computes
with enable_gqa (fp64, CPU); its autograd gives the gradients, dK and dV
summed over each key/value head's query heads."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _inputs(seed, B=1, hq=4, hk=2, grid=(4, 4, 8), d=6):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    q = rng.standard_normal((B, hq, N, d))
    k = rng.standard_normal((B, hk, N, d))
    v = rng.standard_normal((B, hk, N, d))
    return q, k, v


@pytest.mark.parametrize("hq,hk", [(4, 2), (4, 1), (6, 3)])
def test_dense_layer_equals_gqa_sdpa(hq, hk):
    q, k, v = _inputs(101, hq=hq, hk=hk)
    grid, cube = (4, 4, 8), (2, 2, 2)
    nc = 128 // 8
    f = oracle.vsa_forward(q, k, v, grid, cube, nc)
    want = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v)), enable_gqa=True).numpy()
    np.testing.assert_allclose(f["out"], want, rtol=1e-12, atol=1e-12)


def test_dense_layer_backward_equals_gqa_sdpa_autograd():
    q, k, v = _inputs(102, hq=4, hk=2)
    grid, cube = (4, 4, 8), (2, 2, 2)
    nc = 16
    lut = np.tile(np.arange(nc, dtype=np.int32), (1, 4, nc, 1))
    valid = np.full((1, 4, nc), nc, np.int32)
    dout = np.random.default_rng(103).standard_normal(q.shape)
    got = oracle.vsa_backward(q, k, v, grid, cube, lut, valid, dout)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    (o * torch.from_numpy(dout)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_group_of_one_is_plain_heads():
    q, k, v = _inputs(104, hq=2, hk=2)
    a = oracle.expand_kv_heads(k, 1)
    assert np.array_equal(a, k)
    assert np.array_equal(oracle.reduce_kv_heads(k, 1), k)


def test_reduce_is_the_adjoint_of_expand():
    rng = np.random.default_rng(105)
    x = rng.standard_normal((2, 3, 5, 4))
    y = rng.standard_normal((2, 6, 5, 4))
    lhs = (oracle.expand_kv_heads(x, 2) * y).sum()
    rhs = (x * oracle.reduce_kv_heads(y, 2)).sum()
    assert abs(lhs - rhs) < 1e-12


def test_group_must_divide():
    q, k, _ = _inputs(106, hq=4, hk=3)
    with pytest.raises(ValueError):
        oracle.kv_group(q, k)
