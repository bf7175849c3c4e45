"""Pins for a value head size different from the query/key head size
(reading R22: O_f, O_c, the gates and the output take V's width; the
softmax scale is 1/sqrt of the query/key width).  With every key cube
selected the layer is dense attention, which torch's
scaled_dot_product_attention computes for any value width (fp64, CPU); its
autograd gives the gradients.  The coarse stage is checked against a
pooled dense attention written here."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _inputs(seed, dq, dv, hq=2, hk=2, grid=(4, 4, 8)):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return (rng.standard_normal((1, hq, n, dq)), rng.standard_normal((1, hk, n, dq)),
            rng.standard_normal((1, hk, n, dv)))


@pytest.mark.parametrize("dq,dv,hq,hk", [(6, 10, 2, 2), (12, 4, 2, 2), (6, 10, 4, 2)])
def test_dense_layer_equals_sdpa_with_other_value_width(dq, dv, hq, hk):
    q, k, v = _inputs(111, dq, dv, hq, hk)
    grid, cube = (4, 4, 8), (2, 2, 2)
    f = oracle.vsa_forward(q, k, v, grid, cube, 16)
    want = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v)), enable_gqa=hq != hk).numpy()
    assert f["out"].shape == (1, hq, 128, dv)
    np.testing.assert_allclose(f["out"], want, rtol=1e-12, atol=1e-12)
    # the coarse output is dense attention of the cube means, value width dv
    qc, kc, vc = (a.reshape(1, -1, 2, 2, 2, 2, 4, 2, a.shape[-1]).transpose(0, 1, 2, 4, 6, 3, 5, 7, 8)
                  .reshape(1, a.shape[1], 16, 8, a.shape[-1]).mean(axis=3) for a in (q, k, v))
    oc = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (qc, kc, vc)), enable_gqa=hq != hk).numpy()
    assert f["oc"].shape == (1, hq, 16, dv)
    np.testing.assert_allclose(f["oc"], oc, rtol=1e-12, atol=1e-12)


def test_dense_layer_backward_with_other_value_width():
    q, k, v = _inputs(112, 6, 10)
    grid, cube = (4, 4, 8), (2, 2, 2)
    nc = 16
    lut = np.tile(np.arange(nc, dtype=np.int32), (1, 2, nc, 1))
    valid = np.full((1, 2, nc), nc, np.int32)
    dout = np.random.default_rng(113).standard_normal((1, 2, 128, 10))
    got = oracle.vsa_backward(q, k, v, grid, cube, lut, valid, dout)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    (F.scaled_dot_product_attention(tq, tk, tv) * torch.from_numpy(dout)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert got[name].shape == t.shape
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_gated_sparse_layer_with_other_value_width_matches_a_direct_sum():
    """Sparse rows and gates: one query token's output written out from its
    listed key cubes' tokens (softmax over them), plus the gated coarse
    output of its cube."""
    q, k, v = _inputs(114, 8, 4)
    rng = np.random.default_rng(115)
    gc, gf = rng.random((1, 2, 128, 4)), rng.random((1, 2, 128, 4))
    grid, cube = (4, 4, 8), (2, 2, 2)
    f = oracle.vsa_forward(q, k, v, grid, cube, 5, gate_c=gc, gate_f=gf)
    pi = f["pi"]
    for h, p in ((0, 3), (1, 77), (1, 127)):
        i = p // 8
        keys = np.concatenate([np.arange(8 * j, 8 * j + 8) for j in f["kv_block_idx"][0, h, i]])
        s = q[0, h, pi[p]] @ k[0, h, pi[keys]].T / np.sqrt(8)
        w = np.exp(s - s.max())
        of = (w / w.sum()) @ v[0, h, pi[keys]]
        want = gf[0, h, pi[p]] * of + gc[0, h, pi[p]] * f["oc"][0, h, i]
        np.testing.assert_allclose(f["out"][0, h, pi[p]], want, rtol=1e-12, atol=1e-12)
