"""Pins for the oracle's backward of the remaining steps (combine, coarse
attention, pooling) and of the whole layer ("VSA: Faster Video Diffusion with
Trainable Sparse Attention", Abstract: trained end to end; the LUT is held
fixed).

Each oracle gradient is written out by hand.  The pins check it against
torch autograd (fp64, CPU) of forwards written here independently of the
oracle, and against adjoint (dot-product) identities.  The whole-layer test
builds the cube order from a reshape of the token grid, pools with a reshape
mean and runs dense softmax attention over the gathered key rows, then
differentiates <out, dout> with autograd.
"""
import math

import numpy as np
import torch

import oracle


def _t(a, grad=True):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=grad)


def test_coarse_attention_bwd_matches_autograd():
    rng = np.random.default_rng(71)
    qc, kc, vc = (rng.standard_normal((2, 3, 7, 5)) for _ in range(3))
    doc = rng.standard_normal((2, 3, 7, 5))
    scale = 1 / math.sqrt(5)
    q, k, v = _t(qc), _t(kc), _t(vc)
    o = torch.softmax(scale * q @ k.transpose(-1, -2), dim=-1) @ v
    (o * torch.from_numpy(doc)).sum().backward()
    got = oracle.coarse_attention_bwd(qc, kc, vc, scale, doc)
    for g, want in zip(got, (q.grad, k.grad, v.grad)):
        np.testing.assert_allclose(g, want.numpy(), rtol=1e-12, atol=1e-12)


def test_coarse_attention_bwd_one_cube_has_zero_score_gradient():
    """One cube: P = 1 whatever the scores, so dQc = dKc = 0 and dVc = dO_c."""
    rng = np.random.default_rng(72)
    qc, kc, vc, doc = (rng.standard_normal((1, 1, 1, 4)) for _ in range(4))
    dq, dk, dv = oracle.coarse_attention_bwd(qc, kc, vc, 0.5, doc)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, doc, rtol=0, atol=1e-15)


def test_pool_bwd_is_the_adjoint_of_pool():
    """<pool(x), y> = <x, pool_bwd(y)> for every x, y."""
    rng = np.random.default_rng(73)
    for vol in (1, 8, 64):
        x = rng.standard_normal((2, 3, 5 * vol, 4))
        y = rng.standard_normal((2, 3, 5, 4))
        lhs = (oracle.pool(x, vol) * y).sum()
        rhs = (x * oracle.pool_bwd(y, vol)).sum()
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_combine_bwd_matches_autograd():
    rng = np.random.default_rng(74)
    vol, nc, d = 4, 3, 5
    of = rng.standard_normal((1, 2, nc * vol, d))
    oc = rng.standard_normal((1, 2, nc, d))
    gc, gf = rng.random((1, 2, nc * vol, d)), rng.random((1, 2, nc * vol, d))
    dout = rng.standard_normal((1, 2, nc * vol, d))
    o_f, o_c, g_c, g_f = _t(of), _t(oc), _t(gc), _t(gf)
    out = g_f * o_f + g_c * o_c.repeat_interleave(vol, dim=-2)
    (out * torch.from_numpy(dout)).sum().backward()
    dof, doc, dgc, dgf = oracle.combine_bwd(dout, of, oc, vol, gc, gf)
    for g, want in ((dof, o_f.grad), (doc, o_c.grad), (dgc, g_c.grad), (dgf, g_f.grad)):
        np.testing.assert_allclose(g, want.numpy(), rtol=1e-13, atol=1e-13)
    # absent gates: g_f = 1 passes dout through, absent g_c cuts the coarse path
    dof, doc, dgc, dgf = oracle.combine_bwd(dout, of, oc, vol)
    np.testing.assert_array_equal(dof, dout)
    assert np.all(doc == 0) and dgc is None and dgf is None


def _cube_order(T, H, W, ct, ch, cw):
    """Raster index of each cube-major position, from a reshape of the grid."""
    idx = torch.arange(T * H * W).reshape(T // ct, ct, H // ch, ch, W // cw, cw)
    return idx.permute(0, 2, 4, 1, 3, 5).reshape(-1)


def _layer_autograd(q, k, v, grid, cube, lut, valid, dout, gc, gf):
    T, H, W = grid
    ct, ch, cw = cube
    vol = ct * ch * cw
    order = _cube_order(T, H, W, ct, ch, cw)
    tq, tk, tv = _t(q), _t(k), _t(v)
    tgc, tgf = _t(gc), _t(gf)
    d = q.shape[-1]
    scale = 1 / math.sqrt(d)
    B, nh, N, _ = q.shape
    nc = N // vol
    qp, kp, vp = tq[:, :, order], tk[:, :, order], tv[:, :, order]
    gcp, gfp = tgc[:, :, order], tgf[:, :, order]
    qc, kc, vc = (x.reshape(B, nh, nc, vol, d).mean(dim=3) for x in (qp, kp, vp))
    oc = torch.softmax(scale * qc @ kc.transpose(-1, -2), dim=-1) @ vc
    rows = []
    for b in range(B):
        for h in range(nh):
            per_cube = []
            for i in range(nc):
                n = int(valid[b, h, i])
                if n == 0:
                    per_cube.append(torch.zeros(vol, d, dtype=torch.float64))
                    continue
                idx = torch.cat([torch.arange(j * vol, (j + 1) * vol) for j in lut[b, h, i, :n].tolist()])
                s = scale * qp[b, h, i * vol:(i + 1) * vol] @ kp[b, h, idx].T
                per_cube.append(torch.softmax(s, dim=-1) @ vp[b, h, idx])
            rows.append(torch.cat(per_cube))
    of = torch.stack(rows).reshape(B, nh, N, d)
    outp = gfp * of + gcp * oc.repeat_interleave(vol, dim=-2)
    out = torch.empty_like(outp)
    out[:, :, order] = outp
    (out * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tgc.grad.numpy(), tgf.grad.numpy()


def test_whole_layer_backward_matches_autograd():
    rng = np.random.default_rng(75)
    grid, cube = (4, 4, 8), (2, 2, 2)      # 128 tokens, 16 cubes of 8
    B, nh, d = 1, 2, 6
    N = 128
    q, k, v = (rng.standard_normal((B, nh, N, d)) for _ in range(3))
    gc, gf = rng.random((B, nh, N, d)), rng.random((B, nh, N, d))
    dout = rng.standard_normal((B, nh, N, d))
    maxk = 5
    lut = rng.integers(0, 16, size=(B, nh, 16, maxk)).astype(np.int32)
    valid = rng.integers(0, maxk + 1, size=(B, nh, 16)).astype(np.int32)
    lut[0, 0, 3, :2] = 9                   # a cube listed twice
    valid[0, 0, 3] = 3
    valid[0, 1, 5] = 0                     # an empty row
    got = oracle.vsa_backward(q, k, v, grid, cube, lut, valid, dout, gate_c=gc, gate_f=gf)
    want = _layer_autograd(q, k, v, grid, cube, lut, valid, dout, gc, gf)
    for name, w in zip(("dq", "dk", "dv", "dgate_c", "dgate_f"), want):
        np.testing.assert_allclose(got[name], w, rtol=1e-10, atol=1e-11, err_msg=name)
