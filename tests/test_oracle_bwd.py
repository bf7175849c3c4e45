"""Pins for the oracle's fine-stage backward (gradients of block-sparse
attention; "VSA: Faster Video Diffusion with Trainable Sparse Attention",
Abstract: the method is trained end to end).

The oracle writes the gradients out by hand from the forward's definition;
these pins check them against torch autograd (fp64, CPU) of an independent
formulation (index_select of the key rows, dense softmax) and against central
finite differences of the oracle's own forward.
"""
import math

import numpy as np
import torch

import oracle


def _problem(seed, B=1, nh=2, nc=5, vol=8, d=6, maxk=4, dup=False, empty=False):
    rng = np.random.default_rng(seed)
    qp, kp, vp = (rng.standard_normal((B, nh, nc * vol, d)) for _ in range(3))
    lut = np.zeros((B, nh, nc, maxk), np.int32)
    valid = np.zeros((B, nh, nc), np.int32)
    for idx in np.ndindex(B, nh, nc):
        n = int(rng.integers(1, maxk + 1))
        lut[idx][:n] = np.sort(rng.choice(nc, n, replace=False))
        valid[idx] = n
    if dup:
        lut[0, 0, 1, :2] = [3, 3]
        valid[0, 0, 1] = 2
    if empty:
        valid[0, 1, 2] = 0
    return qp, kp, vp, lut, valid, 1.0 / math.sqrt(d), vol


def _autograd(qp, kp, vp, lut, valid, scale, vol, dof):
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (qp, kp, vp))
    B, nh, N, d = qp.shape
    outs = torch.zeros(B, nh, N, d, dtype=torch.float64)
    pieces = []
    for b in range(B):
        for h in range(nh):
            for i in range(N // vol):
                n = int(valid[b, h, i])
                if n == 0:
                    continue
                idx = torch.tensor(np.concatenate([np.arange(j * vol, (j + 1) * vol) for j in lut[b, h, i, :n]]))
                kk = k[b, h].index_select(0, idx)
                vv = v[b, h].index_select(0, idx)
                s = scale * q[b, h, i * vol:(i + 1) * vol] @ kk.T
                o = torch.softmax(s, dim=-1) @ vv
                pieces.append(((b, h, i), o))
    loss = sum((o * torch.from_numpy(dof[b, h, i * vol:(i + 1) * vol])).sum() for (b, h, i), o in pieces)
    loss.backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def test_backward_matches_autograd_with_duplicates_and_empty_rows():
    qp, kp, vp, lut, valid, scale, vol = _problem(41, dup=True, empty=True)
    of, lse = oracle.fine_attention(qp, kp, vp, lut, valid, scale, vol)
    dof = np.random.default_rng(42).standard_normal(of.shape)
    dq, dk, dv = oracle.fine_attention_bwd(qp, kp, vp, lut, valid, scale, vol, of, lse, dof)
    gq, gk, gv = _autograd(qp, kp, vp, lut, valid, scale, vol, dof)
    for got, want in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert np.all(dq[0, 1, 2 * vol:3 * vol] == 0.0)     # the empty row gets no gradient


def test_backward_matches_central_differences():
    """d(sum(dO * O_f))/dx by central differences of the oracle's forward."""
    qp, kp, vp, lut, valid, scale, vol = _problem(43, nh=1, nc=3, vol=4, d=3, maxk=2)
    of, lse = oracle.fine_attention(qp, kp, vp, lut, valid, scale, vol)
    dof = np.random.default_rng(44).standard_normal(of.shape)
    grads = oracle.fine_attention_bwd(qp, kp, vp, lut, valid, scale, vol, of, lse, dof)
    eps = 1e-6
    for which, g in zip(range(3), grads):
        rng = np.random.default_rng(45 + which)
        for _ in range(12):
            pos = tuple(int(rng.integers(0, n)) for n in qp.shape)
            args = [qp.copy(), kp.copy(), vp.copy()]
            args[which][pos] += eps
            fp = (oracle.fine_attention(*args, lut, valid, scale, vol)[0] * dof).sum()
            args[which][pos] -= 2 * eps
            fm = (oracle.fine_attention(*args, lut, valid, scale, vol)[0] * dof).sum()
            assert abs((fp - fm) / (2 * eps) - g[pos]) < 1e-7, (which, pos)


def test_dv_of_uniform_attention_is_column_sum():
    """Q = 0: P is uniform over the listed keys, so dV of every listed key
    row is the mean of dO over the query cube (closed form)."""
    qp, kp, vp, lut, valid, scale, vol = _problem(46, nh=1, nc=4, vol=4, d=3, maxk=1)
    qp[:] = 0.0
    of, lse = oracle.fine_attention(qp, kp, vp, lut, valid, scale, vol)
    dof = np.random.default_rng(47).standard_normal(of.shape)
    _, _, dv = oracle.fine_attention_bwd(qp, kp, vp, lut, valid, scale, vol, of, lse, dof)
    want = np.zeros_like(dv)
    for i in range(4):
        j = lut[0, 0, i, 0]
        want[0, 0, j * vol:(j + 1) * vol] += dof[0, 0, i * vol:(i + 1) * vol].mean(axis=0)
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-13)
