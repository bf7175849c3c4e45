"""Pins for the oracle's block relation matrix -> index list conversion.

Source: "VSA: Accelerating Video Diffusion Inference with Sparse Attention on
AMD GPUs", §Comparison with Jenga ("Sparse Encoding in CK Tile": a block-mask
method stores the M x M one-hot relation matrix, VSA the selected indices and
their count) and §Block-Sparse Encoding.  Reading R15: ascending order; rows
with more selected blocks than the list holds keep the first ones and count
as overflows.
"""
import math

import numpy as np

import oracle
from block_sparse_video_major_amd import workloads as wl


def test_relation_matrix_of_a_topk_lut_gives_the_lut_back():
    """A Top-K LUT written as a one-hot matrix (numpy scatter) converts back
    to itself: same ascending rows, count K, no overflow."""
    rng = np.random.default_rng(21)
    s = rng.standard_normal((2, 3, 12, 12))
    lut, valid = oracle.topk_lut(s, 5)
    mask = np.zeros(s.shape, np.uint8)
    np.put_along_axis(mask, lut.astype(np.int64), 1, axis=-1)
    got, gvalid, over = oracle.mask_to_lut(mask, 5)
    assert np.array_equal(got, lut) and np.array_equal(gvalid, valid) and over == 0


def test_masked_fine_attention_is_dense_masked_softmax():
    """Attention over the converted list equals dense softmax over the token
    mask np.kron(B, ones(vol, vol)) written out directly, including a row
    with no selected block (output 0) and rows of different counts."""
    rng = np.random.default_rng(22)
    B, nh, nc, vol, d = 1, 2, 6, 8, 5
    qp, kp, vp = (rng.standard_normal((B, nh, nc * vol, d)) for _ in range(3))
    mask = (rng.random((B, nh, nc, nc)) < 0.4).astype(np.uint8)
    mask[0, 0, 2, :] = 0          # empty row
    mask[0, 1, 3, :] = 1          # full row
    lut, valid, over = oracle.mask_to_lut(mask, nc)
    assert over == 0
    scale = 1.0 / math.sqrt(d)
    got, _ = oracle.fine_attention(qp, kp, vp, lut, valid, scale, vol)
    for h in range(nh):
        allowed = np.kron(mask[0, h], np.ones((vol, vol))) > 0
        sc = scale * qp[0, h] @ kp[0, h].T
        for r in range(nc * vol):
            if not allowed[r].any():
                assert np.all(got[0, h, r] == 0.0)
                continue
            e = np.exp(sc[r][allowed[r]] - sc[r][allowed[r]].max())
            want = (e / e.sum()) @ vp[0, h][allowed[r]]
            np.testing.assert_allclose(got[0, h, r], want, rtol=0, atol=1e-12)


def test_overflow_rows_are_counted_and_keep_their_first_blocks():
    """Brute force: row i of a 10 x 10 matrix selects cubes 0..i (i + 1
    blocks); with a list of 4 the rows i >= 4 overflow and keep 0, 1, 2, 3."""
    nc, maxk = 10, 4
    mask = np.tril(np.ones((nc, nc), np.uint8))[None, None]
    lut, valid, over = oracle.mask_to_lut(mask, maxk)
    assert over == nc - maxk
    for i in range(nc):
        n = min(i + 1, maxk)
        assert valid[0, 0, i] == n
        assert list(lut[0, 0, i, :n]) == list(range(n))


def test_block_relation_mask_structure():
    """The seeded union mask: every cube attends itself and its grid
    neighbours (symmetric), the condition cubes, and at least K cubes."""
    w = wl.SMALL
    k, ncond = 3, 2
    m = wl.block_relation_mask(w, k, ncond)
    nc = w.n_cubes
    assert m.shape == (w.batch, w.heads, nc, nc)
    rows = m.sum(axis=-1)
    assert rows.min() >= k and np.all(m[..., :ncond] == 1)
    assert np.all(np.diagonal(m, axis1=-2, axis2=-1) == 1)
    adj_part = m[0, 0] & m[0, 0].T
    assert np.all(np.diagonal(adj_part) == 1)
    assert len(np.unique(rows)) > 1, "row counts should vary"
