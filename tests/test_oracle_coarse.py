"""Pins for the oracle's coarse stage: cube scores, coarse softmax/output and
Top-K selection ("VSA: Accelerating Video Diffusion Inference with Sparse
Attention on AMD GPUs", §Two-Stage Architecture Stage 1 and §Generating
Sparsity Patterns)."""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle


def test_scores_brute_force_loop():
    rng = np.random.default_rng(2)
    qc = rng.standard_normal((1, 2, 5, 7))
    kc = rng.standard_normal((1, 2, 6, 7))
    s = oracle.coarse_scores(qc, kc, 0.25)
    for h in range(2):
        for i in range(5):
            for j in range(6):
                acc = 0.0
                for t in range(7):
                    acc += qc[0, h, i, t] * kc[0, h, j, t]
                assert abs(s[0, h, i, j] - 0.25 * acc) < 1e-12


def test_coarse_softmax_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(3)
    qc, kc, vc = (rng.standard_normal((1, 3, 32, 64)) for _ in range(3))
    scale = 1 / math.sqrt(64)
    s, p, oc = oracle.coarse_attention(qc, kc, vc, scale)
    np.testing.assert_allclose(p, scipy.special.softmax(scale * qc @ np.swapaxes(kc, -1, -2), axis=-1),
                               rtol=0, atol=1e-14)
    assert np.max(np.abs(p.sum(-1) - 1)) < 1e-12
    # softmax rows over keys, not over queries
    assert not np.allclose(p.sum(-2), 1)


def test_coarse_output_special_cases():
    rng = np.random.default_rng(4)
    qc, kc = rng.standard_normal((1, 1, 16, 8)), rng.standard_normal((1, 1, 16, 8))
    const = np.broadcast_to(np.arange(8.0), (1, 1, 16, 8))
    _, _, oc = oracle.coarse_attention(qc, kc, const, 0.3)
    np.testing.assert_allclose(oc, const, rtol=0, atol=1e-12)
    # one cube: O_c = Vc
    vc1 = rng.standard_normal((1, 1, 1, 8))
    _, p1, oc1 = oracle.coarse_attention(qc[:, :, :1], kc[:, :, :1], vc1, 0.3)
    assert np.array_equal(p1, np.ones((1, 1, 1, 1)))
    np.testing.assert_allclose(oc1, vc1, rtol=0, atol=0)
    # zero queries: uniform average of Vc
    vc = rng.standard_normal((1, 1, 16, 8))
    _, _, oc0 = oracle.coarse_attention(np.zeros_like(qc), kc, vc, 0.3)
    np.testing.assert_allclose(oc0, np.broadcast_to(vc.mean(-2, keepdims=True), oc0.shape), atol=1e-14)


def test_topk_characterisation():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((2, 3, 32, 32))
    for k in (1, 5, 8, 31, 32):
        lut, valid = oracle.topk_lut(s, k)
        assert lut.shape == (2, 3, 32, k) and lut.dtype == np.int32
        assert np.all(valid == k)
        for idx in np.ndindex(2, 3, 32):
            sel = lut[idx]
            assert np.all(np.diff(sel) > 0), "LUT rows must be ascending and distinct"
            mask = np.zeros(32, bool)
            mask[sel] = True
            row = s[idx]
            if k < 32:
                assert row[mask].min() >= row[~mask].max()


def test_topk_subset_enumeration_tiny():
    """Tiny grid (4 cubes, K=2): the chosen set is the unique maximiser of the
    summed score among all C(4,2) subsets (tie-free data)."""
    rng = np.random.default_rng(7)
    s = rng.standard_normal((1, 1, 4, 4))
    lut, _ = oracle.topk_lut(s, 2)
    for i in range(4):
        best = max(itertools.combinations(range(4), 2), key=lambda c: s[0, 0, i, list(c)].sum())
        assert tuple(lut[0, 0, i]) == best


def test_topk_ties_take_lower_index():
    s = np.array([[[[1.0, 3.0, 3.0, 3.0, 0.0, 3.0]]]])
    lut, _ = oracle.topk_lut(s, 2)
    assert lut[0, 0, 0].tolist() == [1, 2]
    lut, _ = oracle.topk_lut(s, 4)
    assert lut[0, 0, 0].tolist() == [1, 2, 3, 5]
    # signed zeros are equal scores
    z = np.array([[[[-0.0, 0.0, -1.0]]]])
    assert oracle.topk_lut(z, 1)[0][0, 0, 0].tolist() == [0]


def test_topk_all_and_bounds():
    s = np.random.default_rng(8).standard_normal((1, 1, 6, 6))
    lut, _ = oracle.topk_lut(s, 6)
    assert np.array_equal(lut[0, 0], np.tile(np.arange(6), (6, 1)))
    for bad in (0, 7):
        with pytest.raises(ValueError):
            oracle.topk_lut(s, bad)
