"""Mutation checks: plant a plausible mistake in the oracle (on the CPU, by
monkeypatching one of its steps) and require that at least one pin fails.
This shows the pins are tight enough to catch a dropped term, a wrong index,
a transposed operand or a wrong sign."""
import math

import numpy as np
import pytest

import oracle
from oracle import vsa_oracle as vo
import test_oracle_coarse as tc
import test_oracle_curve as tcv
import test_oracle_fine as tf
import test_oracle_bwd as tb
import test_oracle_full_bwd as tfb
import test_oracle_gqa as tg
import test_oracle_padding as tpad
import test_oracle_mask as tm
import test_oracle_reorder as tr
from block_sparse_video_major_amd import workloads as wl


_ORIG = {n: getattr(vo, n) for n in ("pool", "topk_lut", "fine_attention", "combine", "mask_to_lut",
                                     "fine_attention_bwd", "coarse_attention_bwd", "pool_bwd", "combine_bwd",
                                     "pool_real")}


def _hilbert_variant(t, h, w, bits, gray=True, reflect_on_set=True, t_first=True):
    """The oracle's transform with one planted change (see the callers)."""
    x = [t, h, w]
    level = 1 << (bits - 1)
    while level > 1:
        low = level - 1
        for i in range(3):
            if bool(x[i] & level) == reflect_on_set:
                x[0] ^= low
            else:
                swap = (x[0] ^ x[i]) & low
                x[0] ^= swap
                x[i] ^= swap
        level >>= 1
    if gray:
        x[1] ^= x[0]
        x[2] ^= x[1]
        flip = 0
        level = 1 << (bits - 1)
        while level > 1:
            if x[2] & level:
                flip ^= level - 1
            level >>= 1
        x = [c ^ flip for c in x]
    order = (0, 1, 2) if t_first else (2, 1, 0)
    dist = 0
    for b in range(bits - 1, -1, -1):
        for i in order:
            dist = (dist << 1) | ((x[i] >> b) & 1)
    return dist


def _hilbert_no_gray(t, h, w, bits):
    return _hilbert_variant(t, h, w, bits, gray=False)


def _hilbert_branches_swapped(t, h, w, bits):
    return _hilbert_variant(t, h, w, bits, reflect_on_set=False)


def _hilbert_w_first(t, h, w, bits):
    return _hilbert_variant(t, h, w, bits, t_first=False)


def _raster_perm(T, H, W, ct, ch, cw):
    return np.arange(T * H * W, dtype=np.int64)


def _pool_wrong_divisor(xp, vol):
    return _ORIG["pool"](xp, vol) * vol / (vol - 1)


def _scores_no_scale(qc, kc, scale):
    return np.matmul(qc, np.swapaxes(kc, -1, -2))


def _softmax_wrong_axis(s):
    m = s.max(axis=-2, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-2, keepdims=True)


def _topk_smallest(s, k):
    return _ORIG["topk_lut"](-s, k)


def _fine_no_scale(qp, kp, vp, lut, valid, scale, vol, **kw):
    return _ORIG["fine_attention"](qp, kp, vp, lut, valid, 1.0, vol, **kw)


def _fine_q_for_k(qp, kp, vp, lut, valid, scale, vol, **kw):
    return _ORIG["fine_attention"](qp, qp, vp, lut, valid, scale, vol, **kw)


def _fine_shifted_block(qp, kp, vp, lut, valid, scale, vol, **kw):
    nc = qp.shape[-2] // vol
    return _ORIG["fine_attention"](qp, kp, vp, (lut + 1) % nc, valid, scale, vol, **kw)


def _combine_swapped(of, oc, vol, gate_c=None, gate_f=None):
    return _ORIG["combine"](of, oc, vol, gate_f, gate_c)


def _mask_descending(mask, max_kv):
    lut, valid, over = _ORIG["mask_to_lut"](mask, max_kv)
    out = lut.copy()
    for idx in np.ndindex(*valid.shape):
        n = valid[idx]
        out[idx][:n] = lut[idx][:n][::-1]
    return out, valid, over


def _mask_transposed(mask, max_kv):
    return _ORIG["mask_to_lut"](np.swapaxes(np.asarray(mask), -1, -2), max_kv)


def _mask_last_blocks_on_overflow(mask, max_kv):
    m = np.asarray(mask)[..., ::-1]
    lut, valid, over = _ORIG["mask_to_lut"](m, max_kv)
    nc = m.shape[-1]
    out = lut.copy()
    for idx in np.ndindex(*valid.shape):
        n = valid[idx]
        out[idx][:n] = np.sort(nc - 1 - lut[idx][:n])
    return out, valid, over


def _bwd_dk_no_scale(qp, kp, vp, lut, valid, scale, vol, of, lse, dof, **kw):
    dq, dk, dv = _ORIG["fine_attention_bwd"](qp, kp, vp, lut, valid, scale, vol, of, lse, dof, **kw)
    return dq, dk / scale, dv


def _bwd_no_rowsum_term(qp, kp, vp, lut, valid, scale, vol, of, lse, dof, **kw):
    # D = rowsum(dO * O) dropped: equivalent to passing O = 0
    return _ORIG["fine_attention_bwd"](qp, kp, vp, lut, valid, scale, vol, np.zeros_like(of), lse, dof, **kw)


def _bwd_dv_from_q(qp, kp, vp, lut, valid, scale, vol, of, lse, dof, **kw):
    dq, dk, dv = _ORIG["fine_attention_bwd"](qp, kp, vp, lut, valid, scale, vol, of, lse, dof, **kw)
    return dq, dk, dq


def _coarse_bwd_dk_no_scale(qc, kc, vc, scale, doc):
    dq, dk, dv = _ORIG["coarse_attention_bwd"](qc, kc, vc, scale, doc)
    return dq, dk / scale, dv


def _pool_bwd_no_divisor(dxc, vol):
    return _ORIG["pool_bwd"](dxc, vol) * vol


def _combine_bwd_dgc_from_of(dout, of, oc, vol, gate_c=None, gate_f=None):
    dof, doc, dgc, dgf = _ORIG["combine_bwd"](dout, of, oc, vol, gate_c, gate_f)
    return dof, doc, (None if dgc is None else np.asarray(dout) * np.asarray(of)), dgf


def _expand_interleaved(x, group):
    # head h takes key/value head h % kv_heads instead of h // group
    return np.tile(np.asarray(x), (1, group) + (1,) * (np.asarray(x).ndim - 2))


def _fine_attends_padding(qp, kp, vp, lut, valid, scale, vol, **kw):
    kw.pop("key_valid", None)
    return _ORIG["fine_attention"](qp, kp, vp, lut, valid, scale, vol, **kw)


def _pool_real_full_volume(xp, vol, real):
    # divides by the cube volume instead of the real-token count
    return _ORIG["pool_real"](xp, vol, real) * real.reshape(-1, vol).sum(axis=1)[:, None] / vol


def _pins():
    """The pin checks, called directly (each raises AssertionError on failure)."""
    yield lambda: tr.test_each_block_is_one_cube_in_raster_cube_order((4, 8, 8), (4, 4, 4))
    yield lambda: tr.test_hand_worked_example()
    yield lambda: tr.test_pool_one_hot_rows()
    yield lambda: tr.test_pool_mass_conservation_and_constants()
    yield lambda: tc.test_coarse_softmax_matches_scipy_and_sums_to_one()
    yield lambda: tc.test_coarse_output_special_cases()
    yield lambda: tc.test_topk_characterisation()
    yield lambda: tc.test_topk_subset_enumeration_tiny()
    yield lambda: tf.test_all_cubes_selected_is_dense_sdpa(wl.TINY)
    yield lambda: tf.test_gather_equals_materialised_mask(wl.TINY)
    yield lambda: tf.test_single_block_is_attention_inside_one_cube()
    yield lambda: tf.test_gates_select_fine_or_coarse()
    yield lambda: tb.test_backward_matches_autograd_with_duplicates_and_empty_rows()
    yield lambda: tb.test_dv_of_uniform_attention_is_column_sum()
    yield lambda: tm.test_relation_matrix_of_a_topk_lut_gives_the_lut_back()
    yield lambda: tm.test_masked_fine_attention_is_dense_masked_softmax()
    yield lambda: tm.test_overflow_rows_are_counted_and_keep_their_first_blocks()
    yield lambda: tfb.test_coarse_attention_bwd_matches_autograd()
    yield lambda: tfb.test_pool_bwd_is_the_adjoint_of_pool()
    yield lambda: tfb.test_combine_bwd_matches_autograd()
    yield lambda: tfb.test_whole_layer_backward_matches_autograd()
    yield lambda: tg.test_dense_layer_equals_gqa_sdpa(4, 2)
    yield lambda: tpad.test_padded_dense_layer_equals_sdpa_on_real_tokens((5, 6, 7), (2, 2, 2))
    yield lambda: tpad.test_pool_averages_the_real_tokens_only()
    yield lambda: tcv.test_hilbert_curve_is_a_unit_step_walk_through_the_cube(3)
    yield lambda: tcv.test_aligned_subcubes_are_contiguous(3)
    yield lambda: tcv.test_hilbert_token_layout_is_cube_major_along_the_curve((6, 7, 9), (4, 4, 4))


MUTATIONS = {
    "raster order instead of cube-major": ("perm_index", _raster_perm),
    "pool divides by vol-1": ("pool", _pool_wrong_divisor),
    "coarse scores without 1/sqrt(d)": ("coarse_scores", _scores_no_scale),
    "coarse softmax over the query axis": ("softmax_rows", _softmax_wrong_axis),
    "Top-K keeps the smallest scores": ("topk_lut", _topk_smallest),
    "fine softmax without 1/sqrt(d)": ("fine_attention", _fine_no_scale),
    "fine uses Q where K belongs": ("fine_attention", _fine_q_for_k),
    "fine reads the neighbouring cube": ("fine_attention", _fine_shifted_block),
    "gates swapped": ("combine", _combine_swapped),
    "mask rows listed descending": ("mask_to_lut", _mask_descending),
    "backward dK without the softmax scale": ("fine_attention_bwd", _bwd_dk_no_scale),
    "backward dS without the rowsum(dO*O) term": ("fine_attention_bwd", _bwd_no_rowsum_term),
    "backward dV taken from dQ": ("fine_attention_bwd", _bwd_dv_from_q),
    "mask read transposed": ("mask_to_lut", _mask_transposed),
    "mask overflow keeps the last blocks": ("mask_to_lut", _mask_last_blocks_on_overflow),
    "coarse backward dKc without the scale": ("coarse_attention_bwd", _coarse_bwd_dk_no_scale),
    "pool backward without 1/vol": ("pool_bwd", _pool_bwd_no_divisor),
    "combine backward dg_c taken from O_f": ("combine_bwd", _combine_bwd_dgc_from_of),
    "grouped heads interleaved instead of repeated": ("expand_kv_heads", _expand_interleaved),
    "padded positions attended as keys": ("fine_attention", _fine_attends_padding),
    "padded cubes averaged over the full volume": ("pool_real", _pool_real_full_volume),
    "Hilbert transform without the Gray encoding": ("hilbert_index", _hilbert_no_gray),
    "Hilbert transform with reflect and exchange swapped": ("hilbert_index", _hilbert_branches_swapped),
    "Hilbert bits interleaved w first": ("hilbert_index", _hilbert_w_first),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(vo, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for pin in _pins():
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()
