"""GPU parity with the Hilbert cube order (reading R21: cubes follow a 3D
Hilbert curve over the cube grid; tokens inside a cube stay in raster order).

Only the steps that map a cube to grid coordinates change (the reorders,
the pools over padded cubes, the fine kernel's raster epilogue and its
padded-key masks); the coarse stage, the LUT and the backward work on cube
ids whatever their order.  Bars as for the raster order: reorder bit-exact,
pool within vol * 2^-24 * max|x|, attention outputs max-abs 2e-2 and
mean-abs 2e-3, Top-K sets tie-tolerant, O_c within 1e-4, gradients max 2% of
max |grad| and mean 1% of mean |grad|.  The oracle builds its own Hilbert
layout (token_layout); nothing it sees comes from the GPU.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward, VsaForward
from gpu_helpers import (OC_MAX_ABS, assert_out_close, bits, check_lut_against_scores, dev, err, host64,
                         inputs, problem)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(f"\n[case] {msg}", flush=True)


def _bf(a):
    return wl.f32_to_bf16_bits(np.asarray(a, np.float32))


def _bnhd(t):
    return t.permute(0, 2, 1, 3).contiguous()


DIMS = [(1, 2, 8, 16, 16, 4, 4, 4, 128), (1, 3, 16, 32, 64, 4, 4, 4, 64), (1, 2, 21, 30, 52, 4, 4, 4, 128),
        (2, 2, 3, 5, 2, 2, 2, 2, 64)]


@pytest.mark.parametrize("dims", DIMS, ids=["8x16x16", "16x32x64", "21x30x52", "3x5x2-vol8"])
def test_hilbert_reorder_and_pool(dims):
    B, nh, T, H, W, ct, ch, cw, d = dims
    _log(f"hilbert reorder/pool {dims}")
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d, cube_order="hilbert")
    pi = oracle.token_layout(T, H, W, ct, ch, cw, "hilbert")
    real = pi >= 0
    vol = ct * ch * cw
    rng = np.random.default_rng(101)
    x = _bf(rng.standard_normal((B, nh, p.n_tokens, d)))
    xt = dev(x)
    pos, cs = (B, nh, p.n_positions, d), (B, nh, p.n_cubes, d)
    xc = torch.full(pos, float("nan"), dtype=torch.bfloat16, device="cuda")
    pooled = torch.full(cs, float("nan"), device="cuda")
    L.vsa_permute_pool(p, L.VSA_BF16, xt, xc, pooled)
    xc2 = torch.full_like(xc, float("nan"))
    pooled2 = torch.full_like(pooled, float("nan"))
    L.vsa_permute_pool_bnhd(p, L.VSA_BF16, _bnhd(xt), xc2, pooled2)
    back = torch.full_like(xt, float("nan"))
    L.vsa_unpermute(p, L.VSA_BF16, xc, back)
    dx = rng.standard_normal(pos).astype(np.float32)
    dxc = rng.standard_normal(cs).astype(np.float32)
    g = torch.full((B, nh, p.n_tokens, d), float("nan"), device="cuda")
    L.vsa_pool_unpermute_bwd(p, dev(dx), dev(dxc), g)
    torch.cuda.synchronize()
    xv = wl.as_float64(x)
    want = oracle.gather_padded(xv, pi)
    assert np.array_equal(host64(xc), want)
    assert np.array_equal(bits(xc2), bits(xc)) and np.array_equal(bits(pooled2), bits(pooled))
    assert np.array_equal(bits(back), bits(xt))
    assert err(host64(pooled), oracle.pool_real(want, vol, real))[0] <= vol * 2.0 ** -24 * np.abs(xv).max()
    y = oracle.pool_real_bwd(dxc, vol, real)
    gw = oracle.scatter_padded(dx.astype(np.float64) + y, pi, p.n_tokens)
    bound = 2.0 ** -22 * oracle.scatter_padded(np.abs(dx) + np.abs(y), pi, p.n_tokens)
    assert np.all(np.abs(host64(g) - gw) <= bound)


def _hilbert_pipeline_case(w, top_k, cubes, heads_checked, grid=None):
    """VsaForward in Hilbert order on raster inputs, against the oracle's
    Hilbert-order layer on the LUT the GPU chose."""
    p = dataclasses.replace(problem(w), cube_order="hilbert")
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    f = VsaForward(p, top_k)
    out = torch.full_like(q, float("nan"))
    f(q, k, v, out, gc, gf)
    fr = VsaForward(problem(w), top_k)
    out_r = torch.full_like(q, float("nan"))
    fr(q, k, v, out_r, gc, gf)
    torch.cuda.synchronize()
    hs = list(heads_checked)
    pi = oracle.token_layout(w.T, w.H, w.W, *w.cube, "hilbert")
    xs = {n: wl.as_float64(x[n][:, hs]) for n in x}
    qp, kp, vp = (oracle.permute(xs[n], pi) for n in ("q", "k", "v"))
    pooled = [oracle.pool(a, 64) for a in (qp, kp, vp)]
    scale = 1.0 / math.sqrt(w.head_dim)
    s, _, oc_w = oracle.coarse_attention(*pooled, scale)
    lut_w, _ = oracle.topk_lut(s, top_k)
    lut_g = f.lut.cpu().numpy()[:, hs]
    differ = check_lut_against_scores(lut_g, f.valid.cpu().numpy()[:, hs], s, top_k, lut_w)
    assert err(host64(f.oc)[:, hs], oc_w)[0] <= OC_MAX_ABS
    qcs = [(0, hi, i) for hi in range(len(hs)) for i in cubes]
    of, _ = oracle.fine_attention(qp, kp, vp, lut_g, np.full(lut_g.shape[:-1], top_k, np.int32), scale, 64,
                                  query_cubes=qcs)
    outp = oracle.combine(of, host64(f.oc)[:, hs], 64, oracle.permute(xs["gate_c"], pi),
                          oracle.permute(xs["gate_f"], pi))
    rows = np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in cubes])
    got = host64(out)
    assert np.all(np.isfinite(got))
    mx, mean = assert_out_close(got[:, hs][:, :, pi[rows]], outp[:, :, rows], f"hilbert pipeline {w.name}")
    # the raster-order pipeline computes the same layer (same Top-K sets up to ties)
    mx_r, mean_r = err(got, host64(out_r))
    print(f"tie-window LUT rows {differ}; out max-abs {mx:.3e} mean-abs {mean:.3e}; "
          f"vs raster order max-abs {mx_r:.3e} mean-abs {mean_r:.3e}")
    assert mean_r <= 2e-3


def test_hilbert_pipeline_small():
    w = wl.SMALL
    _log("hilbert pipeline small")
    _hilbert_pipeline_case(w, w.top_k, list(range(w.n_cubes)), range(w.heads))


def test_hilbert_pipeline_wan():
    w = wl.WORKLOADS["wan"]
    _log("hilbert pipeline wan K=154")
    _hilbert_pipeline_case(w, 154, [0, 1, 63, 64, 200, 311, 510, 511], [0, 7])


@pytest.mark.parametrize("dims,hk", [((1, 4, 8, 16, 16, 4, 4, 4, 128), 2), ((1, 2, 5, 7, 9, 4, 4, 4, 64), 0)],
                         ids=["8x16x16-gqa", "5x7x9-padded"])
def test_hilbert_layer_backward(dims, hk):
    """Forward intermediates and VsaBackward in Hilbert order against the
    oracle's vsa_backward in Hilbert order (random LUT in Hilbert ids)."""
    B, nh, T, H, W, ct, ch, cw, d = dims
    _log(f"hilbert layer backward {dims} kv heads {hk or nh}")
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d, heads_kv=hk, cube_order="hilbert")
    pkv = p.kv_problem()
    hkv = p.kv_heads
    rng = np.random.default_rng(102)
    q, dout = (_bf(rng.standard_normal((B, nh, p.n_tokens, d))) for _ in range(2))
    gc, gf = (_bf(rng.random((B, nh, p.n_tokens, d))) for _ in range(2))
    k, v = (_bf(rng.standard_normal((B, hkv, p.n_tokens, d))) for _ in range(2))
    maxk = 6
    lut = rng.integers(0, p.n_cubes, size=(B, nh, p.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(B, nh, p.n_cubes)).astype(np.int32)
    pos, kpos = (B, nh, p.n_positions, d), (B, hkv, p.n_positions, d)
    cs, kcs = (B, nh, p.n_cubes, d), (B, hkv, p.n_cubes, d)
    bf = torch.bfloat16
    saved = {"qp": torch.empty(pos, dtype=bf, device="cuda"), "kp": torch.empty(kpos, dtype=bf, device="cuda"),
             "vp": torch.empty(kpos, dtype=bf, device="cuda"), "qc": torch.empty(cs, device="cuda"),
             "oc": torch.empty(cs, device="cuda"), "kc": torch.empty(kcs, device="cuda"),
             "vc": torch.empty(kcs, device="cuda"), "kv_block_idx": dev(lut), "valid_block_num": dev(valid)}
    L.vsa_permute_pool(p, L.VSA_BF16, dev(q), saved["qp"], saved["qc"])
    L.vsa_permute_pool(pkv, L.VSA_BF16, dev(k), saved["kp"], saved["kc"])
    L.vsa_permute_pool(pkv, L.VSA_BF16, dev(v), saved["vp"], saved["vc"])
    tl = torch.empty((B, nh, p.n_cubes, 1), dtype=torch.int32, device="cuda")
    tv = torch.empty((B, nh, p.n_cubes), dtype=torch.int32, device="cuda")
    L.vsa_coarse_topk(p, 1, saved["qc"], saved["kc"], saved["vc"], tl, tv, saved["oc"])
    o_f = torch.empty(pos, dtype=bf, device="cuda")
    lse = torch.empty((B, nh, p.n_positions), device="cuda")
    L.vsa_sparse_attn_fwd(p, saved["qp"], saved["kp"], saved["vp"], saved["kv_block_idx"],
                          saved["valid_block_num"], o_f, lse=lse)
    rs, krs = (B, nh, p.n_tokens, d), (B, hkv, p.n_tokens, d)
    dq, dgc, dgf = (torch.full(rs, float("nan"), device="cuda") for _ in range(3))
    dk, dv = (torch.full(krs, float("nan"), device="cuda") for _ in range(2))
    VsaBackward(p, maxk)(saved, o_f, lse, dev(dout), dq, dk, dv, gate_c=dev(gc), gate_f=dev(gf),
                         dgate_c=dgc, dgate_f=dgf)
    torch.cuda.synchronize()
    f64 = wl.as_float64
    ref = oracle.vsa_backward(f64(q), f64(k), f64(v), (T, H, W), (ct, ch, cw), lut, valid, f64(dout),
                              gate_c=f64(gc), gate_f=f64(gf), cube_order="hilbert")
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dgate_c", dgc), ("dgate_f", dgf)):
        g_, r_ = host64(t), ref[nm]
        assert np.all(np.isfinite(g_)), nm
        e = np.abs(g_ - r_)
        mx, mn = e.max() / np.abs(r_).max(), e.mean() / np.abs(r_).mean()
        print(f"{nm}: max {mx:.2e} of max, mean {mn:.2e} of mean")
        assert mx <= 2e-2 and mn <= 1e-2, nm
