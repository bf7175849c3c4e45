"""GPU parity with a value head size different from the query/key head size
(reading R22: V, Vc, O_c, the gates and the output are d_v wide; the softmax
scale is 1/sqrt of the query/key width).  (d, d_v) in {(128, 64), (64, 128)}.

Bars as for equal head sizes: Top-K sets tie-tolerant, O_c within 1e-4,
attention outputs max-abs 2e-2 and mean-abs 2e-3, LSE within 1e-3, gradients
max 2% of max |grad| and mean 1% of mean |grad|.  Every
input is a seeded draw; nothing the oracle sees comes from the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward, VsaForward
from gpu_helpers import (LSE_MAX_ABS, OC_MAX_ABS, assert_out_close, bits, check_lut_against_scores, dev, err,
                         host64)

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


def _gather_bits(x, pi):
    out = np.zeros(x.shape[:-2] + (len(pi), x.shape[-1]), dtype=x.dtype)
    real = pi >= 0
    out[..., real, :] = x[..., pi[real], :]
    return out


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 128)])
def test_coarse_topk_other_value_width(d, dv):
    _log(f"coarse_topk d={d} d_v={dv}")
    p = L.Problem(1, 4, 8, 16, 16, 4, 4, 4, d, heads_kv=2, head_dim_v=dv)
    rng = np.random.default_rng(121)
    nc, k = p.n_cubes, 7
    qc = (0.5 * rng.standard_normal((1, 4, nc, d))).astype(np.float32)
    kc = rng.standard_normal((1, 2, nc, d)).astype(np.float32)
    vc = rng.standard_normal((1, 2, nc, dv)).astype(np.float32)
    lut = torch.empty((1, 4, nc, k), dtype=torch.int32, device="cuda")
    valid = torch.empty((1, 4, nc), dtype=torch.int32, device="cuda")
    oc = torch.full((1, 4, nc, dv), float("nan"), device="cuda")
    L.vsa_coarse_topk(p, k, dev(qc), dev(kc), dev(vc), lut, valid, oc)
    torch.cuda.synchronize()
    s, _, oc_w = oracle.coarse_attention(qc.astype(np.float64), oracle.expand_kv_heads(kc, 2).astype(np.float64),
                                         oracle.expand_kv_heads(vc, 2).astype(np.float64), 1 / math.sqrt(d))
    lut_w, _ = oracle.topk_lut(s, k)
    check_lut_against_scores(lut.cpu().numpy(), valid.cpu().numpy(), s, k, lut_w)
    assert err(host64(oc), oc_w)[0] <= OC_MAX_ABS


# (batch, heads, kv heads, T, H, W, d, d_v, max_kv, sampled query cubes or None)
FINE = [(1, 4, 4, 8, 16, 16, 128, 64, 9, None), (1, 4, 2, 8, 16, 16, 64, 128, 9, None),
        (2, 2, 1, 5, 7, 9, 64, 128, 6, None), (1, 3, 3, 6, 8, 8, 128, 64, 5, None),
        (1, 12, 12, 16, 32, 64, 128, 64, 154, [0, 1, 200, 511]),
        (1, 12, 12, 16, 32, 64, 64, 128, 154, [0, 77, 510, 511])]


@pytest.mark.parametrize("case", FINE, ids=["8x16x16-128-64", "8x16x16-64-128-gqa", "5x7x9-padded-64-128",
                                            "6x8x8-padded-128-64", "wan-128-64", "wan-64-128"])
def test_sparse_attn_fwd_other_value_width(case):
    """Cube-major O_f and LSE, raster output with gates and O_c, and the
    model layout; random LUT rows with repeats, varying counts and empty
    rows."""
    B, nh, hk, T, H, W, d, dv, maxk, cubes = case
    _log(f"sparse_attn_fwd {case}")
    p = L.Problem(B, nh, T, H, W, 4, 4, 4, d, heads_kv=hk if hk != nh else 0, head_dim_v=dv)
    pi = oracle.token_layout(T, H, W, 4, 4, 4)
    real = pi >= 0
    nc = p.n_cubes
    rng = np.random.default_rng(122)
    q = _bf(rng.standard_normal((B, nh, p.n_tokens, d)))
    k = _bf(rng.standard_normal((B, hk, p.n_tokens, d)))
    v = _bf(rng.standard_normal((B, hk, p.n_tokens, dv)))
    gc, gf = (_bf(rng.random((B, nh, p.n_tokens, dv))) for _ in range(2))
    oc = rng.standard_normal((B, nh, nc, dv)).astype(np.float32)
    lut = rng.integers(0, nc, size=(B, nh, nc, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(B, nh, nc)).astype(np.int32)
    valid[0, 0, 1] = 0                                    # an empty row: O_f = 0, LSE = -inf
    qp, kp, vp = (dev(_gather_bits(a, pi)) for a in (q, k, v))
    o_cube = torch.full((B, nh, p.n_positions, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_cube = torch.full((B, nh, p.n_positions), float("nan"), device="cuda")
    L.vsa_sparse_attn_fwd(p, qp, kp, vp, dev(lut), dev(valid), o_cube, lse=lse_cube)
    o_r = torch.full((B, nh, p.n_tokens, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.vsa_sparse_attn_fwd_raster(p, qp, kp, vp, dev(lut), dev(valid), o_r, oc=dev(oc), gate_c=dev(gc),
                                 gate_f=dev(gf))
    o_b = torch.full((B, p.n_tokens, nh, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.vsa_sparse_attn_fwd_bnhd(p, qp, kp, vp, dev(lut), dev(valid), o_b, oc=dev(oc), gate_c=_bnhd(dev(gc)),
                               gate_f=_bnhd(dev(gf)))
    torch.cuda.synchronize()
    f64 = wl.as_float64
    g = nh // hk
    qc_list = list(range(nc)) if cubes is None else cubes
    qcs = [(b, h, i) for b in range(B) for h in range(nh) for i in qc_list]
    of, lse = oracle.fine_attention(oracle.gather_padded(f64(q), pi),
                                    oracle.expand_kv_heads(oracle.gather_padded(f64(k), pi), g),
                                    oracle.expand_kv_heads(oracle.gather_padded(f64(v), pi), g),
                                    lut, valid, 1 / math.sqrt(d), 64, query_cubes=qcs,
                                    key_valid=None if real.all() else real)
    rows = np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in qc_list])
    rows = rows[real[rows]]
    assert_out_close(host64(o_cube)[:, :, rows], of[:, :, rows], "cube-major O_f")
    lg, lw = host64(lse_cube)[:, :, rows], lse[:, :, rows]
    fin = np.isfinite(lw)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(lg[~fin] == -np.inf)
    assert err(lg[fin], lw[fin])[0] <= LSE_MAX_ABS
    outp = oracle.combine(of, oc.astype(np.float64), 64, oracle.gather_padded(f64(gc), pi),
                          oracle.gather_padded(f64(gf), pi))
    assert_out_close(host64(o_r)[:, :, pi[rows]], outp[:, :, rows], "raster out")
    if cubes is None:
        assert np.all(np.isfinite(host64(o_r)))
    assert np.array_equal(bits(o_b), bits(_bnhd(o_r)))


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 128)])
def test_pipeline_other_value_width(d, dv):
    """VsaForward on raster inputs (grouped heads): the Top-K sets, O_c and
    the output on the LUT the GPU chose, against the oracle."""
    _log(f"pipeline d={d} d_v={dv}")
    B, nh, hk, T, H, W = 1, 4, 2, 8, 16, 16
    p = L.Problem(B, nh, T, H, W, 4, 4, 4, d, heads_kv=hk, head_dim_v=dv)
    rng = np.random.default_rng(123)
    q = _bf(rng.standard_normal((B, nh, p.n_tokens, d)))
    k = _bf(rng.standard_normal((B, hk, p.n_tokens, d)))
    v = _bf(rng.standard_normal((B, hk, p.n_tokens, dv)))
    gc, gf = (_bf(rng.random((B, nh, p.n_tokens, dv))) for _ in range(2))
    top_k = 8
    f = VsaForward(p, top_k)
    out = torch.full((B, nh, p.n_tokens, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    f(dev(q), dev(k), dev(v), out, dev(gc), dev(gf))
    torch.cuda.synchronize()
    f64 = wl.as_float64
    ref = oracle.vsa_forward(f64(q), f64(k), f64(v), (T, H, W), (4, 4, 4), top_k, gate_c=f64(gc),
                             gate_f=f64(gf))
    lut_g, valid_g = f.lut.cpu().numpy(), f.valid.cpu().numpy()
    differ = check_lut_against_scores(lut_g, valid_g, ref["scores"], top_k, ref["kv_block_idx"])
    assert err(host64(f.oc), ref["oc"])[0] <= OC_MAX_ABS
    want = oracle.vsa_forward(f64(q), f64(k), f64(v), (T, H, W), (4, 4, 4), top_k, gate_c=f64(gc),
                              gate_f=f64(gf), kv_block_idx=lut_g, valid_block_num=valid_g)
    mx, mean = assert_out_close(host64(out), want["out"], "pipeline out")
    print(f"tie-window rows {differ}; max-abs {mx:.3e} mean-abs {mean:.3e}")


def _grad_check(name, got, ref):
    g, r = host64(got), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    e = np.abs(g - r)
    mx, mn = e.max() / max(np.abs(r).max(), 1e-30), e.mean() / max(np.abs(r).mean(), 1e-30)
    print(f"{name}: max {mx:.2e} of max, mean {mn:.2e} of mean")
    assert mx <= 2e-2 and mn <= 1e-2, name


@pytest.mark.parametrize("d,dv,hk", [(128, 64, 2), (64, 128, 4), (64, 128, 1)])
def test_sparse_attn_bwd_other_value_width(d, dv, hk):
    """Fine-stage gradients (every element) against the oracle's, on the
    oracle's O_f and LSE; rows with repeats, varying counts, one empty row.
    Bars of the fine backward: max 2% of max |grad|, mean 1% of mean |grad|."""
    B, nh, T, H, W = 1, 4, 8, 16, 16
    _log(f"sparse_attn_bwd d={d} d_v={dv} kv heads {hk}")
    p = L.Problem(B, nh, T, H, W, 4, 4, 4, d, heads_kv=hk if hk != nh else 0, head_dim_v=dv)
    nc, g = p.n_cubes, nh // hk
    rng = np.random.default_rng(124)
    qp = _bf(rng.standard_normal((B, nh, p.n_positions, d)))
    kp = _bf(rng.standard_normal((B, hk, p.n_positions, d)))
    vp = _bf(rng.standard_normal((B, hk, p.n_positions, dv)))
    maxk = 9
    lut = rng.integers(0, nc, size=(B, nh, nc, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(B, nh, nc)).astype(np.int32)
    valid[0, 0, 2] = 0
    lut[0, 1, 0, :3] = 5
    f64 = wl.as_float64
    q64, k64, v64 = f64(qp), oracle.expand_kv_heads(f64(kp), g), oracle.expand_kv_heads(f64(vp), g)
    scale = 1 / math.sqrt(d)
    of, lse = oracle.fine_attention(q64, k64, v64, lut, valid, scale, 64)
    of_bits = _bf(of)
    lse32 = lse.astype(np.float32)
    dof_bits = _bf(rng.standard_normal(of.shape))
    dq = torch.full((B, nh, p.n_positions, d), float("nan"), device="cuda")
    dk = torch.full((B, hk, p.n_positions, d), float("nan"), device="cuda")
    dvt = torch.full((B, hk, p.n_positions, dv), float("nan"), device="cuda")
    ws = torch.full((L.vsa_sparse_attn_bwd_workspace_size(p, maxk),), 0xA5, dtype=torch.uint8, device="cuda")
    L.vsa_sparse_attn_bwd(p, dev(qp), dev(kp), dev(vp), dev(lut), dev(valid), dev(of_bits), dev(lse32),
                          dev(dof_bits), dq, dk, dvt, ws)
    torch.cuda.synchronize()
    ref = oracle.fine_attention_bwd(q64, k64, v64, lut, valid, scale, 64, f64(of_bits), lse32.astype(np.float64),
                                    f64(dof_bits))
    _grad_check("dq", dq, ref[0])
    _grad_check("dk", dk, oracle.reduce_kv_heads(ref[1], g))
    _grad_check("dv", dvt, oracle.reduce_kv_heads(ref[2], g))
    assert np.all(host64(dq)[0, 0, 2 * 64:3 * 64] == 0.0)   # the empty row


@pytest.mark.parametrize("dims,hk", [((1, 4, 8, 16, 16, 128, 64), 2), ((1, 2, 5, 7, 9, 64, 128), 0),
                                     ((1, 4, 6, 8, 8, 64, 128), 1)], ids=["8x16x16-128-64-gqa",
                                                                         "5x7x9-padded-64-128",
                                                                         "6x8x8-padded-64-128-gqa"])
def test_layer_backward_other_value_width(dims, hk):
    """GPU forward (reorder + pool, coarse, fine without gates for O_f and
    LSE) then VsaBackward, against the oracle's vsa_backward."""
    B, nh, T, H, W, d, dv = dims
    _log(f"layer backward {dims} kv heads {hk or nh}")
    p = L.Problem(B, nh, T, H, W, 4, 4, 4, d, heads_kv=hk, head_dim_v=dv)
    hkv = p.kv_heads
    rng = np.random.default_rng(125)
    q = _bf(rng.standard_normal((B, nh, p.n_tokens, d)))
    k = _bf(rng.standard_normal((B, hkv, p.n_tokens, d)))
    v = _bf(rng.standard_normal((B, hkv, p.n_tokens, dv)))
    dout = _bf(rng.standard_normal((B, nh, p.n_tokens, dv)))
    gc, gf = (_bf(rng.random((B, nh, p.n_tokens, dv))) for _ in range(2))
    maxk = 6
    lut = rng.integers(0, p.n_cubes, size=(B, nh, p.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(B, nh, p.n_cubes)).astype(np.int32)
    np_, nc = p.n_positions, p.n_cubes
    bf = torch.bfloat16
    saved = {"qp": torch.empty((B, nh, np_, d), dtype=bf, device="cuda"),
             "kp": torch.empty((B, hkv, np_, d), dtype=bf, device="cuda"),
             "vp": torch.empty((B, hkv, np_, dv), dtype=bf, device="cuda"),
             "qc": torch.empty((B, nh, nc, d), device="cuda"), "oc": torch.empty((B, nh, nc, dv), device="cuda"),
             "kc": torch.empty((B, hkv, nc, d), device="cuda"), "vc": torch.empty((B, hkv, nc, dv), device="cuda"),
             "kv_block_idx": dev(lut), "valid_block_num": dev(valid)}
    L.vsa_permute_pool(p, L.VSA_BF16, dev(q), saved["qp"], saved["qc"])
    L.vsa_permute_pool(p.kv_problem(), L.VSA_BF16, dev(k), saved["kp"], saved["kc"])
    L.vsa_permute_pool(p.v_problem(), L.VSA_BF16, dev(v), saved["vp"], saved["vc"])
    tl = torch.empty((B, nh, nc, 1), dtype=torch.int32, device="cuda")
    tv = torch.empty((B, nh, nc), dtype=torch.int32, device="cuda")
    L.vsa_coarse_topk(p, 1, saved["qc"], saved["kc"], saved["vc"], tl, tv, saved["oc"])
    o_f = torch.empty((B, nh, np_, dv), dtype=bf, device="cuda")
    lse = torch.empty((B, nh, np_), device="cuda")
    L.vsa_sparse_attn_fwd(p, saved["qp"], saved["kp"], saved["vp"], saved["kv_block_idx"],
                          saved["valid_block_num"], o_f, lse=lse)
    dq = torch.full((B, nh, p.n_tokens, d), float("nan"), device="cuda")
    dk = torch.full((B, hkv, p.n_tokens, d), float("nan"), device="cuda")
    dvt = torch.full((B, hkv, p.n_tokens, dv), float("nan"), device="cuda")
    dgc, dgf = (torch.full((B, nh, p.n_tokens, dv), float("nan"), device="cuda") for _ in range(2))
    VsaBackward(p, maxk)(saved, o_f, lse, dev(dout), dq, dk, dvt, gate_c=dev(gc), gate_f=dev(gf),
                         dgate_c=dgc, dgate_f=dgf)
    torch.cuda.synchronize()
    f64 = wl.as_float64
    ref = oracle.vsa_backward(f64(q), f64(k), f64(v), (T, H, W), (4, 4, 4), lut, valid, f64(dout),
                              gate_c=f64(gc), gate_f=f64(gf))
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dvt), ("dgate_c", dgc), ("dgate_f", dgf)):
        _grad_check(nm, t, ref[nm])
