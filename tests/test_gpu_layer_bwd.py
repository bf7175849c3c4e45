"""GPU parity of the backward of the remaining steps (vsa_combine_bwd,
vsa_coarse_bwd, vsa_pool_unpermute_bwd) and of a whole layer (VsaBackward)
against the fp64 oracle.

Bars (from the arithmetic):
* combine: d_of is the bf16 rounding of an exact product of two bf16 values,
  dg_f and dg_c single float32 roundings of exact products: all bit-exact
  against the fp64 products rounded the same way.  d_oc sums 64 exact
  float32 products in float32: within 64 * 2^-24 * sum|terms|.
* coarse: float32 throughout, sums over Nc cubes: max error 1e-4 of max |grad|.
* pool + reorder backward: x + y / vol in float32, at most two roundings:
  within 2^-22 * (|x| + |y| / vol); bit-exact when vol is a power of two.
* whole layer: the fine-stage bar (max 2% of max |grad|, mean 1% of mean
  |grad|, five times the bf16 operand rounding); the GPU forward's O_f is
  bf16, so the gate gradient dg_f = dout * O_f carries that rounding too.
Nothing the oracle sees comes from the GPU: Q, K, V, gates and dout are
seeded draws, the LUT a seeded random list.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward
from gpu_helpers import bits, dev, host64, inputs, problem

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


def _rel_check(name, got, ref, max_rel, mean_rel):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    e = np.abs(g - r)
    mx = e.max() / max(np.abs(r).max(), 1e-30)
    mn = e.mean() / max(np.abs(r).mean(), 1e-30)
    print(f"{name}: max {mx:.2e} of max, mean {mn:.2e} of mean")
    assert mx <= max_rel and mn <= mean_rel, name


@pytest.mark.parametrize("name,gates", [("small", True), ("small", False), ("wan", True)])
def test_combine_bwd(name, gates):
    w = wl.WORKLOADS[name]
    _log(f"combine_bwd {name} gates={gates}")
    p = problem(w)
    rng = np.random.default_rng(81)
    ts = (1, w.heads, w.n_tokens, w.head_dim)
    cs = (1, w.heads, w.n_cubes, w.head_dim)
    dout, of = _bf(rng.standard_normal(ts)), _bf(rng.standard_normal(ts))
    oc = rng.standard_normal(cs).astype(np.float32)
    x = inputs(name)
    gc, gf = (x["gate_c"], x["gate_f"]) if gates else (None, None)
    d_of = torch.empty(ts, dtype=torch.bfloat16, device="cuda")
    d_oc = torch.full(cs, float("nan"), device="cuda")
    dgc = torch.full(ts, float("nan"), device="cuda") if gates else None
    dgf = torch.full(ts, float("nan"), device="cuda") if gates else None
    L.vsa_combine_bwd(p, dev(dout), d_of, d_oc, o_f=dev(of), oc=dev(oc),
                      gate_c=dev(gc) if gates else None, gate_f=dev(gf) if gates else None,
                      d_gate_c=dgc, d_gate_f=dgf)
    torch.cuda.synchronize()
    f64 = wl.as_float64
    r_of, r_oc, r_gc, r_gf = oracle.combine_bwd(f64(dout), f64(of), oc, 64, f64(gc) if gates else None,
                                                f64(gf) if gates else None)
    assert np.array_equal(bits(d_of), _bf(r_of)), "d_of not the RNE of g_f * dout"
    if gates:
        assert np.array_equal(bits(dgf), r_gf.astype(np.float32).view(np.uint32)), "dg_f"
        assert np.array_equal(bits(dgc), r_gc.astype(np.float32).view(np.uint32)), "dg_c"
        terms = np.abs(f64(gc) * f64(dout)).reshape(1, w.heads, w.n_cubes, 64, w.head_dim).sum(axis=3)
        assert np.all(np.abs(host64(d_oc) - r_oc) <= 64 * 2.0 ** -24 * terms + 1e-30)
    else:
        assert np.all(host64(d_oc) == 0.0)


COARSE = [("small", 4), ("wan", 12), ("large", 2)]


@pytest.mark.parametrize("name,heads", COARSE)
def test_coarse_bwd(name, heads):
    """Pooled-like float32 inputs of the workload's cube count; the large
    grid (1920 cubes) takes the 4-row path, the others the 8-row path."""
    w = wl.WORKLOADS[name]
    _log(f"coarse_bwd {name} heads={heads}")
    p = L.Problem(1, heads, w.T, w.H, w.W, *w.cube, w.head_dim)
    rng = np.random.default_rng(82)
    cs = (1, heads, w.n_cubes, w.head_dim)
    qc, kc, vc, doc = (rng.standard_normal(cs).astype(np.float32) for _ in range(4))
    qc *= 0.5
    scale = 1 / math.sqrt(w.head_dim)
    _, _, oc = oracle.coarse_attention(qc, kc, vc, scale)
    oc32 = oc.astype(np.float32)
    outs = [torch.full(cs, float("nan"), device="cuda") for _ in range(3)]
    ws = torch.full((L.vsa_coarse_bwd_workspace_size(p),), 0xA5, dtype=torch.uint8, device="cuda")
    L.vsa_coarse_bwd(p, dev(qc), dev(kc), dev(vc), dev(oc32), dev(doc), *outs, ws)
    torch.cuda.synchronize()
    ref = oracle.coarse_attention_bwd(qc, kc, vc, scale, doc)
    for nm, g, r in zip(("dqc", "dkc", "dvc"), outs, ref):
        _rel_check(f"{name} {nm}", host64(g), r, 1e-4, 1e-4)


@pytest.mark.parametrize("dims", [(1, 4, 8, 16, 16, 4, 4, 4, 64), (1, 12, 16, 32, 64, 4, 4, 4, 128),
                                  (2, 3, 2, 4, 6, 2, 2, 2, 64), (1, 2, 3, 6, 4, 3, 2, 1, 128)])
def test_pool_unpermute_bwd(dims):
    B, nh, T, H, W, ct, ch, cw, d = dims
    _log(f"pool_unpermute_bwd {dims}")
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d)
    vol = ct * ch * cw
    rng = np.random.default_rng(83)
    xs = (B, nh, T * H * W, d)
    dx = rng.standard_normal(xs).astype(np.float32)
    dxc = rng.standard_normal((B, nh, T * H * W // vol, d)).astype(np.float32)
    out = torch.full(xs, float("nan"), device="cuda")
    L.vsa_pool_unpermute_bwd(p, dev(dx), dev(dxc), out)
    out2 = torch.full(xs, float("nan"), device="cuda")
    L.vsa_pool_unpermute_bwd(p, dev(dx), None, out2)
    torch.cuda.synchronize()
    pi = oracle.perm_index(T, H, W, ct, ch, cw)
    want = oracle.unpermute(dx.astype(np.float64) + oracle.pool_bwd(dxc, vol), pi)
    bound = 2.0 ** -22 * oracle.unpermute(np.abs(dx) + np.abs(oracle.pool_bwd(dxc, vol)), pi)
    assert np.all(np.abs(host64(out) - want) <= bound)
    if vol & (vol - 1) == 0:
        assert np.array_equal(bits(out), want.astype(np.float32).view(np.uint32))
    assert np.array_equal(bits(out2), oracle.unpermute(dx, pi).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("gates", [True, False])
def test_layer_backward(gates):
    """Whole layer on the small workload: GPU forward (reorder + pool, coarse,
    fine without gates for O_f and LSE) then VsaBackward, against the
    oracle's vsa_backward on the same seeded inputs and LUT."""
    w = wl.SMALL
    _log(f"layer backward small gates={gates}")
    p = problem(w)
    x = inputs(w.name)
    rng = np.random.default_rng(84)
    maxk = 10
    lut = rng.integers(0, w.n_cubes, size=(1, w.heads, w.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(1, w.heads, w.n_cubes)).astype(np.int32)
    valid[0, 0, :3] = 0
    dout = _bf(rng.standard_normal((1, w.heads, w.n_tokens, w.head_dim)))
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    ts, cs = (1, w.heads, w.n_tokens, w.head_dim), (1, w.heads, w.n_cubes, w.head_dim)
    saved = {n: torch.empty(ts, dtype=torch.bfloat16, device="cuda") for n in ("qp", "kp", "vp")}
    saved.update({n: torch.empty(cs, device="cuda") for n in ("qc", "kc", "vc", "oc")})
    saved["kv_block_idx"], saved["valid_block_num"] = dev(lut), dev(valid)
    for t, a, c in ((q, "qp", "qc"), (k, "kp", "kc"), (v, "vp", "vc")):
        L.vsa_permute_pool(p, L.VSA_BF16, t, saved[a], saved[c])
    tmp_lut = torch.empty((1, w.heads, w.n_cubes, 1), dtype=torch.int32, device="cuda")
    tmp_valid = torch.empty((1, w.heads, w.n_cubes), dtype=torch.int32, device="cuda")
    L.vsa_coarse_topk(p, 1, saved["qc"], saved["kc"], saved["vc"], tmp_lut, tmp_valid, saved["oc"])
    o_f = torch.empty(ts, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, w.heads, w.n_tokens), device="cuda")
    L.vsa_sparse_attn_fwd(p, saved["qp"], saved["kp"], saved["vp"], saved["kv_block_idx"],
                          saved["valid_block_num"], o_f, lse=lse)
    grads = [torch.full(ts, float("nan"), device="cuda") for _ in range(5)]
    bw = VsaBackward(p, maxk)
    gc, gf = (dev(x["gate_c"]), dev(x["gate_f"])) if gates else (None, None)
    bw(saved, o_f, lse, dev(dout), *grads[:3], gate_c=gc, gate_f=gf,
       dgate_c=grads[3] if gates else None, dgate_f=grads[4] if gates else None)
    torch.cuda.synchronize()
    f64 = wl.as_float64
    ref = oracle.vsa_backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), (w.T, w.H, w.W), w.cube, lut, valid,
                              f64(dout), gate_c=f64(x["gate_c"]) if gates else None,
                              gate_f=f64(x["gate_f"]) if gates else None)
    names = ("dq", "dk", "dv", "dgate_c", "dgate_f") if gates else ("dq", "dk", "dv")
    for nm, g in zip(names, grads):
        _rel_check(f"layer {nm}", host64(g), ref[nm], 2e-2, 1e-2)
