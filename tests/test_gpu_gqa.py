"""GPU parity with grouped key/value heads (heads_kv < heads; reading R19:
query head h uses key/value head h // G).  Same bars as the plain-head
tests: Top-K sets tie-tolerant, O_c within 1e-4, attention outputs max-abs
2e-2 / mean-abs 2e-3, gradients max 2% of max |grad| / mean 1% of mean
|grad|.  The oracle repeats each key/value head G times."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward
from gpu_helpers import (OC_MAX_ABS, assert_out_close, check_lut_against_scores, dev, err, host64, inputs)

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


def _gqa_inputs(w, hk):
    x = inputs(w.name)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    qp = np.take(x["q"], pi, axis=2)
    kp = np.ascontiguousarray(np.take(x["k"], pi, axis=2)[:, :hk])
    vp = np.ascontiguousarray(np.take(x["v"], pi, axis=2)[:, :hk])
    return x, pi, qp, kp, vp


@pytest.mark.parametrize("hk", [2, 1])
def test_coarse_topk_grouped(hk):
    w = wl.SMALL
    _log(f"coarse_topk heads 4, kv heads {hk}")
    p = L.Problem(1, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, heads_kv=hk)
    _, _, qp, kp, vp = _gqa_inputs(w, hk)
    qc, kc, vc = (oracle.pool(wl.as_float64(a), 64).astype(np.float32) for a in (qp, kp, vp))
    lut = torch.empty((1, w.heads, w.n_cubes, w.top_k), dtype=torch.int32, device="cuda")
    valid = torch.empty((1, w.heads, w.n_cubes), dtype=torch.int32, device="cuda")
    oc = torch.empty((1, w.heads, w.n_cubes, w.head_dim), device="cuda")
    L.vsa_coarse_topk(p, w.top_k, dev(qc), dev(kc), dev(vc), lut, valid, oc)
    torch.cuda.synchronize()
    g = w.heads // hk
    s, _, oc_want = oracle.coarse_attention(qc.astype(np.float64), oracle.expand_kv_heads(kc, g).astype(np.float64),
                                            oracle.expand_kv_heads(vc, g).astype(np.float64), 1 / math.sqrt(w.head_dim))
    lut_want, _ = oracle.topk_lut(s, w.top_k)
    check_lut_against_scores(lut.cpu().numpy(), valid.cpu().numpy(), s, w.top_k, lut_want)
    assert err(host64(oc), oc_want)[0] <= OC_MAX_ABS


@pytest.mark.parametrize("name,hk,heads_checked", [("small", 2, None), ("small", 1, None), ("wan", 4, [0, 5, 11])])
def test_sparse_attn_fwd_grouped(name, hk, heads_checked):
    w = wl.WORKLOADS[name]
    _log(f"sparse_attn_fwd {name} kv heads {hk}")
    p = L.Problem(1, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, heads_kv=hk)
    _, _, qp, kp, vp = _gqa_inputs(w, hk)
    rng = np.random.default_rng(111)
    lut = np.stack([np.sort(rng.permutation(w.n_cubes)[:w.top_k])
                    for _ in range(w.heads * w.n_cubes)]).reshape(1, w.heads, w.n_cubes, w.top_k).astype(np.int32)
    valid = np.full((1, w.heads, w.n_cubes), w.top_k, np.int32)
    out = torch.empty((1, w.heads, w.n_tokens, w.head_dim), dtype=torch.bfloat16, device="cuda")
    L.vsa_sparse_attn_fwd(p, dev(qp), dev(kp), dev(vp), dev(lut), dev(valid), out)
    torch.cuda.synchronize()
    g = w.heads // hk
    hs = list(range(w.heads)) if heads_checked is None else heads_checked
    cubes = range(w.n_cubes) if heads_checked is None else sorted({0, 1, 255, w.n_cubes - 1})
    q64 = wl.as_float64(qp)[:, hs]
    k64 = oracle.expand_kv_heads(wl.as_float64(kp), g)[:, hs]
    v64 = oracle.expand_kv_heads(wl.as_float64(vp), g)[:, hs]
    todo = [(0, hi, i) for hi in range(len(hs)) for i in cubes]
    of, _ = oracle.fine_attention(q64, k64, v64, lut[:, hs], valid[:, hs], 1 / math.sqrt(w.head_dim), 64,
                                  query_cubes=todo)
    rows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in cubes])
    assert_out_close(host64(out)[:, hs][:, :, rows], of[:, :, rows], f"fine {name} kv {hk}")


def test_sparse_attn_bwd_grouped_wan():
    """The 32K-token layer with 12 query heads on 4 key/value heads: dK and
    dV of a key cube sum over the 3 query heads of its group."""
    w = wl.WAN
    hk, g = 4, 3
    _log("sparse_attn_bwd wan kv heads 4 (sampled)")
    p = L.Problem(1, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, heads_kv=hk)
    _, _, qp, kp, vp = _gqa_inputs(w, hk)
    k = w.top_k
    rng = np.random.default_rng(112)
    lut = np.stack([np.sort(rng.permutation(w.n_cubes)[:k])
                    for _ in range(w.heads * w.n_cubes)]).reshape(1, w.heads, w.n_cubes, k).astype(np.int32)
    valid = np.full((1, w.heads, w.n_cubes), k, np.int32)
    scale = 1 / math.sqrt(w.head_dim)
    kvh, kcube = 1, 7                            # key cube 7 of key/value head 1 = query heads 3, 4, 5
    heads = [3, 4, 5]
    need = {h: sorted({0, 300} | {i for i in range(w.n_cubes) if kcube in lut[0, h, i, :k]}) for h in heads}
    q64 = wl.as_float64(qp)
    ke, ve = (oracle.expand_kv_heads(wl.as_float64(a), g) for a in (kp, vp))
    todo = [(0, h, i) for h in heads for i in need[h]]
    of, lse = oracle.fine_attention(q64, ke, ve, lut, valid, scale, 64, query_cubes=todo)
    fill = np.ones((1, w.heads, w.n_cubes), bool)
    for h in heads:
        fill[0, h, need[h]] = False
    ft = np.repeat(fill, 64, axis=-1)
    of[ft] = rng.standard_normal((int(ft.sum()), w.head_dim)) * 0.1
    lse[ft] = 8.0
    of_bits = wl.f32_to_bf16_bits(of.astype(np.float32))
    lse32 = lse.astype(np.float32)
    dof_bits = wl.f32_to_bf16_bits(rng.standard_normal(qp.shape).astype(np.float32))
    ts = (1, w.heads, w.n_tokens, w.head_dim)
    kts = (1, hk, w.n_tokens, w.head_dim)
    dq = torch.empty(ts, device="cuda")
    dk, dv = torch.empty(kts, device="cuda"), torch.empty(kts, device="cuda")
    ws = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(p, k), dtype=torch.uint8, device="cuda")
    L.vsa_sparse_attn_bwd(p, dev(qp), dev(kp), dev(vp), dev(lut), dev(valid), dev(of_bits), dev(lse32),
                          dev(dof_bits), dq, dk, dv, ws)
    torch.cuda.synchronize()
    sub = np.zeros((1, w.heads, w.n_cubes), np.int32)
    for h in heads:
        sub[0, h, need[h]] = k
    hsl = slice(3, 6)
    ref = oracle.fine_attention_bwd(q64[:, hsl], ke[:, hsl], ve[:, hsl], lut[:, hsl], sub[:, hsl], scale, 64,
                                    wl.as_float64(of_bits)[:, hsl], lse32[:, hsl].astype(np.float64),
                                    wl.as_float64(dof_bits)[:, hsl])
    krows = np.arange(kcube * 64, kcube * 64 + 64)
    dk_want = ref[1][0][:, krows].sum(axis=0)    # sum over the group's 3 query heads
    dv_want = ref[2][0][:, krows].sum(axis=0)
    for name, got, want in (("dk", host64(dk)[0, kvh, krows], dk_want), ("dv", host64(dv)[0, kvh, krows], dv_want)):
        e = np.abs(got - want)
        print(f"{name}: max {e.max() / np.abs(want).max():.2e} of max, mean {e.mean() / np.abs(want).mean():.2e}")
        assert e.max() <= 2e-2 * np.abs(want).max() and e.mean() <= 1e-2 * np.abs(want).mean(), name
    qrows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in (0, 300)])
    for hi, h in enumerate(heads):
        got, want = host64(dq)[0, h, qrows], ref[0][0, hi, qrows]
        e = np.abs(got - want)
        assert e.max() <= 2e-2 * np.abs(want).max() and e.mean() <= 1e-2 * np.abs(want).mean(), f"dq h{h}"


@pytest.mark.parametrize("hk", [2, 1])
def test_layer_backward_grouped(hk):
    w = wl.SMALL
    _log(f"layer backward small kv heads {hk}")
    p = L.Problem(1, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, heads_kv=hk)
    pkv = p.kv_problem()
    x = inputs(w.name)
    rng = np.random.default_rng(113)
    maxk = 10
    lut = rng.integers(0, w.n_cubes, size=(1, w.heads, w.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(1, maxk + 1, size=(1, w.heads, w.n_cubes)).astype(np.int32)
    dout = wl.f32_to_bf16_bits(rng.standard_normal((1, w.heads, w.n_tokens, w.head_dim)).astype(np.float32))
    kx, vx = (np.ascontiguousarray(x[n][:, :hk]) for n in ("k", "v"))
    q, k, v = dev(x["q"]), dev(kx), dev(vx)
    ts, cs = (1, w.heads, w.n_tokens, w.head_dim), (1, w.heads, w.n_cubes, w.head_dim)
    kts, kcs = (1, hk, w.n_tokens, w.head_dim), (1, hk, w.n_cubes, w.head_dim)
    saved = {"qp": torch.empty(ts, dtype=torch.bfloat16, device="cuda"),
             "kp": torch.empty(kts, dtype=torch.bfloat16, device="cuda"),
             "vp": torch.empty(kts, dtype=torch.bfloat16, device="cuda"),
             "qc": torch.empty(cs, device="cuda"), "oc": torch.empty(cs, device="cuda"),
             "kc": torch.empty(kcs, device="cuda"), "vc": torch.empty(kcs, device="cuda"),
             "kv_block_idx": dev(lut), "valid_block_num": dev(valid)}
    L.vsa_permute_pool(p, L.VSA_BF16, q, saved["qp"], saved["qc"])
    L.vsa_permute_pool(pkv, L.VSA_BF16, k, saved["kp"], saved["kc"])
    L.vsa_permute_pool(pkv, L.VSA_BF16, v, saved["vp"], saved["vc"])
    tl = torch.empty((1, w.heads, w.n_cubes, 1), dtype=torch.int32, device="cuda")
    tv = torch.empty((1, w.heads, w.n_cubes), dtype=torch.int32, device="cuda")
    L.vsa_coarse_topk(p, 1, saved["qc"], saved["kc"], saved["vc"], tl, tv, saved["oc"])
    o_f = torch.empty(ts, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, w.heads, w.n_tokens), device="cuda")
    L.vsa_sparse_attn_fwd(p, saved["qp"], saved["kp"], saved["vp"], saved["kv_block_idx"],
                          saved["valid_block_num"], o_f, lse=lse)
    dq = torch.empty(ts, device="cuda")
    dk, dv = torch.empty(kts, device="cuda"), torch.empty(kts, device="cuda")
    dgc, dgf = torch.empty(ts, device="cuda"), torch.empty(ts, device="cuda")
    VsaBackward(p, maxk)(saved, o_f, lse, dev(dout), dq, dk, dv, gate_c=dev(x["gate_c"]), gate_f=dev(x["gate_f"]),
                         dgate_c=dgc, dgate_f=dgf)
    torch.cuda.synchronize()
    f64 = wl.as_float64
    ref = oracle.vsa_backward(f64(x["q"]), f64(kx), f64(vx), (w.T, w.H, w.W), w.cube, lut, valid, f64(dout),
                              gate_c=f64(x["gate_c"]), gate_f=f64(x["gate_f"]))
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dgate_c", dgc), ("dgate_f", dgf)):
        g_, r_ = host64(t), ref[nm]
        e = np.abs(g_ - r_)
        mx, mn = e.max() / np.abs(r_).max(), e.mean() / np.abs(r_).mean()
        print(f"{nm}: max {mx:.2e} of max, mean {mn:.2e} of mean")
        assert mx <= 2e-2 and mn <= 1e-2, nm
