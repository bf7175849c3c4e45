"""GPU checks of vsa_attention, the differentiable layer (VsaAttentionFunction).

* Its output equals the hand-sequenced training forward (the fine stage
  without gates, then vsa_combine) bit for bit, and VsaForward's fused
  epilogue within the one extra bf16 rounding of O_f (bit for bit without
  gates).
* Its gradients equal a hand-sequenced VsaBackward on the same forward
  intermediates bit for bit (after the cast to the inputs' bf16 dtype that
  autograd applies), for plain, grouped-head and padded problems.
* Against the fp64 oracle's whole-layer backward on the LUT the GPU chose,
  within the whole-layer bar of tests/test_gpu_layer_bwd.py (max 2% of max
  |grad|, mean 1% of mean |grad|).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward, VsaForward, vsa_attention
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


def _manual(p, top_k, q, k, v, gc, gf, dout):
    """The same layer sequenced by hand: VsaForward (its fused output, and the
    intermediates), the cube-major fine pass for O_f and LSE, vsa_combine for
    the training output, then VsaBackward."""
    f = VsaForward(p, top_k)
    fused = q.new_empty(q.shape[:-1] + (p.v_dim,))
    f(q, k, v, fused, gc, gf)
    o_f = torch.empty((p.batch, p.heads, p.n_positions, p.v_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((p.batch, p.heads, p.n_positions), dtype=torch.float32, device="cuda")
    L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse=lse)
    out = torch.empty_like(fused)
    L.vsa_combine(p, o_f, out, oc=f.oc if gc is not None else None, gate_c=gc, gate_f=gf)
    f32 = torch.float32
    dq = torch.empty((p.batch, p.heads, p.n_tokens, p.head_dim), dtype=f32, device="cuda")
    dk = torch.empty((p.batch, p.kv_heads, p.n_tokens, p.head_dim), dtype=f32, device="cuda")
    dv = torch.empty((p.batch, p.kv_heads, p.n_tokens, p.v_dim), dtype=f32, device="cuda")
    gs = (p.batch, p.heads, p.n_tokens, p.v_dim)
    dgc = torch.empty(gs, dtype=f32, device="cuda") if gc is not None else None
    dgf = torch.empty(gs, dtype=f32, device="cuda") if gf is not None else None
    VsaBackward(p, top_k)(f.intermediates(), o_f, lse, dout, dq, dk, dv, gate_c=gc, gate_f=gf,
                          dgate_c=dgc, dgate_f=dgf)
    return out, fused, (dq, dk, dv, dgc, dgf)


def _inputs(p, seed, gates):
    g = torch.Generator(device="cuda").manual_seed(seed)
    def draw(heads, d):
        return torch.randn((p.batch, heads, p.n_tokens, d), generator=g, device="cuda").to(torch.bfloat16)
    q, k, v = draw(p.heads, p.head_dim), draw(p.kv_heads, p.head_dim), draw(p.kv_heads, p.v_dim)
    gc = gf = None
    if gates:
        gc = torch.rand((p.batch, p.heads, p.n_tokens, p.v_dim), generator=g, device="cuda").to(torch.bfloat16)
        gf = torch.rand((p.batch, p.heads, p.n_tokens, p.v_dim), generator=g, device="cuda").to(torch.bfloat16)
    dout = torch.randn((p.batch, p.heads, p.n_tokens, p.v_dim), generator=g, device="cuda").to(torch.bfloat16)
    return q, k, v, gc, gf, dout


CASES = [
    ("small", dict(), 8, True),
    ("small", dict(), 8, False),
    ("small-gqa", dict(heads_kv=2), 6, True),
    ("padded-5x7x9", dict(T=5, H=7, W=9, heads=2), 3, True),
]


@pytest.mark.parametrize("name,repl,top_k,gates", CASES, ids=[f"{c[0]}-g{int(c[3])}" for c in CASES])
def test_autograd_matches_hand_sequenced_layer(name, repl, top_k, gates):
    _log(f"vsa_attention {name} gates={gates}")
    p = dataclasses.replace(problem(wl.SMALL), **repl)
    q, k, v, gc, gf, dout = _inputs(p, 7, gates)
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v)]
    gleaves = [t.clone().requires_grad_(True) if t is not None else None for t in (gc, gf)]
    out = vsa_attention(*leaves, p, top_k, gate_c=gleaves[0], gate_f=gleaves[1])
    out.backward(dout)
    torch.cuda.synchronize()
    want_out, fused, want_grads = _manual(p, top_k, q, k, v, gc, gf, dout)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out.detach()), bits(want_out)), "output"
    if not gates:
        assert np.array_equal(bits(out.detach()), bits(fused)), "output without gates"
    else:
        # one more rounding of O_f to bf16 (relative 2^-9, times g_f <= 1) and
        # possibly one bf16 ulp (2^-8) of the result apart
        a, b = host64(out.detach()), host64(fused)
        assert np.all(np.abs(a - b) <= 2 ** -7 * np.abs(b) + 2 ** -9 * np.abs(b).max()), "output vs fused"
    got = [t.grad for t in leaves] + [t.grad if t is not None else None for t in gleaves]
    for nm, g, w in zip(("dq", "dk", "dv", "dgate_c", "dgate_f"), got, want_grads):
        if w is None:
            assert g is None, nm
            continue
        assert g.dtype == torch.bfloat16, nm
        assert np.array_equal(bits(g), bits(w.to(torch.bfloat16))), nm


def test_autograd_against_oracle():
    """The small workload's seeded inputs, gates and a seeded upstream
    gradient: the gradients of vsa_attention against the oracle's layer
    backward on the LUT the GPU selected."""
    _log("vsa_attention small vs oracle")
    w = wl.SMALL
    p = problem(w)
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]).requires_grad_(True) for n in ("q", "k", "v", "gate_c", "gate_f"))
    rng = np.random.default_rng(91)
    dout_bits = wl.f32_to_bf16_bits(rng.standard_normal((1, w.heads, w.n_tokens, w.head_dim)).astype(np.float32))
    out = vsa_attention(q, k, v, p, w.top_k, gate_c=gc, gate_f=gf)
    out.backward(dev(dout_bits))
    torch.cuda.synchronize()
    # the LUT the GPU chose (a Top-K selection has no gradient; the oracle uses the same one)
    f = VsaForward(p, w.top_k)
    f(dev(x["q"]), dev(x["k"]), dev(x["v"]), torch.empty_like(q.detach()), dev(x["gate_c"]), dev(x["gate_f"]))
    torch.cuda.synchronize()
    lut, valid = f.lut.cpu().numpy(), f.valid.cpu().numpy()
    f64 = wl.as_float64
    ref = oracle.vsa_backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), (w.T, w.H, w.W), w.cube, lut, valid,
                              f64(dout_bits), gate_c=f64(x["gate_c"]), gate_f=f64(x["gate_f"]))
    for nm, t in zip(("dq", "dk", "dv", "dgate_c", "dgate_f"), (q, k, v, gc, gf)):
        g, r = host64(t.grad), ref[nm]
        e = np.abs(g - r)
        mx = e.max() / np.abs(r).max()
        mn = e.mean() / np.abs(r).mean()
        print(f"{nm}: max {mx:.2e} of max, mean {mn:.2e} of mean")
        # the gradients come back in bf16 (the inputs' dtype): half an ulp,
        # 2^-9 of each value, on top of the whole-layer bar
        assert mx <= 2e-2 + 2 ** -9 and mn <= 1e-2 + 2 ** -9, nm
