"""GPU parity of the fine stage that gathers its cube tiles from raster-order
Q, K, V (vsa_sparse_attn_fwd_gather) and of the pool on its own from raster
rows (vsa_permute_pool with no cube-major output).

* against the fp64 oracle, element by element on the checked query cubes
  (the bars of tests/gpu_helpers.py), with Q, K, V, the gates, the output
  and the LSE all in raster token order;
* bit for bit against vsa_permute of Q, K, V followed by
  vsa_sparse_attn_fwd_raster wherever that path runs the same pair kernel
  (rows listing fewer than half of the cubes): the gathered tiles land in
  LDS exactly as the reordered copies' tiles do;
* the pool from raster rows against vsa_permute_pool's pooled output, bit
  for bit, in both raster layouts and on a padded grid;
* the shapes the gathering loads do not cover are refused.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from gpu_helpers import LSE_MAX_ABS, assert_out_close, bits, dev, err, host64, inputs, problem

pytestmark = pytest.mark.gpu

# a d = 128 layer small enough for the oracle on every query cube: grid
# 8x16x16 (2,048 tokens, 32 cubes), 2 heads, locality-structured Q/K
G128 = wl.Workload("g128", 8, 16, 16, (4, 4, 4), 1, 2, 128, "bf16", 8, 21, 4)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(f"\n[case] {msg}", flush=True)


_G128_INPUTS = {}


def _inputs(w):
    if w.name == "g128":
        if "x" not in _G128_INPUTS:
            _G128_INPUTS["x"] = wl.make_inputs(G128, with_gates=True, workers=4)
        return _G128_INPUTS["x"]
    return inputs(w.name)


def _pooled_oracle(w, x, hs):
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    return {n: oracle.pool(wl.as_float64(np.take(x[n][:, hs], pi, axis=2)), w.cube_volume)
            for n in ("q", "k", "v")}


def _gather_case(w, k, cubes, heads_checked=None):
    """Gathering fine stage on raster inputs with the oracle's LUT and O_c for
    the checked heads (a seeded random LUT elsewhere); checks the raster
    output and LSE of the checked query cubes against the oracle."""
    p = problem(w)
    x = _inputs(w)
    vol = w.cube_volume
    hs = list(range(w.heads)) if heads_checked is None else list(heads_checked)
    scale = 1.0 / math.sqrt(w.head_dim)
    pooled = _pooled_oracle(w, x, hs)
    s, _, oc_h = oracle.coarse_attention(pooled["q"], pooled["k"], pooled["v"], scale)
    lut_h, valid_h = oracle.topk_lut(s, k)
    rng = np.random.default_rng(12)
    lut = np.empty((p.batch, p.heads, p.n_cubes, k), np.int32)
    for idx in np.ndindex(p.batch, p.heads, p.n_cubes):
        lut[idx] = np.sort(rng.permutation(p.n_cubes)[:k])
    lut[:, hs] = lut_h
    valid = np.full((p.batch, p.heads, p.n_cubes), k, np.int32)
    oc = rng.standard_normal((p.batch, p.heads, p.n_cubes, p.head_dim)).astype(np.float32)
    oc[:, hs] = oc_h.astype(np.float32)
    q, kk, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((p.batch, p.heads, p.n_tokens), float("nan"), device="cuda")
    L.vsa_sparse_attn_fwd_gather(p, q, kk, v, dev(lut), dev(valid), out, oc=dev(oc), gate_c=gc, gate_f=gf, lse=lse)
    torch.cuda.synchronize()
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    got = np.take(host64(out), pi, axis=2)       # cube-major view of the raster output
    got_lse = np.take(host64(lse), pi, axis=2)
    assert np.all(np.isfinite(got)), "output has non-finite values"
    xp = {n: np.take(x[n][:, hs], pi, axis=2) for n in ("q", "k", "v", "gate_c", "gate_f")}
    qcs = [(0, hi, i) for hi in range(len(hs)) for i in cubes]
    q64, k64, v64 = (wl.as_float64(xp[n]) for n in ("q", "k", "v"))
    of, lse_w = oracle.fine_attention(q64, k64, v64, lut_h, valid_h, scale, vol, query_cubes=qcs)
    want = oracle.combine(of, oc_h.astype(np.float32).astype(np.float64), vol,
                          wl.as_float64(xp["gate_c"]), wl.as_float64(xp["gate_f"]))
    rows = np.concatenate([np.arange(i * vol, (i + 1) * vol) for i in cubes])
    res = assert_out_close(got[:, hs][:, :, rows], want[:, :, rows], f"gather {w.name} K={k}")
    le = err(got_lse[:, hs][:, :, rows], lse_w[:, :, rows])
    assert le[0] <= LSE_MAX_ABS, f"lse max-abs {le[0]:.3e}"
    return res


def _sampled(w):
    rng = np.random.default_rng(7)
    return sorted(set(rng.choice(w.n_cubes, size=min(w.n_cubes, 24), replace=False).tolist())
                  | {0, w.n_cubes - 1})


GATHER = [("g128", 8, None, None), ("g128", 1, None, None), ("g128", 32, None, None),
          ("wan", 154, "sampled", [0, 5]), ("wan", 300, "sampled", [9]), ("large", 192, "sampled", [0])]


@pytest.mark.parametrize("name,k,cubes,heads", GATHER, ids=[f"{g[0]}-k{g[1]}" for g in GATHER])
def test_gather_against_oracle(name, k, cubes, heads):
    w = G128 if name == "g128" else wl.WORKLOADS[name]
    _log(f"sparse_attn_fwd_gather {name} K={k}")
    cs = list(range(w.n_cubes)) if cubes is None else _sampled(w)
    mx, mean = _gather_case(w, k, cs, heads_checked=heads)
    print(f"max-abs {mx:.3e} mean-abs {mean:.3e}")


def _both_paths(p, q, k, v, lut, valid, oc=None, gc=None, gf=None, with_lse=True):
    """(gathered out, lse), (reorder + raster entry point out, lse)."""
    kvp = p.kv_problem()
    qp = torch.empty((p.batch, p.heads, p.n_positions, p.head_dim), dtype=torch.bfloat16, device="cuda")
    kp = torch.empty((p.batch, p.kv_heads, p.n_positions, p.head_dim), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    L.vsa_permute(p, L.VSA_BF16, q, qp)
    L.vsa_permute(kvp, L.VSA_BF16, k, kp)
    L.vsa_permute(kvp, L.VSA_BF16, v, vp)
    res = []
    for fn, args in ((L.vsa_sparse_attn_fwd_gather, (q, k, v)), (L.vsa_sparse_attn_fwd_raster, (qp, kp, vp))):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((p.batch, p.heads, p.n_tokens), float("nan"), device="cuda") if with_lse else None
        fn(p, *args, lut, valid, out, oc=oc, gate_c=gc, gate_f=gf, lse=lse)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


def _coarse(p, q, k, v, top_k):
    kvp = p.kv_problem()
    qc = torch.empty((p.batch, p.heads, p.n_cubes, p.head_dim), device="cuda")
    kc = torch.empty((p.batch, p.kv_heads, p.n_cubes, p.head_dim), device="cuda")
    vc = torch.empty_like(kc)
    L.vsa_permute_pool(p, L.VSA_BF16, q, None, qc)
    L.vsa_permute_pool(kvp, L.VSA_BF16, k, None, kc)
    L.vsa_permute_pool(kvp, L.VSA_BF16, v, None, vc)
    lut = torch.empty((p.batch, p.heads, p.n_cubes, top_k), dtype=torch.int32, device="cuda")
    valid = torch.empty((p.batch, p.heads, p.n_cubes), dtype=torch.int32, device="cuda")
    oc = torch.empty_like(qc)
    L.vsa_coarse_topk(p, top_k, qc, kc, vc, lut, valid, oc)
    return lut, valid, oc


@pytest.mark.parametrize("order,heads_kv,top_k", [("raster", 0, 154), ("raster", 0, 51), ("hilbert", 0, 154),
                                                  ("raster", 4, 154)],
                         ids=["raster-k154", "raster-k51", "hilbert-k154", "gqa4-k154"])
def test_gather_bit_equal_to_reorder_then_raster(order, heads_kv, top_k):
    """The 32K-token layer: the gathered path writes exactly the bits of the
    reorder followed by the raster-output entry point (gates, O_c and LSE)."""
    _log(f"gather vs reorder+raster, {order} cubes, kv heads {heads_kv or 12}, K={top_k}")
    w = wl.WAN
    p = L.Problem(w.batch, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, heads_kv=heads_kv, cube_order=order)
    x = inputs("wan")
    q, gc, gf = (dev(x[n]) for n in ("q", "gate_c", "gate_f"))
    k, v = dev(x["k"]), dev(x["v"])
    if heads_kv:
        k, v = k[:, :heads_kv].contiguous(), v[:, :heads_kv].contiguous()
    lut, valid, oc = _coarse(p, q, k, v, top_k)
    (og, lg), (orf, lr) = _both_paths(p, q, k, v, lut, valid, oc=oc, gc=gc, gf=gf)
    assert np.all(np.isfinite(host64(og)))
    assert np.array_equal(bits(og), bits(orf)), "outputs differ"
    assert np.array_equal(bits(lg), bits(lr)), "lse differs"


def test_gather_variable_rows_duplicates_and_empty_rows():
    """Rows of every length from 0 to Nc / 2 - 1, some listing a cube twice:
    still the same bits as the reorder and the raster entry point."""
    _log("gather variable LUT rows")
    w = G128
    p = problem(w)
    x = _inputs(w)
    nc, mk = p.n_cubes, p.n_cubes // 2 - 1
    rng = np.random.default_rng(3)
    lut = np.zeros((1, p.heads, nc, mk), np.int32)
    valid = np.zeros((1, p.heads, nc), np.int32)
    for h in range(p.heads):
        for i in range(nc):
            n = (i * 7 + h) % (mk + 1)
            row = np.sort(rng.choice(nc, size=n, replace=False)) if i % 5 else rng.integers(0, nc, size=n)
            lut[0, h, i, :n] = row
            valid[0, h, i] = n
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    (og, lg), (orf, lr) = _both_paths(p, q, k, v, dev(lut), dev(valid))
    assert np.array_equal(bits(og), bits(orf))
    assert np.array_equal(bits(lg), bits(lr))
    empty = valid[0] == 0
    assert empty.any()
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    o_cube = np.take(host64(og), pi, axis=2)
    for h, i in zip(*np.nonzero(empty)):
        assert np.all(o_cube[0, h, i * 64:(i + 1) * 64] == 0.0)


@pytest.mark.parametrize("dims,kw", [((1, 2, 8, 16, 16, 4, 4, 4, 64), {}),
                                     ((1, 2, 8, 16, 16, 2, 8, 4, 128), {"cube": "2x8x4"}),
                                     ((1, 2, 8, 16, 14, 4, 4, 4, 128), {"padded": True}),
                                     ((1, 2, 8, 16, 16, 4, 8, 2, 128), {})],
                         ids=["d64", "cube2x8x4-ok", "padded", "cw2"])
def test_gather_shapes(dims, kw):
    """d = 64, cubes 2 tokens wide and padded grids are refused; a 2x8x4 cube
    (4 tokens wide) is gathered, with the same bits as the reorder path."""
    p = L.Problem(*dims)
    _log(f"gather shape {dims}")
    x = torch.randn((p.batch, p.heads, p.n_tokens, p.head_dim), device="cuda").to(torch.bfloat16)
    lut = torch.zeros((1, p.heads, p.n_cubes, 4), dtype=torch.int32, device="cuda")
    lut[..., 1] = 1; lut[..., 2] = 2; lut[..., 3] = 3
    valid = torch.full((1, p.heads, p.n_cubes), 4, dtype=torch.int32, device="cuda")
    if kw.get("cube") == "2x8x4":
        (og, lg), (orf, lr) = _both_paths(p, x, x, x, lut, valid)
        assert np.array_equal(bits(og), bits(orf)) and np.array_equal(bits(lg), bits(lr))
        return
    out = torch.empty_like(x)
    with pytest.raises(L.VsaError) as e:
        L.vsa_sparse_attn_fwd_gather(p, x, x, x, lut, valid, out)
    assert e.value.status == L.VSA_ERR_UNSUPPORTED


POOL = [("wan-bf16", (1, 12, 16, 32, 64, 4, 4, 4, 128), L.VSA_BF16, False),
        ("padded-bf16", (1, 2, 21, 30, 52, 4, 4, 4, 128), L.VSA_BF16, False),
        ("small-f32", (1, 4, 8, 16, 16, 4, 4, 4, 64), L.VSA_F32, False),
        ("wan-bnhd", (1, 12, 16, 32, 64, 4, 4, 4, 128), L.VSA_BF16, True),
        ("vol6-bf16", (1, 2, 3, 6, 4, 3, 2, 1, 128), L.VSA_BF16, False)]


@pytest.mark.parametrize("name,dims,dtype,bnhd", POOL, ids=[c[0] for c in POOL])
def test_pool_from_raster_rows_bit_equal(name, dims, dtype, bnhd):
    """vsa_permute_pool without a cube-major output writes the same pooled bits."""
    _log(f"pool from raster rows {name}")
    p = L.Problem(*dims)
    td = torch.bfloat16 if dtype == L.VSA_BF16 else torch.float32
    shape = (p.batch, p.n_tokens, p.heads, p.head_dim) if bnhd else (p.batch, p.heads, p.n_tokens, p.head_dim)
    g = torch.Generator(device="cuda").manual_seed(9)
    x = torch.randn(shape, device="cuda", generator=g).to(td)
    xcube = torch.empty((p.batch, p.heads, p.n_positions, p.head_dim), dtype=td, device="cuda")
    want = torch.full((p.batch, p.heads, p.n_cubes, p.head_dim), float("nan"), device="cuda")
    got = torch.full_like(want, float("nan"))
    fn = L.vsa_permute_pool_bnhd if bnhd else L.vsa_permute_pool
    fn(p, dtype, x, xcube, want)
    fn(p, dtype, x, None, got)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want))


def test_vsa_forward_gather_mode_matches_reorder_mode():
    """VsaForward with gather=True (pool-only first pass, gathering fine stage,
    no cube-major copies) writes the bits of the reordering sequence, and
    vsa_forward picks it for the 32K-token layer."""
    from block_sparse_video_major_amd.pipeline import VsaForward, vsa_forward, gather_supported
    _log("VsaForward gather mode")
    w = wl.WAN
    p = problem(w)
    assert gather_supported(p)
    x = inputs("wan")
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    outs = []
    for gather in (False, True):
        f = VsaForward(p, w.top_k, gather=gather, with_lse=True)
        assert (f.qp is None) == gather
        out = torch.empty_like(q)
        f(q, k, v, out, gate_c=gc, gate_f=gf)
        outs.append((out, f.lse, f.intermediates()))
    torch.cuda.synchronize()
    (o0, l0, i0), (o1, l1, i1) = outs
    assert np.array_equal(bits(o0), bits(o1)) and np.array_equal(bits(l0), bits(l1))
    for n in ("qc", "kc", "vc", "oc", "kv_block_idx", "valid_block_num"):
        assert np.array_equal(bits(i0[n]), bits(i1[n])), n
    assert "qp" not in i1
    o2 = vsa_forward(q, k, v, p, w.top_k, gate_c=gc, gate_f=gf)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o2), bits(o0))
