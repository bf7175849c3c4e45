"""GPU parity: every C-ABI entry point against the fp64 oracle.

Bars (stated in tests/gpu_helpers.py):
* reorder: bit-exact (integer index work);
* pool: within the fp32 recursive-summation bound vol * 2^-24 * max|x|;
* Top-K sets: identical except swaps among near-ties of the K-th score;
  valid counts exact; O_c within 1e-4;
* attention outputs: max-abs <= 2e-2 and mean-abs <= 2e-3 against the oracle
  evaluated on the same LUT; LSE within 1e-3.
Inputs are the seeded synthetic workloads; at full sizes the oracle checks
sampled query cubes / heads while the GPU runs the whole launch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaForward
from gpu_helpers import (LSE_MAX_ABS, OC_MAX_ABS, assert_out_close, bits, check_lut_against_scores,
                         dev, err, host64, inputs, problem)

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


def _sync():
    torch.cuda.synchronize()


def test_device_peak_query():
    """The measurement helper reports what the runtime reports, and the peak is
    the product CUs x clock x 4096 flop per clock per CU."""
    _log("vsa_device_peak")
    cus, khz, tf = L.vsa_device_peak(0)
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert khz > 0
    assert tf == pytest.approx(cus * khz * 1e3 * 4096 / 1e12, rel=1e-12)


# ------------------------------------------------------------------ reorder
REORDER = [
    ("tiny-f32", (1, 1, 4, 8, 8, 4, 4, 4, 64), L.VSA_F32),
    ("small-bf16", (1, 4, 8, 16, 16, 4, 4, 4, 64), L.VSA_BF16),
    ("wan-bf16", (1, 12, 16, 32, 64, 4, 4, 4, 128), L.VSA_BF16),
    ("vol8-f32-b2", (2, 3, 2, 4, 6, 2, 2, 2, 64), L.VSA_F32),
    ("vol6-bf16", (1, 2, 3, 6, 4, 3, 2, 1, 128), L.VSA_BF16),
    ("row512-f32", (1, 2, 4, 8, 12, 4, 4, 4, 128), L.VSA_F32),
    ("vol1-bf16", (1, 1, 3, 5, 7, 1, 1, 1, 64), L.VSA_BF16),
    ("large-bf16", (1, 40, 32, 48, 80, 4, 4, 4, 128), L.VSA_BF16),
]


@pytest.mark.parametrize("name,dims,dtype", REORDER, ids=[r[0] for r in REORDER])
def test_reorder_bit_exact(name, dims, dtype):
    _log(f"reorder {name}")
    p = L.Problem(*dims)
    rng = np.random.default_rng(100)
    shape = (p.batch, p.heads, p.n_tokens, p.head_dim)
    if dtype == L.VSA_BF16:
        x = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)
        xt = torch.from_numpy(x.view(np.float32)).cuda()
    xc = torch.empty_like(xt)
    back = torch.empty_like(xt)
    L.vsa_permute(p, dtype, xt, xc)
    L.vsa_unpermute(p, dtype, xc, back)
    _sync()
    pi = oracle.perm_index(p.T, p.H, p.W, p.ct, p.ch, p.cw)
    want = np.take(x, pi, axis=2)
    assert np.array_equal(bits(xc), want.view(bits(xc).dtype))
    assert np.array_equal(bits(back), x.view(bits(back).dtype))
    # the fused reorder + pool writes the same bits as the two separate passes
    pooled_shape = (p.batch, p.heads, p.n_cubes, p.head_dim)
    pooled = torch.empty(pooled_shape, dtype=torch.float32, device="cuda")
    pooled_fused = torch.empty(pooled_shape, dtype=torch.float32, device="cuda")
    xc_fused = torch.empty_like(xt)
    L.vsa_pool(p, dtype, xc, pooled)
    L.vsa_permute_pool(p, dtype, xt, xc_fused, pooled_fused)
    _sync()
    assert np.array_equal(bits(xc_fused), bits(xc))
    # random bit patterns include NaNs, whose payload the two passes may pick
    # from either operand of an add: NaN positions must agree, other bits too
    a, b = pooled_fused.cpu().numpy(), pooled.cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    keep = ~np.isnan(a)
    assert np.array_equal(a[keep].view(np.uint32), b[keep].view(np.uint32))


# ------------------------------------------------------------------ pool
def _pool_case(w, heads=None):
    x = inputs(w.name)
    p = problem(w)
    dtype = L.VSA_BF16 if w.dtype == "bf16" else L.VSA_F32
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    res = {}
    for n in ("q", "k", "v"):
        xt = dev(x[n])
        xcube = torch.empty_like(xt)
        L.vsa_permute(p, dtype, xt, xcube)
        pooled = torch.empty((p.batch, p.heads, p.n_cubes, p.head_dim), dtype=torch.float32, device="cuda")
        L.vsa_pool(p, dtype, xcube, pooled)
        xcube2 = torch.empty_like(xt)
        pooled2 = torch.empty_like(pooled)
        L.vsa_permute_pool(p, dtype, xt, xcube2, pooled2)
        _sync()
        assert torch.equal(xcube2, xcube)
        assert np.array_equal(bits(pooled2), bits(pooled)), "fused pool differs from vsa_pool"
        hs = range(w.heads) if heads is None else heads
        got = host64(pooled)[:, list(hs)]
        x64 = wl.as_float64(x[n][:, list(hs)])
        want = oracle.pool(oracle.permute(x64, pi), w.cube_volume)
        tol = w.cube_volume * 2.0 ** -24 * float(np.abs(x64).max())
        res[n] = err(got, want)
        assert res[n][0] <= tol, f"pool {n}: max-abs {res[n][0]:.3e} > {tol:.3e}"
    return res


@pytest.mark.parametrize("name,heads", [("tiny", None), ("small", None), ("wan", None), ("large", [0, 39])],
                         ids=["tiny", "small", "wan", "large"])
def test_pool(name, heads):
    _log(f"pool {name}")
    _pool_case(wl.WORKLOADS[name], heads)


def test_pool_other_cube_shape():
    _log("pool vol8 f32")
    p = L.Problem(2, 3, 2, 4, 6, 2, 2, 2, 64)
    rng = np.random.default_rng(101)
    x = rng.standard_normal((2, 3, p.n_tokens, 64)).astype(np.float32)
    xc = torch.from_numpy(x).cuda()
    pooled = torch.empty((2, 3, p.n_cubes, 64), dtype=torch.float32, device="cuda")
    L.vsa_pool(p, L.VSA_F32, xc, pooled)
    _sync()
    want = oracle.pool(x.astype(np.float64), 8)
    assert err(host64(pooled), want)[0] <= 8 * 2.0 ** -24 * np.abs(x).max()


# ------------------------------------------------------------------ coarse + Top-K
def _oracle_pooled(w, heads):
    """Oracle pooled Q/K/V (fp64) for the given heads, from the raw inputs."""
    x = inputs(w.name)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    return {n: oracle.pool(oracle.permute(wl.as_float64(x[n][:, list(heads)]), pi), w.cube_volume)
            for n in ("q", "k", "v")}


def _coarse_case(w, k, heads_checked):
    """GPU coarse_topk over all heads; the checked heads get the oracle's
    pooled values (rounded to fp32), the others random fp32 values."""
    p = problem(w)
    pooled = _oracle_pooled(w, heads_checked)
    shape = (p.batch, p.heads, p.n_cubes, p.head_dim)
    rng = np.random.default_rng(7)
    host = {n: rng.standard_normal(shape).astype(np.float32) for n in ("q", "k", "v")}
    for n in host:
        host[n][:, list(heads_checked)] = pooled[n].astype(np.float32)
    qc, kc, vc = (dev(host[n]) for n in ("q", "k", "v"))
    lut = torch.full((p.batch, p.heads, p.n_cubes, k), -7, dtype=torch.int32, device="cuda")
    valid = torch.full((p.batch, p.heads, p.n_cubes), -7, dtype=torch.int32, device="cuda")
    oc = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    L.vsa_coarse_topk(p, k, qc, kc, vc, lut, valid, oc)
    _sync()
    hs = list(heads_checked)
    q64, k64, v64 = (host[n][:, hs].astype(np.float64) for n in ("q", "k", "v"))
    s, _, oc_want = oracle.coarse_attention(q64, k64, v64, 1.0 / math.sqrt(w.head_dim))
    lut_want, _ = oracle.topk_lut(s, k)
    lut_got = lut.cpu().numpy()[:, hs]
    differ = check_lut_against_scores(lut_got, valid.cpu().numpy()[:, hs], s, k, lut_want)
    oc_err = err(host64(oc)[:, hs], oc_want)
    assert oc_err[0] <= OC_MAX_ABS, f"O_c max-abs {oc_err[0]:.3e}"
    assert np.all(valid.cpu().numpy() == k)
    return differ


COARSE = [("tiny", 2, [0]), ("small", 8, [0, 1, 2, 3]), ("small", 1, [0, 1, 2, 3]),
          ("small", 32, [0, 1, 2, 3]), ("small", 31, [0, 1, 2, 3]),
          ("wan", 154, list(range(12))), ("wan", 256, [0, 5, 11]), ("wan", 102, [1, 7]),
          ("wan", 51, [2, 9]), ("wan", 512, [3]), ("large", 192, [0, 17, 39])]


@pytest.mark.parametrize("name,k,heads", COARSE, ids=[f"{c[0]}-k{c[1]}" for c in COARSE])
def test_coarse_topk(name, k, heads):
    _log(f"coarse_topk {name} K={k}")
    differ = _coarse_case(wl.WORKLOADS[name], k, heads)
    print(f"rows differing within the tie window: {differ}")


def test_coarse_topk_ties_take_lower_index():
    """Exact ties: identical key cubes give identical scores; the lower index
    must win, as in the oracle."""
    _log("coarse_topk exact ties")
    p = L.Problem(1, 1, 4, 8, 16, 4, 4, 4, 64)     # Nc = 8
    rng = np.random.default_rng(3)
    qc = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    kc[0, 0, 5] = kc[0, 0, 2]
    kc[0, 0, 6] = kc[0, 0, 2]
    vc = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    for k in range(1, 9):
        lut = torch.empty((1, 1, 8, k), dtype=torch.int32, device="cuda")
        valid = torch.empty((1, 1, 8), dtype=torch.int32, device="cuda")
        L.vsa_coarse_topk(p, k, dev(qc), dev(kc), dev(vc), lut, valid, None)
        _sync()
        # the fp32 scores of the duplicated cubes are bitwise equal on both sides
        s = np.einsum("id,jd->ij", qc[0, 0].astype(np.float64), kc[0, 0].astype(np.float64))
        want, _ = oracle.topk_lut(s[None, None], k)
        assert np.array_equal(lut.cpu().numpy(), want), f"K={k}"


# Cube counts outside the workloads: the largest Nc the coarse stage accepts
# at both head sizes (fewer query rows per workgroup, the key range split
# across row groups for the coarse output, keys in 64 slots per lane), a
# count that is not a multiple of 4 (padded score rows), one between, and
# the two sides of the limit of the sixteen-row kernel.
COARSE_GEOM = [(128, (64, 64, 64), 192), (64, (64, 64, 64), 100),
               (64, (20, 36, 44), 37), (128, (4, 4, 6124), 64),
               # 2,012 cubes (32 key slots per lane), the largest count whose
               # sixteen score rows fit in LDS (the matrix-core kernel, 40
               # slots, the plain padded row stride) and the next one up (the
               # vector kernel)
               (128, (4, 4, 8048), 201), (128, (4, 4, 10224), 201), (128, (4, 4, 10240), 201),
               # 2,500 cubes at d = 64: the matrix-core kernel with 40 key slots
               # per lane and eight key splits of its coarse output
               (64, (4, 4, 10000), 150)]


@pytest.mark.parametrize("d,dims,k", COARSE_GEOM, ids=[f"d{c[0]}-nc{c[1][0] * c[1][1] * c[1][2] // 64}"
                                                       for c in COARSE_GEOM])
def test_coarse_topk_cube_counts(d, dims, k):
    T, H, W = dims
    p = L.Problem(1, 1, T, H, W, 4, 4, 4, d)
    nc = p.n_cubes
    _log(f"coarse_topk Nc={nc} d={d} K={k}")
    rng = np.random.default_rng(11)
    host = {n: rng.standard_normal((1, 1, nc, d)).astype(np.float32) for n in ("q", "k", "v")}
    lut = torch.full((1, 1, nc, k), -7, dtype=torch.int32, device="cuda")
    valid = torch.full((1, 1, nc), -7, dtype=torch.int32, device="cuda")
    oc = torch.full((1, 1, nc, d), float("nan"), dtype=torch.float32, device="cuda")
    L.vsa_coarse_topk(p, k, dev(host["q"]), dev(host["k"]), dev(host["v"]), lut, valid, oc)
    _sync()
    q64, k64, v64 = (host[n].astype(np.float64) for n in ("q", "k", "v"))
    s, _, oc_want = oracle.coarse_attention(q64, k64, v64, 1.0 / math.sqrt(d))
    lut_want, _ = oracle.topk_lut(s, k)
    differ = check_lut_against_scores(lut.cpu().numpy(), valid.cpu().numpy(), s, k, lut_want)
    oc_err = err(host64(oc), oc_want)
    assert oc_err[0] <= OC_MAX_ABS, f"O_c max-abs {oc_err[0]:.3e}"
    print(f"rows differing within the tie window: {differ}")


# ------------------------------------------------------------------ fine attention
def _fine_case(w, k, check_cubes, gates=True, lse=True, heads_checked=None, lut_kind="oracle"):
    """Fine kernel on oracle-permuted inputs with a LUT covering every head.
    Checked heads get the oracle's LUT / O_c; the rest get a seeded random LUT.
    Returns (max_abs, mean_abs) on the checked query cubes."""
    p = problem(w)
    x = inputs(w.name, with_gates=gates)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    vol = w.cube_volume
    hs = list(range(w.heads)) if heads_checked is None else list(heads_checked)
    bf = (lambda a: a) if w.dtype == "bf16" else wl.f32_to_bf16_bits
    names = ("q", "k", "v", "gate_c", "gate_f") if gates else ("q", "k", "v")
    xp = {n: np.take(bf(x[n]), pi, axis=2) for n in names}      # exact bf16 bit gather
    pooled = _oracle_pooled(w, hs)
    scale = 1.0 / math.sqrt(w.head_dim)
    s, _, oc_h = oracle.coarse_attention(pooled["q"], pooled["k"], pooled["v"], scale)
    lut_h, valid_h = oracle.topk_lut(s, k)
    rng = np.random.default_rng(11)
    lut = np.empty((p.batch, p.heads, p.n_cubes, k), np.int32)
    for idx in np.ndindex(p.batch, p.heads, p.n_cubes):
        lut[idx] = np.sort(rng.permutation(p.n_cubes)[:k])
    lut[:, hs] = lut_h
    valid = np.full((p.batch, p.heads, p.n_cubes), k, np.int32)
    oc = rng.standard_normal((p.batch, p.heads, p.n_cubes, p.head_dim)).astype(np.float32)
    oc[:, hs] = oc_h.astype(np.float32)
    q, kk, v = (dev(xp[n]) for n in ("q", "k", "v"))
    gc = dev(xp["gate_c"]) if gates else None
    gf = dev(xp["gate_f"]) if gates else None
    out = torch.full_like(q, float("nan"))
    lse_t = torch.full((p.batch, p.heads, p.n_tokens), float("nan"), device="cuda") if lse else None
    L.vsa_sparse_attn_fwd(p, q, kk, v, dev(lut), dev(valid), out, oc=dev(oc) if gates else None,
                          gate_c=gc, gate_f=gf, lse=lse_t)
    _sync()
    got = host64(out)
    assert np.all(np.isfinite(got)), "output has non-finite values"
    cubes = [(0, hi, i) for hi in range(len(hs)) for i in check_cubes(w)]
    q64, k64, v64 = (wl.as_float64(xp[n][:, hs]) for n in ("q", "k", "v"))
    of, lse_w = oracle.fine_attention(q64, k64, v64, lut_h, valid_h, scale, vol, query_cubes=cubes)
    want = oracle.combine(of, oc_h.astype(np.float32).astype(np.float64), vol,
                          wl.as_float64(xp["gate_c"][:, hs]) if gates else None,
                          wl.as_float64(xp["gate_f"][:, hs]) if gates else None)
    rows = np.concatenate([np.arange(i * vol, (i + 1) * vol) for i in check_cubes(w)])
    res = assert_out_close(got[:, hs][:, :, rows], want[:, :, rows], f"fine {w.name} K={k}")
    if lse:
        lg = host64(lse_t)[:, hs][:, :, rows]
        le = err(lg, lse_w[:, :, rows])
        assert le[0] <= LSE_MAX_ABS, f"lse max-abs {le[0]:.3e}"
    return res


def _all_cubes(w):
    return range(w.n_cubes)


def _sampled_cubes(w):
    rng = np.random.default_rng(5)
    picks = set(rng.choice(w.n_cubes, size=min(w.n_cubes, 24), replace=False).tolist())
    picks |= {0, w.n_cubes - 1}
    return sorted(picks)


FINE = [("tiny", 2, _all_cubes, None), ("tiny", 4, _all_cubes, None),
        ("small", 8, _all_cubes, None), ("small", 1, _all_cubes, None), ("small", 32, _all_cubes, None),
        ("wan", 154, _sampled_cubes, [0, 6, 11]), ("wan", 51, _sampled_cubes, [4]),
        ("wan", 102, _sampled_cubes, [8]), ("wan", 256, _sampled_cubes, [2]),
        ("wan", 512, _sampled_cubes, [10]), ("large", 192, _sampled_cubes, [0, 39])]


@pytest.mark.parametrize("name,k,cubes,heads", FINE, ids=[f"{c[0]}-k{c[1]}" for c in FINE])
def test_sparse_attn_fwd(name, k, cubes, heads):
    _log(f"sparse_attn_fwd {name} K={k}")
    mx, mean = _fine_case(wl.WORKLOADS[name], k, cubes, heads_checked=heads)
    print(f"max-abs {mx:.3e} mean-abs {mean:.3e}")


@pytest.mark.parametrize("name", ["small", "wan"])
def test_sparse_attn_fwd_no_gates(name):
    _log(f"sparse_attn_fwd {name} without gates / lse")
    w = wl.WORKLOADS[name]
    _fine_case(w, w.top_k, _sampled_cubes, gates=False, lse=False,
               heads_checked=[0] if name == "wan" else None)


def test_sparse_attn_variable_counts_duplicates_and_empty_rows():
    """Valid counts 0..max, unsorted and repeated entries, max_kv > count."""
    _log("sparse_attn_fwd variable LUT rows")
    w = wl.SMALL
    p = problem(w)
    x = inputs(w.name)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    xp = {n: np.take(x[n], pi, axis=2) for n in ("q", "k", "v")}
    rng = np.random.default_rng(21)
    maxk = 12
    lut = rng.integers(0, p.n_cubes, size=(1, w.heads, p.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(0, maxk + 1, size=(1, w.heads, p.n_cubes)).astype(np.int32)
    valid[0, 0, :4] = 0
    valid[0, 1, :4] = maxk
    lut[0, 2, 0, :3] = 5                                  # repeated entry
    q, k, v = (dev(xp[n]) for n in ("q", "k", "v"))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, w.heads, p.n_tokens), float("nan"), device="cuda")
    L.vsa_sparse_attn_fwd(p, q, k, v, dev(lut), dev(valid), out, lse=lse)
    _sync()
    of, lse_w = oracle.fine_attention(*(wl.as_float64(xp[n]) for n in ("q", "k", "v")), lut, valid,
                                      1 / math.sqrt(w.head_dim), 64)
    got = host64(out)
    assert_out_close(got, of, "variable rows")
    empty = np.repeat(valid == 0, 64, axis=-1)
    assert np.all(got[empty] == 0.0)
    lg = host64(lse)
    assert np.all(np.isneginf(lg[empty]))
    assert err(lg[~empty], lse_w[~empty])[0] <= LSE_MAX_ABS


def test_sparse_attn_empty_rows_give_gated_coarse_output():
    _log("sparse_attn_fwd empty rows with gates")
    w = wl.SMALL
    p = problem(w)
    x = inputs(w.name, with_gates=True)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    lut = torch.zeros((1, w.heads, p.n_cubes, 4), dtype=torch.int32, device="cuda")
    valid = torch.zeros((1, w.heads, p.n_cubes), dtype=torch.int32, device="cuda")
    oc = torch.randn((1, w.heads, p.n_cubes, 64), device="cuda")
    out = torch.empty_like(q)
    L.vsa_sparse_attn_fwd(p, q, k, v, lut, valid, out, oc=oc, gate_c=gc, gate_f=gf)
    _sync()
    want = oracle.combine(np.zeros((1, w.heads, p.n_tokens, 64)), host64(oc), 64, host64(gc), host64(gf))
    assert err(host64(out), want)[0] <= 2.0 ** -8 * np.abs(want).max()


def test_sparse_attn_raster_output_matches_unpermute():
    """vsa_sparse_attn_fwd_raster = vsa_sparse_attn_fwd on cube-major gates
    followed by vsa_unpermute of out and lse, bit for bit."""
    _log("fine raster output")
    for name, k in (("small", 8), ("wan", 154)):
        w = wl.WORKLOADS[name]
        p = problem(w)
        x = inputs(name, with_gates=True)
        raster = {n: dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f")}
        cube = {}
        for n, t in raster.items():
            cube[n] = torch.empty_like(t)
            L.vsa_permute(p, L.VSA_BF16, t, cube[n])
        rng = np.random.default_rng(5)
        lut = np.sort(rng.permuted(np.tile(np.arange(p.n_cubes, dtype=np.int32), (1, p.heads, p.n_cubes, 1)),
                                   axis=-1)[..., :k], axis=-1)
        lut_d, valid_d = dev(lut), dev(np.full((1, p.heads, p.n_cubes), k, np.int32))
        oc = torch.randn((1, p.heads, p.n_cubes, p.head_dim), device="cuda")
        out_c = torch.empty_like(cube["q"])
        lse_c = torch.empty((1, p.heads, p.n_tokens), dtype=torch.float32, device="cuda")
        L.vsa_sparse_attn_fwd(p, cube["q"], cube["k"], cube["v"], lut_d, valid_d, out_c, oc=oc,
                              gate_c=cube["gate_c"], gate_f=cube["gate_f"], lse=lse_c)
        out_r = torch.full_like(out_c, float("nan"))
        lse_r = torch.full_like(lse_c, float("nan"))
        L.vsa_sparse_attn_fwd_raster(p, cube["q"], cube["k"], cube["v"], lut_d, valid_d, out_r, oc=oc,
                                     gate_c=raster["gate_c"], gate_f=raster["gate_f"], lse=lse_r)
        back = torch.empty_like(out_c)
        L.vsa_unpermute(p, L.VSA_BF16, out_c, back)
        _sync()
        assert np.array_equal(bits(out_r), bits(back)), name
        pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
        lse_back = np.empty_like(lse_c.cpu().numpy())
        lse_back[..., pi] = lse_c.cpu().numpy()
        assert np.array_equal(lse_r.cpu().numpy().view(np.uint32), lse_back.view(np.uint32)), name


@pytest.mark.parametrize("kk", [154, 300])
def test_sparse_attn_without_gates_equals_unit_gates(kk):
    """Without gates out = O_f; with g_f = 1 and g_c = 0 the gated epilogue
    forms fma(0, O_c, 1 * O_f) = O_f exactly.  The two take different output
    loops (the gate-free one has no per-row gate tests), so they must agree
    bit for bit, in cube-major and in raster order, for pairs (Top-154) and
    quads (Top-300) of query cubes."""
    _log(f"fine gate-free output K={kk}")
    w = wl.WAN
    p = problem(w)
    x = inputs("wan")
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    qp, kp, vp = (torch.empty_like(q) for _ in range(3))
    for t, c in ((q, qp), (k, kp), (v, vp)):
        L.vsa_permute(p, L.VSA_BF16, t, c)
    rng = np.random.default_rng(11)
    lut = np.sort(np.stack([rng.permutation(w.n_cubes)[:kk] for _ in range(w.heads * w.n_cubes)]), axis=1)
    lut_d = dev(lut.reshape(1, w.heads, w.n_cubes, kk).astype(np.int32))
    valid_d = torch.full((1, w.heads, w.n_cubes), kk, dtype=torch.int32, device="cuda")
    oc = torch.randn((1, w.heads, w.n_cubes, w.head_dim), device="cuda")
    ones = torch.ones_like(q)
    zeros = torch.zeros_like(q)
    for fwd in (L.vsa_sparse_attn_fwd, L.vsa_sparse_attn_fwd_raster):
        plain = torch.full_like(q, float("nan"))
        unit = torch.full_like(q, float("nan"))
        fwd(p, qp, kp, vp, lut_d, valid_d, plain)
        fwd(p, qp, kp, vp, lut_d, valid_d, unit, oc=oc, gate_c=zeros, gate_f=ones)
        _sync()
        assert np.array_equal(bits(plain), bits(unit)), fwd.__name__


# Top-154 of 512 cubes runs the kernel over pairs of query cubes, Top-300
# the one over quads (rows listing at least half of the cubes).
@pytest.mark.parametrize("kk", [154, 300])
def test_sparse_attn_deterministic(kk):
    _log(f"sparse_attn_fwd determinism K={kk}")
    w = wl.WAN
    p = problem(w)
    x = inputs(w.name)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    rng = np.random.default_rng(4)
    lut = np.sort(np.stack([rng.permutation(512)[:kk] for _ in range(12 * 512)]), axis=1)
    lut = dev(lut.reshape(1, 12, 512, kk).astype(np.int32))
    valid = torch.full((1, 12, 512), kk, dtype=torch.int32, device="cuda")
    outs, lses = [], []
    for _ in range(3):
        o = torch.empty_like(q)
        lse = torch.empty((1, 12, p.n_positions), dtype=torch.float32, device="cuda")
        L.vsa_sparse_attn_fwd(p, q, k, v, lut, valid, o, lse=lse)
        outs.append(o)
        lses.append(lse)
    _sync()
    for o, lse in zip(outs[1:], lses[1:]):
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))
        assert torch.equal(lses[0].view(torch.int32), lse.view(torch.int32))


def test_errors_leave_outputs_untouched():
    _log("error paths keep canaries")
    w = wl.SMALL
    p = problem(w)
    q = torch.randn((1, 4, p.n_tokens, 64), device="cuda").to(torch.bfloat16)
    out = torch.full_like(q, 3.0)
    lut = torch.zeros((1, 4, p.n_cubes, 8), dtype=torch.int32, device="cuda")
    valid = torch.full((1, 4, p.n_cubes), 8, dtype=torch.int32, device="cuda")
    bad = L.Problem(1, 4, 8, 16, 16, 2, 2, 2, 64)      # cube volume 8: unsupported by the fine kernel
    with pytest.raises(L.VsaError):
        L.vsa_sparse_attn_fwd(L.Problem(1, 4, 8, 16, 16, 4, 4, 4, 64), q, q, q,
                              torch.zeros((1, 4, p.n_cubes, 33), dtype=torch.int32, device="cuda"),
                              valid, out)
    lib = L.load()
    import ctypes
    st = lib.vsa_sparse_attn_fwd(ctypes.byref(bad.c_struct()), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                 lut.data_ptr(), valid.data_ptr(), 8, None, None, None, out.data_ptr(),
                                 None, None)
    assert st == L.VSA_ERR_UNSUPPORTED
    xc = torch.full((1, 4, p.n_cubes, 64), 5.0, device="cuda")
    with pytest.raises(L.VsaError):
        L.vsa_coarse_topk(p, 0, xc, xc, xc, torch.zeros((1, 4, p.n_cubes, 0), dtype=torch.int32,
                                                        device="cuda"), valid, xc)
    _sync()
    assert torch.all(out.float() == 3.0)
    assert torch.all(xc == 5.0)
    assert torch.all(valid == 8)


def test_check_lut():
    _log("check_lut")
    p = problem(wl.SMALL)
    rng = np.random.default_rng(9)
    lut = rng.integers(0, p.n_cubes, size=(1, 4, p.n_cubes, 6)).astype(np.int32)
    valid = np.full((1, 4, p.n_cubes), 6, np.int32)
    bad_rows = set()
    lut[0, 1, 3, 2] = p.n_cubes; bad_rows.add((1, 3))
    lut[0, 2, 7, 0] = -1; bad_rows.add((2, 7))
    valid[0, 3, 9] = 7; bad_rows.add((3, 9))
    valid[0, 0, 1] = -2; bad_rows.add((0, 1))
    lut[0, 0, 4, 5] = 999; valid[0, 0, 4] = 5            # bad entry beyond the count: fine
    counter = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    L.vsa_check_lut(p, dev(lut), dev(valid), counter)
    _sync()
    assert int(counter.item()) == len(bad_rows)
    ok = np.sort(rng.integers(0, p.n_cubes, size=(1, 4, p.n_cubes, 6)), axis=-1).astype(np.int32)
    L.vsa_check_lut(p, dev(ok), dev(np.full((1, 4, p.n_cubes), 6, np.int32)), counter)
    _sync()
    assert int(counter.item()) == 0


# ------------------------------------------------------------------ block relation matrix -> LUT
MASKS = [("small-random", "small", None), ("small-overflow", "small", 6), ("wan-union", "wan", None),
         ("large-union", "large", None)]


def _mask_for(name, w):
    if name.endswith("random"):
        rng = np.random.default_rng(31)
        m = (rng.random((w.batch, w.heads, w.n_cubes, w.n_cubes)) < 0.3).astype(np.uint8)
        m[0, 0, 0, :] = 0
        m[0, 1, 1, :] = 1
        return m
    if name.endswith("overflow"):
        return np.tril(np.ones((w.n_cubes, w.n_cubes), np.uint8))[None, None].repeat(w.heads, axis=1)
    return wl.block_relation_mask(w, 48 if w.name == "wan" else 64, 4)


@pytest.mark.parametrize("case,name,maxk", MASKS, ids=[m[0] for m in MASKS])
def test_mask_to_lut(case, name, maxk):
    """Converted rows and counts match the oracle exactly; entries past a
    row's count stay untouched; the overflow count is exact."""
    _log(f"mask_to_lut {case}")
    w = wl.WORKLOADS[name]
    p = problem(w)
    mask = _mask_for(case, w)
    rows_max = int(mask.astype(np.int64).sum(axis=-1).max())
    maxk = maxk or rows_max
    lut = torch.full((w.batch, w.heads, w.n_cubes, maxk), -7, dtype=torch.int32, device="cuda")
    valid = torch.full((w.batch, w.heads, w.n_cubes), -7, dtype=torch.int32, device="cuda")
    over = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    L.vsa_mask_to_lut(p, torch.from_numpy(mask).cuda(), lut, valid, over)
    _sync()
    hs = [0, w.heads - 1] if w.heads > 4 else list(range(w.heads))
    want_lut, want_valid, want_over = oracle.mask_to_lut(mask[:, hs], maxk)
    got_lut, got_valid = lut.cpu().numpy()[:, hs], valid.cpu().numpy()[:, hs]
    assert np.array_equal(got_valid, want_valid)
    for idx in np.ndindex(*want_valid.shape):
        n = want_valid[idx]
        assert np.array_equal(got_lut[idx][:n], want_lut[idx][:n]), idx
        assert np.all(got_lut[idx][n:] == -7), idx
    total_over = int((mask.astype(np.int64).sum(axis=-1) > maxk).sum())
    assert int(over.item()) == total_over
    if len(hs) == w.heads:
        assert want_over == total_over


def test_mask_to_lut_odd_cube_count():
    """Nc = 45 (not a multiple of 4: one mask byte per lane per pass)."""
    _log("mask_to_lut odd Nc")
    p = L.Problem(2, 3, 12, 12, 20, 4, 4, 4, 64)    # Nc = 3 * 3 * 5 = 45
    nc = p.n_cubes
    rng = np.random.default_rng(32)
    mask = (rng.random((2, 3, nc, nc)) < 0.5).astype(np.uint8)
    mask[1, 2, 7, :] = 0
    maxk = 20
    lut = torch.full((2, 3, nc, maxk), -7, dtype=torch.int32, device="cuda")
    valid = torch.full((2, 3, nc), -7, dtype=torch.int32, device="cuda")
    over = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    L.vsa_mask_to_lut(p, torch.from_numpy(mask).cuda(), lut, valid, over)
    _sync()
    want_lut, want_valid, want_over = oracle.mask_to_lut(mask, maxk)
    got_lut, got_valid = lut.cpu().numpy(), valid.cpu().numpy()
    assert np.array_equal(got_valid, want_valid)
    for idx in np.ndindex(*want_valid.shape):
        n = want_valid[idx]
        assert np.array_equal(got_lut[idx][:n], want_lut[idx][:n]), idx
    assert int(over.item()) == want_over


@pytest.mark.parametrize("name", ["small", "wan"])
def test_sparse_attn_on_union_mask(name):
    """The fine kernel on the LUT of a union mask (importance + condition +
    adjacency; a different count per row) against the oracle on the same
    list.  The pattern comes from vsa_mask_to_lut."""
    _log(f"sparse_attn on union mask {name}")
    w = wl.WORKLOADS[name]
    p = problem(w)
    x = inputs(w.name, with_gates=False)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    mask = wl.block_relation_mask(w, 48 if name == "wan" else 3, 2)
    maxk = int(mask.astype(np.int64).sum(axis=-1).max())
    lut = torch.zeros((w.batch, w.heads, w.n_cubes, maxk), dtype=torch.int32, device="cuda")
    valid = torch.empty((w.batch, w.heads, w.n_cubes), dtype=torch.int32, device="cuda")
    over = torch.empty((1,), dtype=torch.int32, device="cuda")
    L.vsa_mask_to_lut(p, torch.from_numpy(mask).cuda(), lut, valid, over)
    xp = {n: np.take(x[n], pi, axis=2) for n in ("q", "k", "v")}
    q, kk, v = (dev(xp[n]) for n in ("q", "k", "v"))
    out = torch.full_like(q, float("nan"))
    lse_t = torch.full((p.batch, p.heads, p.n_tokens), float("nan"), device="cuda")
    L.vsa_sparse_attn_fwd(p, q, kk, v, lut, valid, out, lse=lse_t)
    _sync()
    assert int(over.item()) == 0
    hs = [0, w.heads - 1] if w.heads > 4 else list(range(w.heads))
    cubes = _all_cubes(w) if name == "small" else _sampled_cubes(w)
    lut_h, valid_h, _ = oracle.mask_to_lut(mask[:, hs], maxk)
    q64, k64, v64 = (wl.as_float64(xp[n][:, hs]) for n in ("q", "k", "v"))
    of, lse_w = oracle.fine_attention(q64, k64, v64, lut_h, valid_h, 1.0 / math.sqrt(w.head_dim),
                                      w.cube_volume, query_cubes=[(0, hi, i) for hi in range(len(hs)) for i in cubes])
    rows = np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in cubes])
    got = host64(out)[:, hs]
    mx, mean = assert_out_close(got[:, :, rows], of[:, :, rows], f"union mask {name}")
    le = err(host64(lse_t)[:, hs][:, :, rows], lse_w[:, :, rows])
    assert le[0] <= LSE_MAX_ABS, f"lse max-abs {le[0]:.3e}"
    print(f"row counts {int(valid_h.min())}..{int(valid_h.max())}; max-abs {mx:.3e} mean-abs {mean:.3e}")


# ------------------------------------------------------------------ whole pipeline
def _pipeline_case(w, k, cubes, heads_checked):
    p = problem(w)
    x = inputs(w.name, with_gates=True)
    q, kk, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    f = VsaForward(p, k, with_gates=True, with_lse=True)
    out = torch.full_like(q, float("nan"))
    f(q, kk, v, out, gc, gf)
    _sync()
    hs = list(heads_checked)
    pooled = _oracle_pooled(w, hs)
    scale = 1.0 / math.sqrt(w.head_dim)
    s, _, oc_w = oracle.coarse_attention(pooled["q"], pooled["k"], pooled["v"], scale)
    lut_w, _ = oracle.topk_lut(s, k)
    lut_g = f.lut.cpu().numpy()[:, hs]
    differ = check_lut_against_scores(lut_g, f.valid.cpu().numpy()[:, hs], s, k, lut_w)
    assert err(host64(f.oc)[:, hs], oc_w)[0] <= OC_MAX_ABS
    # score the fine stage on the LUT the GPU actually used
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    xs = {n: wl.as_float64(x[n][:, hs]) for n in x}
    of, _ = oracle.fine_attention(*(oracle.permute(xs[n], pi) for n in ("q", "k", "v")), lut_g,
                                  np.full(lut_g.shape[:-1], k, np.int32), scale, 64,
                                  query_cubes=[(0, hi, i) for hi in range(len(hs)) for i in cubes(w)])
    out_cube = oracle.combine(of, host64(f.oc)[:, hs], 64, oracle.permute(xs["gate_c"], pi),
                              oracle.permute(xs["gate_f"], pi))
    want = oracle.unpermute(out_cube, pi)
    rows_cube = np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in cubes(w)])
    rows = pi[rows_cube]
    got = host64(out)[:, hs]
    assert np.all(np.isfinite(host64(out)))
    mx, mean = assert_out_close(got[:, :, rows], want[:, :, rows], f"pipeline {w.name}")
    return differ, mx, mean


PIPE = [("small", 8, _all_cubes, [0, 1, 2, 3]), ("wan", 154, _sampled_cubes, [0, 5, 11]),
        ("large", 192, _sampled_cubes, [7])]


@pytest.mark.parametrize("name,k,cubes,heads", PIPE, ids=[f"{c[0]}-k{c[1]}" for c in PIPE])
def test_pipeline_end_to_end(name, k, cubes, heads):
    _log(f"pipeline {name} K={k}")
    differ, mx, mean = _pipeline_case(wl.WORKLOADS[name], k, cubes, heads)
    print(f"tie-window LUT rows {differ}; out max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_pipeline_tiny_fp32_coarse_bf16_fine():
    """Tiny grid in fp32: reorder, pool and selection run on the fp32 inputs;
    the fine kernel (bf16 only) runs on their bf16 rounding."""
    _log("pipeline tiny fp32/bf16")
    w = wl.TINY
    p = problem(w)
    x = inputs("tiny")
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    cube32, pooled = {}, {}
    for n in ("q", "k", "v"):
        t = dev(x[n])
        cube32[n] = torch.empty_like(t)
        L.vsa_permute(p, L.VSA_F32, t, cube32[n])
        pooled[n] = torch.empty((1, 1, p.n_cubes, 64), dtype=torch.float32, device="cuda")
        L.vsa_pool(p, L.VSA_F32, cube32[n], pooled[n])
    lut = torch.empty((1, 1, p.n_cubes, 2), dtype=torch.int32, device="cuda")
    valid = torch.empty((1, 1, p.n_cubes), dtype=torch.int32, device="cuda")
    oc = torch.empty((1, 1, p.n_cubes, 64), dtype=torch.float32, device="cuda")
    L.vsa_coarse_topk(p, 2, pooled["q"], pooled["k"], pooled["v"], lut, valid, oc)
    bfc = {n: cube32[n].to(torch.bfloat16) for n in cube32}
    out_c = torch.empty_like(bfc["q"])
    L.vsa_sparse_attn_fwd(p, bfc["q"], bfc["k"], bfc["v"], lut, valid, out_c)
    out = torch.empty_like(out_c)
    L.vsa_unpermute(p, L.VSA_BF16, out_c, out)
    _sync()
    x64 = {n: x[n].astype(np.float64) for n in x}
    r = oracle.vsa_forward(x64["q"], x64["k"], x64["v"], (w.T, w.H, w.W), w.cube, 2)
    check_lut_against_scores(lut.cpu().numpy(), valid.cpu().numpy(), r["scores"], 2, r["kv_block_idx"])
    assert err(host64(oc), r["oc"])[0] <= OC_MAX_ABS
    xb = {n: wl.as_float64(wl.f32_to_bf16_bits(x[n])) for n in x}
    rb = oracle.vsa_forward(xb["q"], xb["k"], xb["v"], (w.T, w.H, w.W), w.cube, 2,
                            kv_block_idx=lut.cpu().numpy(), valid_block_num=valid.cpu().numpy())
    assert_out_close(host64(out), rb["out"], "tiny pipeline")


@pytest.mark.parametrize("name", ["small", "wan"])
def test_dense_topk_equals_full_attention(name):
    """Top-K = all cubes: the output is dense softmax attention."""
    _log(f"dense {name}")
    w = wl.WORKLOADS[name]
    p = problem(w)
    x = inputs(name)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    f = VsaForward(p, w.n_cubes)
    out = torch.empty_like(q)
    f(q, k, v, out)
    _sync()
    assert np.all(f.lut.cpu().numpy() == np.arange(w.n_cubes))
    got = host64(out)
    if name == "small":
        with torch.no_grad():
            want = torch.nn.functional.scaled_dot_product_attention(
                *(torch.from_numpy(wl.as_float64(x[n])) for n in ("q", "k", "v"))).numpy()
        assert_out_close(got, want, "dense small")
    else:
        rng = np.random.default_rng(8)
        for h in (0, 11):
            toks = rng.choice(w.n_tokens, size=128, replace=False)
            q64, k64, v64 = (wl.as_float64(x[n][0, h]) for n in ("q", "k", "v"))
            s = q64[toks] @ k64.T / math.sqrt(w.head_dim)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            want = (e @ v64) / e.sum(axis=1, keepdims=True)
            assert_out_close(got[0, h, toks], want, f"dense wan head {h}")


# ------------------------------------------- LUT rows over half the cubes
# Rows that list at least half of the cubes take the fine kernel that walks
# four neighbouring query cubes together (their union of key cubes in steps,
# each step giving every cube at most one key cube).  Every feature of the
# fine stage on that path: grouped key/value heads, the Hilbert cube order,
# grids padded to whole cubes, gates with the coarse output, raster and
# model-layout outputs, LSE; rows with repeated entries (then the quad is
# walked position by position), empty rows and a last quad with fewer than
# four cubes.
WIDE = [((1, 4, 8, 16, 16, 4, 4, 4, 64), 2, "raster"), ((1, 2, 8, 16, 20, 4, 4, 4, 128), 0, "hilbert"),
        ((1, 3, 6, 10, 9, 4, 4, 4, 128), 3, "raster"), ((2, 2, 5, 7, 9, 4, 4, 4, 64), 1, "hilbert")]


@pytest.mark.parametrize("dims,hk,order", WIDE, ids=["8x16x16-d64-gqa2", "8x16x20-d128-hilbert",
                                                     "6x10x9-d128-padded", "5x7x9-d64-padded-hilbert-gqa"])
def test_sparse_attn_fwd_wide_rows(dims, hk, order):
    B, nh, T, H, W, ct, ch, cw, d = dims
    p = L.Problem(B, nh, T, H, W, ct, ch, cw, d, heads_kv=hk, cube_order=order)
    nc, hkv = p.n_cubes, p.kv_heads
    _log(f"sparse_attn_fwd wide rows {dims} kv heads {hkv} {order} ({nc} cubes)")
    pi = oracle.token_layout(T, H, W, ct, ch, cw, order)
    real = pi >= 0
    rng = np.random.default_rng(131)

    def bf(shape, uniform=False):
        a = rng.random(shape) if uniform else rng.standard_normal(shape)
        return wl.f32_to_bf16_bits(a.astype(np.float32))
    q = bf((B, nh, p.n_tokens, d))
    k, v = bf((B, hkv, p.n_tokens, d)), bf((B, hkv, p.n_tokens, d))
    gc, gf = bf((B, nh, p.n_tokens, d), True), bf((B, nh, p.n_tokens, d), True)
    oc = rng.standard_normal((B, nh, nc, d)).astype(np.float32)
    maxk = max(nc // 2 + 1, min(nc, 12))
    lut = np.stack([rng.permutation(nc)[:maxk] for _ in range(B * nh * nc)]).reshape(B, nh, nc, maxk)
    valid = rng.integers(maxk // 2, maxk + 1, size=(B, nh, nc))
    # sorted rows, unsorted rows, a row listing a cube twice, empty rows
    lut[..., ::2, :] = np.sort(lut[..., ::2, :], axis=-1)
    lut[0, 0, 1, :2] = lut[0, 0, 1, 2]
    valid[0, 0, 4:8] = 0
    valid[-1, -1, 3] = 0
    lut, valid = lut.astype(np.int32), valid.astype(np.int32)
    qp = dev(oracle.gather_padded(wl.as_float64(q), pi).astype(np.float32)).to(torch.bfloat16)
    kp = dev(oracle.gather_padded(wl.as_float64(k), pi).astype(np.float32)).to(torch.bfloat16)
    vp = dev(oracle.gather_padded(wl.as_float64(v), pi).astype(np.float32)).to(torch.bfloat16)
    rs = (B, nh, p.n_tokens, d)
    o_cube = torch.full((B, nh, p.n_positions, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_cube = torch.full((B, nh, p.n_positions), float("nan"), device="cuda")
    L.vsa_sparse_attn_fwd(p, qp, kp, vp, dev(lut), dev(valid), o_cube, lse=lse_cube)
    o_r = torch.full(rs, float("nan"), dtype=torch.bfloat16, device="cuda")
    L.vsa_sparse_attn_fwd_raster(p, qp, kp, vp, dev(lut), dev(valid), o_r, oc=dev(oc), gate_c=dev(gc),
                                 gate_f=dev(gf))
    o_b = torch.full((B, p.n_tokens, nh, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.vsa_sparse_attn_fwd_bnhd(p, qp, kp, vp, dev(lut), dev(valid), o_b, oc=dev(oc),
                               gate_c=dev(gc).permute(0, 2, 1, 3).contiguous(),
                               gate_f=dev(gf).permute(0, 2, 1, 3).contiguous())
    _sync()
    g = nh // hkv
    f64 = wl.as_float64
    kq = oracle.expand_kv_heads(oracle.gather_padded(f64(k), pi), g)
    vq = oracle.expand_kv_heads(oracle.gather_padded(f64(v), pi), g)
    of, lse = oracle.fine_attention(oracle.gather_padded(f64(q), pi), kq, vq, lut, valid, 1 / math.sqrt(d), 64,
                                    key_valid=real)
    rows = np.nonzero(real)[0]
    assert_out_close(host64(o_cube)[:, :, rows], of[:, :, rows], "cube-major O_f")
    empty = np.repeat(valid == 0, 64, axis=-1)
    assert np.all(host64(o_cube)[empty] == 0.0) and np.all(np.isneginf(host64(lse_cube)[empty]))
    full = ~empty & real[None, None, :]
    assert err(host64(lse_cube)[full], lse[full])[0] <= LSE_MAX_ABS
    outp = oracle.combine(of, oc.astype(np.float64), 64, oracle.gather_padded(f64(gc), pi),
                          oracle.gather_padded(f64(gf), pi))
    assert_out_close(host64(o_r)[:, :, pi[rows]], outp[:, :, rows], "raster out")
    assert np.array_equal(bits(o_b), bits(o_r.permute(0, 2, 1, 3).contiguous()))
