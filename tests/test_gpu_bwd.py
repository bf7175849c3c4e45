"""GPU parity of the fine-stage backward (vsa_sparse_attn_bwd) against the
fp64 oracle (oracle.fine_attention_bwd).

Inputs: Q, K, V are the seeded workload tensors in cube-major order (exact
bf16 bit gathers); O_f and LSE come from the oracle's forward on the same
LUT, rounded to bf16 / float32 and handed identically to both sides; dO is a
seeded N(0, 1) draw rounded to bf16.  Nothing the oracle sees comes from the
GPU.

Bar (from the arithmetic, not the pages, which give no backward tolerance):
the kernels round P and dS to bf16 as MFMA operands (relative rounding
2^-9) and accumulate in fp32.  Emulating exactly that rounding on the CPU
gives mean errors of about 0.2% of mean |grad| and max errors of 0.3-0.5% of
max |grad| on these workloads, so each gradient must satisfy
    max |got - ref| <= 2e-2 * max |ref|   and
    mean |got - ref| <= 1e-2 * mean |ref|,
about five times that.  Dropped terms, wrong signs or transposed operands
give errors of order one.  At the 32K-token size the GPU runs the whole launch
and the oracle checks sampled query cubes (dQ) and key cubes (dK, dV).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from gpu_helpers import bits, dev, host64, inputs, problem

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 2e-2
GRAD_MEAN_REL = 1e-2

MID = wl.Workload("mid", 8, 16, 32, (4, 4, 4), 1, 2, 128, "bf16", 16, 9, 8)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(f"\n[case] {msg}", flush=True)


def _bf16_bits(a):
    return wl.f32_to_bf16_bits(np.asarray(a, np.float32))


def _cube_major(w, heads=None):
    """Q, K, V of workload w as cube-major bf16 bits (exact gathers)."""
    x = inputs(w.name) if w.name in wl.WORKLOADS else wl.make_inputs(w)
    pi = oracle.perm_index(w.T, w.H, w.W, *w.cube)
    bf = (lambda a: a) if w.dtype == "bf16" else wl.f32_to_bf16_bits
    out = {n: np.take(bf(x[n]), pi, axis=2) for n in ("q", "k", "v")}
    if heads is not None:
        out = {n: np.ascontiguousarray(a[:, heads]) for n, a in out.items()}
    return out


def _random_lut(rng, shape, nc, k):
    lut = np.empty(shape + (k,), np.int32)
    for idx in np.ndindex(*shape):
        lut[idx] = np.sort(rng.permutation(nc)[:k])
    return lut


def _check(name, got, ref):
    g, r = host64(got), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    e = np.abs(g - r)
    mx_rel = e.max() / max(np.abs(r).max(), 1e-30)
    mean_rel = e.mean() / max(np.abs(r).mean(), 1e-30)
    print(f"{name}: max-abs {e.max():.3e} ({mx_rel:.2e} of max), mean-abs {e.mean():.3e} "
          f"({mean_rel:.2e} of mean)")
    assert mx_rel <= GRAD_MAX_REL and mean_rel <= GRAD_MEAN_REL, name


def _run_gpu(p, xp, lut, valid, of_bits, lse32, dof_bits, ws_extra=0):
    q, k, v = (dev(xp[n]) for n in ("q", "k", "v"))
    o, d_o = dev(of_bits), dev(dof_bits)
    lse = dev(lse32)
    lut_t, valid_t = dev(lut), dev(valid)
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    dk, dv = torch.full_like(dq, float("nan")), torch.full_like(dq, float("nan"))
    nbytes = L.vsa_sparse_attn_bwd_workspace_size(p, lut.shape[-1])
    ws = torch.full((nbytes + ws_extra,), 0xA5, dtype=torch.uint8, device="cuda")   # contents must not matter
    L.vsa_sparse_attn_bwd(p, q, k, v, lut_t, valid_t, o, lse, d_o, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def _full_case(w, lut, valid, seed):
    """Every gradient element of every head checked."""
    p = problem(w)
    xp = _cube_major(w)
    q64, k64, v64 = (wl.as_float64(xp[n]) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(w.head_dim)
    of, lse = oracle.fine_attention(q64, k64, v64, lut, valid, scale, 64)
    of_bits = _bf16_bits(of)
    lse32 = lse.astype(np.float32)
    rng = np.random.default_rng(seed)
    dof_bits = _bf16_bits(rng.standard_normal(q64.shape))
    dq, dk, dv = _run_gpu(p, xp, lut, valid, of_bits, lse32, dof_bits)
    ref = oracle.fine_attention_bwd(q64, k64, v64, lut, valid, scale, 64, wl.as_float64(of_bits),
                                    lse32.astype(np.float64), wl.as_float64(dof_bits))
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(f"{w.name} {name}", g, r)
    return (dq, dk, dv), ref


FULL = [("tiny", 2), ("tiny", 4), ("small", 8), ("small", 1), ("small", 32), ("mid", 16), ("mid", 64)]


@pytest.mark.parametrize("name,k", FULL, ids=[f"{n}-k{k}" for n, k in FULL])
def test_sparse_attn_bwd(name, k):
    w = MID if name == "mid" else wl.WORKLOADS[name]
    _log(f"sparse_attn_bwd {name} K={k} d={w.head_dim}")
    rng = np.random.default_rng(31 + k)
    lut = _random_lut(rng, (w.batch, w.heads, w.n_cubes), w.n_cubes, k)
    valid = np.full((w.batch, w.heads, w.n_cubes), k, np.int32)
    _full_case(w, lut, valid, seed=41 + k)


def test_sparse_attn_bwd_variable_rows():
    """Counts 0..max, unsorted and repeated entries, max_kv above the counts;
    unlisted key cubes get dK = dV = 0 and empty rows dQ = 0."""
    w = wl.SMALL
    _log("sparse_attn_bwd variable LUT rows")
    rng = np.random.default_rng(22)
    maxk = 12
    lut = rng.integers(0, w.n_cubes, size=(1, w.heads, w.n_cubes, maxk)).astype(np.int32)
    valid = rng.integers(0, maxk + 1, size=(1, w.heads, w.n_cubes)).astype(np.int32)
    valid[0, 0, :4] = 0
    valid[0, 1, :4] = maxk
    lut[0, 2, 0, :3] = 5                       # a cube listed three times by one row
    lut[0, 3] = np.where(lut[0, 3] == 7, 8, lut[0, 3])   # key cube 7 of head 3 never listed
    (dq, dk, dv), _ = _full_case(w, lut, valid, seed=23)
    dqh, dkh, dvh = host64(dq), host64(dk), host64(dv)
    empty = np.repeat(valid == 0, 64, axis=-1)
    assert np.all(dqh[empty] == 0.0)
    assert np.all(dkh[0, 3, 7 * 64:8 * 64] == 0.0) and np.all(dvh[0, 3, 7 * 64:8 * 64] == 0.0)


def test_sparse_attn_bwd_wan_sampled():
    """The 32,768-token, 12-head, d = 128 layer at Top-K 154 as one launch;
    the oracle checks sampled query cubes and key cubes of two heads."""
    w = wl.WAN
    _log("sparse_attn_bwd wan K=154 (sampled)")
    p = problem(w)
    xp = _cube_major(w)
    k = w.top_k
    scale = 1.0 / math.sqrt(w.head_dim)
    rng = np.random.default_rng(51)
    lut = _random_lut(rng, (1, w.heads, w.n_cubes), w.n_cubes, k)
    valid = np.full((1, w.heads, w.n_cubes), k, np.int32)
    heads = [0, 7]
    dq_cubes = [0, 1, 200, w.n_cubes - 1]
    key_cubes = {0: 3, 7: w.n_cubes - 2}      # one key cube per checked head
    # query cubes whose values the checked outputs depend on
    need = {h: sorted(set(dq_cubes) | {i for i in range(w.n_cubes) if key_cubes[h] in lut[0, h, i, :k]})
            for h in heads}
    q64, k64, v64 = (wl.as_float64(xp[n]) for n in ("q", "k", "v"))
    todo = [(0, h, i) for h in heads for i in need[h]]
    of, lse = oracle.fine_attention(q64, k64, v64, lut, valid, scale, 64, query_cubes=todo)
    # rows the checks do not depend on get finite seeded stand-ins
    filler = np.ones((1, w.heads, w.n_cubes), bool)
    for h in heads:
        filler[0, h, need[h]] = False
    fill_tok = np.repeat(filler, 64, axis=-1)
    of[fill_tok] = rng.standard_normal((int(fill_tok.sum()), w.head_dim)) * 0.1
    lse[fill_tok] = 8.0
    of_bits = _bf16_bits(of)
    lse32 = lse.astype(np.float32)
    dof_bits = _bf16_bits(rng.standard_normal(q64.shape).astype(np.float32))
    dq, dk, dv = _run_gpu(p, xp, lut, valid, of_bits, lse32, dof_bits)
    dqh, dkh, dvh = host64(dq), host64(dk), host64(dv)
    for h in heads:
        sub = np.zeros((1, 1, w.n_cubes), np.int32)
        sub[0, 0, need[h]] = k                  # only the needed rows contribute
        ref = oracle.fine_attention_bwd(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1], lut[:, h:h + 1],
                                        sub, scale, 64, wl.as_float64(of_bits[:, h:h + 1]),
                                        lse32[:, h:h + 1].astype(np.float64),
                                        wl.as_float64(dof_bits[:, h:h + 1]))
        qrows = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in dq_cubes])
        krows = np.arange(key_cubes[h] * 64, key_cubes[h] * 64 + 64)
        _check(f"wan h{h} dq", torch.from_numpy(dqh[0, h, qrows]), ref[0][0, 0, qrows])
        _check(f"wan h{h} dk", torch.from_numpy(dkh[0, h, krows]), ref[1][0, 0, krows])
        _check(f"wan h{h} dv", torch.from_numpy(dvh[0, h, krows]), ref[2][0, 0, krows])
    assert np.all(np.isfinite(dqh)) and np.all(np.isfinite(dkh)) and np.all(np.isfinite(dvh))


def test_sparse_attn_bwd_deterministic():
    """No atomics on the gradients: two calls give identical bits, whatever
    the workspace held before."""
    w = MID
    _log("sparse_attn_bwd determinism")
    p = problem(w)
    xp = _cube_major(w)
    rng = np.random.default_rng(61)
    lut = _random_lut(rng, (1, w.heads, w.n_cubes), w.n_cubes, 24)
    valid = np.full((1, w.heads, w.n_cubes), 24, np.int32)
    of_bits = _bf16_bits(rng.standard_normal(xp["q"].shape) * 0.3)
    lse32 = (np.full((1, w.heads, w.n_tokens), 9.0) + rng.random((1, w.heads, w.n_tokens))).astype(np.float32)
    dof_bits = _bf16_bits(rng.standard_normal(xp["q"].shape))
    a = _run_gpu(p, xp, lut, valid, of_bits, lse32, dof_bits)
    b = _run_gpu(p, xp, lut, valid, of_bits, lse32, dof_bits, ws_extra=4096)
    for x, y in zip(a, b):
        assert np.array_equal(bits(x), bits(y))


def test_sparse_attn_bwd_errors_leave_outputs_untouched():
    w = wl.SMALL
    _log("sparse_attn_bwd argument errors")
    p = problem(w)
    shape = (1, w.heads, w.n_tokens, w.head_dim)
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, w.heads, w.n_tokens), device="cuda")
    lut = torch.zeros((1, w.heads, w.n_cubes, 4), dtype=torch.int32, device="cuda")
    valid = torch.full((1, w.heads, w.n_cubes), 4, dtype=torch.int32, device="cuda")
    dq = torch.full(shape, 7.0, device="cuda")
    dk, dv = dq.clone(), dq.clone()
    need = L.vsa_sparse_attn_bwd_workspace_size(p, 4)
    small_ws = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.VsaError) as ei:
        L.vsa_sparse_attn_bwd(p, q, q, q, lut, valid, q, lse, q, dq, dk, dv, small_ws)
    assert ei.value.status == L.VSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool((t == 7.0).all())
