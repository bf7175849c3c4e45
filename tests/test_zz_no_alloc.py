"""GPU test of vsa_sparse_attn_bwd_noalloc, the backward entry point that
allocates nothing (its workspace is the library's fixed per-GPU array):
called through the C ABI twice in a row, the second time on a smaller
problem (so it runs on the first call's leftover workspace contents), each
time bit-identical to vsa_sparse_attn_bwd with a caller workspace on the same
inputs (the backward is deterministic: no atomics touch dq, dk, dv)."""
import numpy as np
import pytest
import torch

from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaForward
from gpu_helpers import bits, dev, problem

pytestmark = pytest.mark.gpu

# 8 x 16 x 32 tokens, 2 heads, d = 128, Top-16 of 64 cubes; then the small
# workload (8 x 16 x 16 tokens, 4 heads, d = 64, Top-8 of 32 cubes)
MID = wl.Workload("mid", 8, 16, 32, (4, 4, 4), 1, 2, 128, "bf16", 16, 9, 8)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _case(w, seed):
    p = problem(w)
    x = wl.make_inputs(w)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    f = VsaForward(p, w.top_k)
    out = torch.empty_like(q)
    f(q, k, v, out)
    o_f = torch.empty_like(f.qp)
    lse = torch.empty((w.batch, w.heads, p.n_positions), device="cuda")
    L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse=lse)
    rng = np.random.default_rng(seed)
    d_o = dev(wl.f32_to_bf16_bits(rng.standard_normal(o_f.shape).astype(np.float32)))
    ref = [torch.full(f.qp.shape, float("nan"), device="cuda") for _ in range(3)]
    ws = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(p, w.top_k), dtype=torch.uint8, device="cuda")
    got = [torch.full(f.qp.shape, float("nan"), device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    return p, f, o_f, lse, d_o, ref, ws, got


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [_case(MID, 41), _case(wl.SMALL, 42)]   # every buffer allocated before the calls
    for (p, f, o_f, lse, d_o, ref, ws, got), name in zip(cases, ("8x16x32 d128", "8x16x16 d64")):
        print(f"\n[case] noalloc backward {name}", flush=True)
        L.vsa_sparse_attn_bwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse, d_o, *ref, ws)
        L.vsa_sparse_attn_bwd_noalloc(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse, d_o, *got)
        torch.cuda.synchronize()
        for nm, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert np.all(np.isfinite(a.cpu().numpy())), nm
            assert np.array_equal(bits(a), bits(b)), f"{name}: {nm} differs from vsa_sparse_attn_bwd"
