"""GPU parity of vsa_combine, the gated combination as a pass of its own
("VSA: Accelerating Video Diffusion Inference with Sparse Attention on AMD
GPUs", §Two-Stage Architecture: the output combines the coarse and fine
outputs through gates).

The pass forms g_f * O_f (bf16 times bf16: exact in float32), then one fused
multiply-add with g_c * O_c, and rounds to bf16.  The reference below forms the
same value exactly in float64 (the product g_c * O_c has at most 32 significant
bits and the sum stays exact for these magnitudes), rounds it once to float32
(what the fused multiply-add returns) and then to bf16 with round-to-nearest-
even: so the comparison is bit for bit.  Without gates the pass must equal
vsa_unpermute of O_f.  Inputs are seeded draws; the token order comes from the
oracle's permutation.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from gpu_helpers import bits, dev, problem

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


def _bf16(a):
    return wl.f32_to_bf16_bits(np.asarray(a, np.float32))


CASES = [
    ("small", wl.SMALL, dict()),
    ("wan-2heads", wl.WAN, dict(heads=2)),
    ("padded-5x7x9", wl.SMALL, dict(T=5, H=7, W=9, heads=2)),
    ("wan-dv64", wl.WAN, dict(head_dim_v=64, heads=2)),
]


@pytest.mark.parametrize("name,w,repl", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("gates", ["both", "f", "c", "none"])
def test_combine(name, w, repl, gates):
    _log(f"vsa_combine {name} gates={gates}")
    p = dataclasses.replace(problem(w), **repl)
    rng = np.random.default_rng([ord(ch) for ch in name + gates])
    dv = p.v_dim
    of_bits = _bf16(rng.standard_normal((p.batch, p.heads, p.n_positions, dv)))
    oc = rng.standard_normal((p.batch, p.heads, p.n_cubes, dv)).astype(np.float32)
    gc_bits = _bf16(rng.random((p.batch, p.heads, p.n_tokens, dv))) if gates in ("both", "c") else None
    gf_bits = _bf16(rng.random((p.batch, p.heads, p.n_tokens, dv))) if gates in ("both", "f") else None
    out = torch.full((p.batch, p.heads, p.n_tokens, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.vsa_combine(p, dev(of_bits), out, oc=dev(oc) if gc_bits is not None else None,
                  gate_c=dev(gc_bits) if gc_bits is not None else None,
                  gate_f=dev(gf_bits) if gf_bits is not None else None)
    torch.cuda.synchronize()
    got = bits(out)

    # reference: token at cube-major position pos goes to raster row perm[pos]
    perm = oracle.token_layout(p.T, p.H, p.W, p.ct, p.ch, p.cw)   # -1 at padded positions
    real = perm >= 0
    cube_of = np.arange(p.n_positions) // (p.ct * p.ch * p.cw)
    o = wl.bf16_bits_to_f32(of_bits).astype(np.float64)[:, :, real]
    val = o
    if gf_bits is not None:
        gf = wl.bf16_bits_to_f32(gf_bits).astype(np.float64)[:, :, perm[real]]
        val = val * gf                                   # exact: 8-bit by 8-bit significands
    if gc_bits is not None:
        gc = wl.bf16_bits_to_f32(gc_bits).astype(np.float64)[:, :, perm[real]]
        val = gc * oc.astype(np.float64)[:, :, cube_of[real]] + val
    want = np.empty((p.batch, p.heads, p.n_tokens, dv), np.uint16)
    want[:, :, perm[real]] = _bf16(val.astype(np.float32))
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} elements differ"

    if gates == "none":
        back = torch.empty_like(out)
        pv = dataclasses.replace(p, head_dim=dv, head_dim_v=0)
        L.vsa_unpermute(pv, L.VSA_BF16, dev(of_bits), back)
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(back))
