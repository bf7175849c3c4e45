"""Seeded synthetic workloads for the VSA forward path.

This module only *draws inputs*: it holds none of the attention arithmetic, so
both the fp64 CPU oracle (``oracle/``) and the HIP path can be fed from it
without sharing any of the method's code.

Shapes and the value distributions stand in for the activations of the
Wan2.1-T2V-1.3B attention layer described on the page "VSA: Accelerating Video
Diffusion Inference with Sparse Attention on AMD GPUs" (AMD ROCm blog),
§Performance Benchmarks and §Appendix - Tensor Specifications: Q/K/V of shape
[1, 12, 32768, 128] in bf16.  Real activations and weights are not used.

Recipe (identical for every consumer):

* For every (batch b, head h) in that order a fresh generator
  ``numpy.random.default_rng(SeedSequence([seed, b, h]))`` (PCG64) is used,
  so any subset of heads can be regenerated on its own.
* Plain configs draw Zq, Zk, Zv ~ N(0, 1) of shape (T, H, W, d) in float32,
  and Q = Zq, K = Zk, V = Zv.
* Locality configs first draw a coarse Gaussian grid G of shape
  (ceil(T/s)+1, ceil(H/s)+1, ceil(W/s)+1, d), upsample it trilinearly to the
  token grid (node n sits at token n*s) to get a smooth field F, then draw
  Zq, Zk, Zv and set Q = 0.5*Zq + F, K = 0.5*Zk + F, V = Zv.  Q and K share
  the field, so coarse cube-to-cube scores peak between nearby cubes.
* Optional gates g_c, g_f ~ U(0, 1) are drawn after V.
* bf16 configs round every float32 value to bf16 with round-to-nearest-even;
  the oracle and the GPU consume the identical rounded values.

Tensors are returned in the caller-facing raster layout [B, heads, N, d] with
token index n = (t*H + h)*W + w.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    cube: tuple
    batch: int
    heads: int
    head_dim: int
    dtype: str            # "bf16" or "f32"
    top_k: int
    seed: int
    field_stride: Optional[int]   # None: plain N(0,1) Q/K/V

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def cube_volume(self) -> int:
        ct, ch, cw = self.cube
        return ct * ch * cw

    @property
    def n_cubes(self) -> int:
        return self.n_tokens // self.cube_volume

    @property
    def sparsity(self) -> float:
        return 1.0 - self.top_k / self.n_cubes

    def with_top_k(self, k: int) -> "Workload":
        return dataclasses.replace(self, top_k=k, name=f"{self.name}_k{k}")

    def selected_flops(self, top_k: Optional[int] = None) -> int:
        """Attention FLOPs over selected (query cube, key cube) pairs only:
        2*vol*vol*d for Q.K^T plus the same for P.V, per pair."""
        k = self.top_k if top_k is None else top_k
        v = self.cube_volume
        return 4 * self.batch * self.heads * self.n_tokens * v * k * self.head_dim


# The five workloads: a tiny fp32 grid the oracle finishes instantly, a small
# bf16 grid, the 32,768-token Wan2.1-scale layer at 70% sparsity (154 of 512
# cubes), the sparsity sweep on that shape, and a 122,880-token large layer.
TINY = Workload("tiny", 4, 8, 8, (4, 4, 4), 1, 1, 64, "f32", 2, 0, None)
SMALL = Workload("small", 8, 16, 16, (4, 4, 4), 1, 4, 64, "bf16", 8, 1, 4)
WAN = Workload("wan", 16, 32, 64, (4, 4, 4), 1, 12, 128, "bf16", 154, 2, 8)
SWEEP_TOPK = (256, 154, 102, 51, 512)
LARGE = Workload("large", 32, 48, 80, (4, 4, 4), 1, 40, 128, "bf16", 192, 3, 8)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in (TINY, SMALL, WAN, LARGE)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _lerp_axis(g: np.ndarray, n_out: int, s: int, axis: int) -> np.ndarray:
    idx = np.arange(n_out)
    i0 = idx // s
    f = ((idx % s).astype(np.float32) / np.float32(s))
    shape = [1] * g.ndim
    shape[axis] = n_out
    f = f.reshape(shape)
    a = np.take(g, i0, axis=axis)
    b = np.take(g, i0 + 1, axis=axis)
    return (np.float32(1) - f) * a + f * b


def smooth_field(rng: np.random.Generator, T: int, H: int, W: int, d: int, s: int) -> np.ndarray:
    """Trilinear upsample of a stride-s Gaussian grid to (T, H, W, d), float32."""
    nt, nh, nw = -(-T // s) + 1, -(-H // s) + 1, -(-W // s) + 1
    g = rng.standard_normal((nt, nh, nw, d), dtype=np.float32)
    g = _lerp_axis(g, T, s, 0)
    g = _lerp_axis(g, H, s, 1)
    g = _lerp_axis(g, W, s, 2)
    return g


def draw_head(w: Workload, b: int, h: int, with_gates: bool = False) -> Dict[str, np.ndarray]:
    """float32 (T*H*W, d) arrays for one (batch, head), before any rounding."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h]))
    T, H, W, d = w.T, w.H, w.W, w.head_dim
    out = {}
    if w.field_stride is None:
        q = rng.standard_normal((T, H, W, d), dtype=np.float32)
        k = rng.standard_normal((T, H, W, d), dtype=np.float32)
        v = rng.standard_normal((T, H, W, d), dtype=np.float32)
    else:
        f = smooth_field(rng, T, H, W, d, w.field_stride)
        half = np.float32(0.5)
        q = half * rng.standard_normal((T, H, W, d), dtype=np.float32) + f
        k = half * rng.standard_normal((T, H, W, d), dtype=np.float32) + f
        v = rng.standard_normal((T, H, W, d), dtype=np.float32)
    out["q"], out["k"], out["v"] = q, k, v
    if with_gates:
        out["gate_c"] = rng.random((T, H, W, d), dtype=np.float32)
        out["gate_f"] = rng.random((T, H, W, d), dtype=np.float32)
    return {n: a.reshape(T * H * W, d) for n, a in out.items()}


def make_inputs(w: Workload, with_gates: bool = False,
                heads: Optional[Sequence[int]] = None,
                batches: Optional[Sequence[int]] = None,
                workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs in raster layout [B', heads', N, d].

    For bf16 workloads the arrays are uint16 bf16 bits; for f32 workloads they
    are float32.  ``heads`` / ``batches`` select a subset (defaults: all); the
    values of a selected head do not depend on which others are selected, nor
    on ``workers`` (heads are drawn in parallel threads, each from its own
    seeded generator).
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    names = ["q", "k", "v"] + (["gate_c", "gate_f"] if with_gates else [])
    N, d = w.n_tokens, w.head_dim
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    res = {n: np.empty((len(batches), len(heads), N, d), dtype=dt) for n in names}

    def one(job):
        bi, b, hi, h = job
        x = draw_head(w, b, h, with_gates)
        for n in names:
            res[n][bi, hi] = f32_to_bf16_bits(x[n]) if w.dtype == "bf16" else x[n]

    jobs = [(bi, b, hi, h) for bi, b in enumerate(batches) for hi, h in enumerate(heads)]
    if workers is None:
        workers = min(len(jobs), 8, os.cpu_count() or 1)
    if workers <= 1:
        for j in jobs:
            one(j)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, jobs))
    return res


def as_float64(a: np.ndarray) -> np.ndarray:
    """Exact float64 view of a workload array (bf16 bits or float32)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def block_relation_mask(w: Workload, k_importance: int, n_condition: int, seed: int = 4) -> np.ndarray:
    """A block relation matrix of the kind a block-mask method hands to the
    fine stage (page "VSA: Accelerating Video Diffusion Inference with Sparse
    Attention on AMD GPUs", §Comparison with Jenga: the union of an
    importance mask, a condition mask and an adjacency mask).  Shape
    [B, heads, Nc, Nc], uint8, 1 = query cube i attends key cube j.  Purely
    structural stand-ins, drawn per (batch, head) like the activations:

    * importance: k_importance cubes per row chosen uniformly at random;
    * condition: cubes 0 .. n_condition - 1 for every row (stands in for the
      blocks that carry the text-condition tokens; this token grid has none);
    * adjacency: every cube within one cube step in t, h and w (the 3 x 3 x 3
      neighbourhood in the cube grid, clipped at the edges).

    Row counts therefore vary from row to row.
    """
    gT, gH, gW = w.T // w.cube[0], w.H // w.cube[1], w.W // w.cube[2]
    nc = gT * gH * gW
    t, h, x = np.meshgrid(np.arange(gT), np.arange(gH), np.arange(gW), indexing="ij")
    t, h, x = t.ravel(), h.ravel(), x.ravel()
    adj = ((np.abs(t[:, None] - t[None, :]) <= 1) & (np.abs(h[:, None] - h[None, :]) <= 1)
           & (np.abs(x[:, None] - x[None, :]) <= 1))
    out = np.zeros((w.batch, w.heads, nc, nc), dtype=np.uint8)
    for b in range(w.batch):
        for hh in range(w.heads):
            rng = np.random.default_rng(np.random.SeedSequence([seed, b, hh]))
            imp = np.argsort(rng.random((nc, nc)), axis=1)[:, :k_importance]
            m = adj.copy()
            np.put_along_axis(m, imp, True, axis=1)
            m[:, :n_condition] = True
            out[b, hh] = m
    return out
