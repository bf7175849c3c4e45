"""Helpers shared by the GPU parity tests: host<->device transfer of workload
arrays, error metrics and the tie-tolerant comparison of Top-K cube sets."""
from __future__ import annotations

import functools

import numpy as np
import torch

from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd import _lib as L

# Attention outputs (bf16 in, fp32 accumulate): the stated acceptance bar.
OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 2e-3
# Natural-log LSE of fp32 online softmax: fp32 rounding of ~d-term dot
# products times the scale, far below this bound.
LSE_MAX_ABS = 1e-3
# Coarse output O_c (fp32 throughout).
OC_MAX_ABS = 1e-4
# Top-K: a set difference is allowed only among scores within this relative
# window of the K-th largest oracle score.
TIE_REL = 1e-5


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Workload array -> device tensor (uint16 bf16 bits become bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for bf16 and float32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return wl.bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def err(got: np.ndarray, want: np.ndarray):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_out_close(got, want, what=""):
    mx, mean = err(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= OUT_MAX_ABS and mean <= OUT_MEAN_ABS, f"{what}: max-abs {mx:.3e}, mean-abs {mean:.3e}"
    return mx, mean


def check_lut_against_scores(lut: np.ndarray, valid: np.ndarray, scores: np.ndarray, k: int,
                             oracle_lut: np.ndarray):
    """Every GPU row: k distinct ascending indices in range, valid == k, and
    equal to the oracle's set except for swaps among near-ties of the K-th
    largest score.  Returns the number of rows that differ (all within the
    tie window)."""
    nc = scores.shape[-1]
    assert lut.shape == scores.shape[:-1] + (k,)
    assert np.all(valid == k)
    assert np.all((lut >= 0) & (lut < nc))
    assert np.all(np.diff(lut, axis=-1) > 0), "rows must be strictly ascending"
    differ = 0
    flat_s = scores.reshape(-1, nc)
    flat_g = lut.reshape(-1, k)
    flat_o = oracle_lut.reshape(-1, k)
    for r in range(flat_s.shape[0]):
        g, o = set(flat_g[r].tolist()), set(flat_o[r].tolist())
        if g == o:
            continue
        differ += 1
        row = flat_s[r]
        s_k = np.sort(row)[::-1][k - 1]
        tol = TIE_REL * max(1.0, abs(s_k))
        for j in g - o:
            assert row[j] >= s_k - tol, f"row {r}: extra cube {j} score {row[j]} vs s_K {s_k}"
        for j in o - g:
            assert row[j] <= s_k + tol, f"row {r}: missing cube {j} score {row[j]} vs s_K {s_k}"
    return differ


@functools.lru_cache(maxsize=4)
def _inputs(name: str):
    return wl.make_inputs(wl.WORKLOADS[name], with_gates=True, workers=16)


def inputs(name: str, with_gates: bool = True):
    """Seeded workload inputs (cached).  The gates are drawn after V, so Q, K
    and V are the same whether or not gates are requested; they are always
    generated and simply ignored by callers that do not use them."""
    return _inputs(name)


def problem(w: wl.Workload) -> L.Problem:
    return L.Problem(w.batch, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim)
