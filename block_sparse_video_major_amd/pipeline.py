"""The whole VSA forward pass, and its backward, as sequences of C-ABI calls.

Order of the steps ("VSA: Accelerating Video Diffusion Inference with Sparse
Attention on AMD GPUs", §Two-Stage Architecture): reorder tokens into cubes
and mean-pool them (one fused pass per tensor), coarse cube attention with
Top-K selection, fine block-sparse attention over the selected cubes combined
with the coarse output through the gates, written straight back in the
model's token order (the reorder back runs in the fine kernel's epilogue).
Where the shapes allow, the reorder runs in the fine kernel's tile loads
instead (it gathers every cube from the raster rows), and the first pass
only pools.
The backward ("VSA: Faster Video Diffusion with Trainable Sparse
Attention", Abstract: trained end to end) takes those steps in reverse with
the index list held fixed.  This module only allocates the intermediate
buffers (through torch) and calls the library; every step runs in the HIP
kernels of libvsa.so.
"""
from __future__ import annotations

import collections
import dataclasses
import threading
from typing import Dict, Optional

import torch

from . import _lib as L
from ._lib import Problem


def gather_supported(p: Problem) -> bool:
    """Whether vsa_sparse_attn_fwd_gather takes this problem's shapes: head
    sizes 128, cubes of 64 tokens 4 wide, a grid that divides into cubes (the
    LUT row length is checked by the library at the call)."""
    return (p.head_dim == 128 and p.v_dim == 128 and p.cw == 4 and p.cube_volume == 64 and not p.padded)


class VsaForward:
    """Preallocated buffers for one problem size; call() runs one forward pass."""

    def __init__(self, p: Problem, top_k: int, device="cuda", with_gates: bool = False,
                 with_lse: bool = False, layout: str = "bhnd", gather: bool = False):
        # with_gates is accepted for callers that pass gates; the raster-order
        # gates are read directly, so no buffer is needed for them.  lse (if
        # kept) is in raster token order.  layout "bnhd" takes q, k, v, the
        # gates and out in the model's [batch, N, heads, d] order.  With
        # gather, no cube-major copies of q, k, v are made: the pool reads the
        # raster rows and the fine stage gathers its cube tiles from them
        # (vsa_sparse_attn_fwd_gather; see gather_supported).
        if not 1 <= top_k <= p.n_cubes:
            raise ValueError(f"top_k={top_k} outside [1, {p.n_cubes}]")
        if layout not in ("bhnd", "bnhd"):
            raise ValueError(f"layout {layout!r} is not 'bhnd' or 'bnhd'")
        if gather and (layout != "bhnd" or not gather_supported(p)):
            raise ValueError("the gathering fine stage needs the [batch, heads, N, d] layout, head sizes 128, "
                             "cubes 4 tokens wide and a grid that divides into cubes")
        self.p, self.top_k, self.layout, self.gather = p, top_k, layout, gather
        ts = (p.batch, p.heads, p.n_positions, p.head_dim)   # cube-major (padded) rows
        cs = (p.batch, p.heads, p.n_cubes, p.head_dim)
        kts = (p.batch, p.kv_heads, p.n_positions, p.head_dim)
        kcs = (p.batch, p.kv_heads, p.n_cubes, p.head_dim)
        vts = (p.batch, p.kv_heads, p.n_positions, p.v_dim)   # values may be narrower or wider
        vcs = (p.batch, p.kv_heads, p.n_cubes, p.v_dim)
        bf, f32 = torch.bfloat16, torch.float32
        self.qp = None if gather else torch.empty(ts, dtype=bf, device=device)
        self.kp = None if gather else torch.empty(kts, dtype=bf, device=device)
        self.vp = None if gather else torch.empty(vts, dtype=bf, device=device)
        self.qc = torch.empty(cs, dtype=f32, device=device)
        self.oc = torch.empty((p.batch, p.heads, p.n_cubes, p.v_dim), dtype=f32, device=device)
        self.kc = torch.empty(kcs, dtype=f32, device=device)
        self.vc = torch.empty(vcs, dtype=f32, device=device)
        self.lut = torch.empty((p.batch, p.heads, p.n_cubes, top_k), dtype=torch.int32, device=device)
        self.valid = torch.empty((p.batch, p.heads, p.n_cubes), dtype=torch.int32, device=device)
        self.lse = torch.empty((p.batch, p.heads, p.n_tokens), dtype=f32, device=device) if with_lse else None

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                 gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
        p, B = self.p, L.VSA_BF16
        bnhd = self.layout == "bnhd"
        permute_pool = L.vsa_permute_pool_bnhd if bnhd else L.vsa_permute_pool
        # K and V may have fewer (grouped) heads, and V its own head size
        permute_pool(p, B, q, self.qp, self.qc, stream)   # the cube-major copy is None when gathering
        permute_pool(p.kv_problem(), B, k, self.kp, self.kc, stream)
        permute_pool(p.v_problem(), B, v, self.vp, self.vc, stream)
        L.vsa_coarse_topk(p, self.top_k, self.qc, self.kc, self.vc, self.lut, self.valid, self.oc, stream)
        # fine attention reading the raster-order gates and writing the
        # raster-order output directly (the reorder back is in its epilogue)
        if self.gather:   # q, k, v themselves: the fine kernel gathers their cubes
            L.vsa_sparse_attn_fwd_gather(p, q, k, v, self.lut, self.valid, out,
                                         oc=self.oc, gate_c=gate_c, gate_f=gate_f, lse=self.lse, stream=stream)
            return out
        fine = L.vsa_sparse_attn_fwd_bnhd if bnhd else L.vsa_sparse_attn_fwd_raster
        fine(p, self.qp, self.kp, self.vp, self.lut, self.valid, out,
             oc=self.oc, gate_c=gate_c, gate_f=gate_f, lse=self.lse, stream=stream)
        return out

    def intermediates(self) -> Dict[str, torch.Tensor]:
        d = dict(qc=self.qc, kc=self.kc, vc=self.vc, oc=self.oc, kv_block_idx=self.lut,
                 valid_block_num=self.valid)
        if not self.gather:
            d.update(qp=self.qp, kp=self.kp, vp=self.vp)
        if self.lse is not None:
            d["lse"] = self.lse
        return d


# Buffers of vsa_forward, per calling thread, kept for the last few (problem,
# Top-K, device, stream) keys: successive calls on one stream are ordered by
# that stream, so they may share intermediates; calls on other streams or
# threads get buffers of their own.
_FORWARD_CACHE_SIZE = 4
# LUT rows of up to this many cubes always fit the gathering pair kernel's
# on-chip schedule (28 bytes per entry beside the tile ring and the zero tile)
_GATHER_MAX_KV = 512
_forward_cache = threading.local()


def _cached_forward(p: Problem, top_k: int, device: torch.device, stream) -> "VsaForward":
    # raster inputs the fine stage can gather from need no cube-major copies
    cache = getattr(_forward_cache, "entries", None)
    if cache is None:
        cache = _forward_cache.entries = collections.OrderedDict()
    key = (p, top_k, str(device), L._stream(stream, device))
    f = cache.get(key)
    if f is None:
        f = VsaForward(p, top_k, device, gather=gather_supported(p) and top_k <= _GATHER_MAX_KV)
        cache[key] = f
        while len(cache) > _FORWARD_CACHE_SIZE:
            cache.popitem(last=False)
    else:
        cache.move_to_end(key)
    return f


def clear_forward_cache() -> None:
    """Drop the calling thread's cached vsa_forward buffers."""
    _forward_cache.entries = collections.OrderedDict()


def vsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Problem, top_k: int,
                gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """One VSA forward pass on raster bf16 inputs [B, heads, N, d].  The
    intermediates (pooled tensors, the index list, and cube-major copies of
    q, k, v unless the fine stage gathers its cubes from the raster rows: see
    gather_supported) live in buffers reused by later calls with the same
    problem on the same stream and thread; the returned output is a new
    tensor."""
    if not 1 <= top_k <= p.n_cubes:
        raise ValueError(f"top_k={top_k} outside [1, {p.n_cubes}]")
    f = _cached_forward(p, top_k, q.device, stream)
    out = q.new_empty(q.shape[:-1] + (p.v_dim,))
    return f(q, k, v, out, gate_c, gate_f, stream)


class VsaBackward:
    """Buffers for the backward of one layer; call() runs it.

    Inputs are the forward's cube-major intermediates (qp, kp, vp, qc, kc, vc,
    oc, the LUT and counts), O_f and its LSE (cube-major: vsa_sparse_attn_fwd
    without gates), and the raster-order upstream gradient dout and gates.
    Outputs are the raster-order float32 gradients of q, k, v and the gates.
    Steps: reorder dout and the gates into cubes, combine backward, fine
    backward, coarse backward, then the reorder back with each pooled
    gradient added."""

    def __init__(self, p: Problem, max_kv: int, device="cuda"):
        self.p = p
        # the output side (dout, the gates, O) is as wide as V
        self.p_out = dataclasses.replace(p, head_dim=p.v_dim, head_dim_v=0)
        dv_ = p.v_dim
        ts = (p.batch, p.heads, p.n_positions, p.head_dim)   # cube-major (padded) rows
        tvs = (p.batch, p.heads, p.n_positions, dv_)
        cs = (p.batch, p.heads, p.n_cubes, p.head_dim)
        kts = (p.batch, p.kv_heads, p.n_positions, p.head_dim)
        kcs = (p.batch, p.kv_heads, p.n_cubes, p.head_dim)
        bf, f32 = torch.bfloat16, torch.float32
        self.doutp, self.gcp, self.gfp, self.d_of = (torch.empty(tvs, dtype=bf, device=device) for _ in range(4))
        self.dgcp, self.dgfp = (torch.empty(tvs, dtype=f32, device=device) for _ in range(2))
        self.dqf = torch.empty(ts, dtype=f32, device=device)
        self.dkf = torch.empty(kts, dtype=f32, device=device)
        self.dvf = torch.empty((p.batch, p.kv_heads, p.n_positions, dv_), dtype=f32, device=device)
        self.d_oc = torch.empty((p.batch, p.heads, p.n_cubes, dv_), dtype=f32, device=device)
        self.dqc = torch.empty(cs, dtype=f32, device=device)
        self.dkc = torch.empty(kcs, dtype=f32, device=device)
        self.dvc = torch.empty((p.batch, p.kv_heads, p.n_cubes, dv_), dtype=f32, device=device)
        self.ws_fine = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(p, max_kv), dtype=torch.uint8,
                                   device=device)
        self.ws_coarse = torch.empty(L.vsa_coarse_bwd_workspace_size(p), dtype=torch.uint8, device=device)

    def __call__(self, saved: Dict[str, torch.Tensor], o_f: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                 dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                 gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                 dgate_c: Optional[torch.Tensor] = None, dgate_f: Optional[torch.Tensor] = None,
                 stream=None) -> None:
        p, po, B = self.p, self.p_out, L.VSA_BF16
        L.vsa_permute(po, B, dout, self.doutp, stream)
        gcp = gfp = None
        if gate_c is not None:
            L.vsa_permute(po, B, gate_c, self.gcp, stream)
            gcp = self.gcp
        if gate_f is not None:
            L.vsa_permute(po, B, gate_f, self.gfp, stream)
            gfp = self.gfp
        L.vsa_combine_bwd(p, self.doutp, self.d_of, self.d_oc, o_f=o_f, oc=saved["oc"], gate_c=gcp, gate_f=gfp,
                          d_gate_c=self.dgcp if gcp is not None else None,
                          d_gate_f=self.dgfp if gfp is not None else None, stream=stream)
        L.vsa_sparse_attn_bwd(p, saved["qp"], saved["kp"], saved["vp"], saved["kv_block_idx"],
                              saved["valid_block_num"], o_f, lse, self.d_of, self.dqf, self.dkf, self.dvf,
                              self.ws_fine, stream)
        L.vsa_coarse_bwd(p, saved["qc"], saved["kc"], saved["vc"], saved["oc"], self.d_oc, self.dqc, self.dkc,
                         self.dvc, self.ws_coarse, stream)
        L.vsa_pool_unpermute_bwd(p, self.dqf, self.dqc, dq, stream)
        L.vsa_pool_unpermute_bwd(p.kv_problem(), self.dkf, self.dkc, dk, stream)
        L.vsa_pool_unpermute_bwd(p.v_problem(), self.dvf, self.dvc, dv, stream)
        if gcp is not None and dgate_c is not None:
            L.vsa_pool_unpermute_bwd(po, self.dgcp, None, dgate_c, stream)
        if gfp is not None and dgate_f is not None:
            L.vsa_pool_unpermute_bwd(po, self.dgfp, None, dgate_f, stream)


class VsaAttentionFunction(torch.autograd.Function):
    """One VSA layer as a differentiable PyTorch operation ("VSA: Faster Video
    Diffusion with Trainable Sparse Attention", Abstract: the sparse attention
    is trained end to end).  The forward pass keeps what the backward needs:
    the cube-major intermediates, the index list, and the fine output O_f
    without gates with its log-sum-exp; the output is then formed from O_f by
    vsa_combine (so it differs from VsaForward's fused epilogue by one bf16
    rounding of O_f).  The index list is held fixed in the
    backward (a Top-K selection has no gradient).  Every step runs in the
    library's kernels; this class only sequences the calls and owns the
    buffers.  Raster [batch, heads, N, d] layout, bf16 inputs; the gradients
    come back in the inputs' dtype."""

    @staticmethod
    def forward(ctx, q, k, v, gate_c, gate_f, p: Problem, top_k: int):
        dev = q.device
        f = VsaForward(p, top_k, dev)
        B = L.VSA_BF16
        L.vsa_permute_pool(p, B, q, f.qp, f.qc)
        L.vsa_permute_pool(p.kv_problem(), B, k, f.kp, f.kc)
        L.vsa_permute_pool(p.v_problem(), B, v, f.vp, f.vc)
        L.vsa_coarse_topk(p, top_k, f.qc, f.kc, f.vc, f.lut, f.valid, f.oc)
        # the fine stage without gates, cube-major, for O_f and its LSE
        o_f = torch.empty((p.batch, p.heads, p.n_positions, p.v_dim), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((p.batch, p.heads, p.n_positions), dtype=torch.float32, device=dev)
        L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse=lse)
        # the layer's output from O_f: the gated combination in raster order
        # (without gates, O_f reordered back)
        out = q.new_empty(q.shape[:-1] + (p.v_dim,))
        L.vsa_combine(p, o_f, out, oc=f.oc if gate_c is not None else None, gate_c=gate_c, gate_f=gate_f)
        ctx.p, ctx.top_k, ctx.fwd = p, top_k, f
        ctx.save_for_backward(o_f, lse, gate_c, gate_f)
        return out

    @staticmethod
    def backward(ctx, dout):
        o_f, lse, gate_c, gate_f = ctx.saved_tensors
        p, f = ctx.p, ctx.fwd
        dev = o_f.device
        bw = VsaBackward(p, ctx.top_k, dev)
        f32 = torch.float32
        dq = torch.empty((p.batch, p.heads, p.n_tokens, p.head_dim), dtype=f32, device=dev)
        dk = torch.empty((p.batch, p.kv_heads, p.n_tokens, p.head_dim), dtype=f32, device=dev)
        dv = torch.empty((p.batch, p.kv_heads, p.n_tokens, p.v_dim), dtype=f32, device=dev)
        gshape = (p.batch, p.heads, p.n_tokens, p.v_dim)
        dgc = torch.empty(gshape, dtype=f32, device=dev) if gate_c is not None and ctx.needs_input_grad[3] else None
        dgf = torch.empty(gshape, dtype=f32, device=dev) if gate_f is not None and ctx.needs_input_grad[4] else None
        dout_bf = dout if dout.dtype == torch.bfloat16 and dout.is_contiguous() else \
            dout.to(torch.bfloat16).contiguous()
        bw(f.intermediates(), o_f, lse, dout_bf, dq, dk, dv, gate_c=gate_c, gate_f=gate_f,
           dgate_c=dgc, dgate_f=dgf)
        # autograd casts each gradient to its input's dtype
        return dq, dk, dv, dgc, dgf, None, None


def vsa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Problem, top_k: int,
                  gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Differentiable VSA layer on raster bf16 inputs [batch, heads, N, d]:
    out = g_f * O_f + g_c * O_c (O_f alone without gates).  Backward gives
    the gradients of q, k, v and the gates with the Top-K index list fixed."""
    if not 1 <= top_k <= p.n_cubes:
        raise ValueError(f"top_k={top_k} outside [1, {p.n_cubes}]")
    return VsaAttentionFunction.apply(q, k, v, gate_c, gate_f, p, top_k)
