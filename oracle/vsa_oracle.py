"""Plain, slow fp64 CPU oracle of the Video Sparse Attention (VSA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants); the seeded input
generators are the only thing both sides read.

Pages followed (cited by title and section):

* [VSA-ROCm] "VSA: Accelerating Video Diffusion Inference with Sparse
  Attention on AMD GPUs" (AMD ROCm blog).
* [VSA-arXiv] "VSA: Faster Video Diffusion with Trainable Sparse Attention"
  (arXiv 2505.13389), Abstract.

Every function works in float64 on the exact values it is given (bf16 and
float32 inputs widen to float64 without rounding).  There is no blocking,
fusion or reordering beyond what each step states.

Readings taken where the pages leave a step open:

* R1 the "3D space-filling curve" order is cube-major: cubes in raster order
  over the cube grid, tokens in raster order inside a cube.
* R2 a grid that does not divide into whole cubes is padded (R20).
* R3 coarse attention is softmax(scale * Qc Kc^T) over all cubes with
  scale = 1/sqrt(d), and O_c = P_c Vc; Top-K ranks the same scores.
* R4 each token of cube i receives O_c[i] (broadcast).
* R5 gates are elementwise: out = g_f * O_f + g_c * O_c; absent g_f means 1,
  absent g_c means 0.
* R6 Top-K ties go to the lower cube index; LUT rows are stored ascending.
* R7 a query cube with zero valid blocks gets O_f = 0 and LSE = -inf.
* R8 a LUT entry listed twice is attended twice (gather semantics).
* R15 a block relation matrix becomes an index list in ascending order; rows
  with more selected blocks than the list holds keep the first ones and are
  counted as overflows.
* R17 the backward differentiates the layer with its LUT held fixed (Top-K
  selection has no gradient); P is recomputed from the forward's LSE.
* R20 a grid that does not divide into cubes is padded up to whole cubes;
  padded positions hold no token: they are never attended as keys, pooling
  averages the real tokens of a cube only, and only real tokens have
  outputs and gradients.
* R21 optional Hilbert cube order: cubes follow the 3D Hilbert curve of
  Skilling's transform over the smallest power-of-two cube that covers the
  cube grid (axis t first), cells outside the grid skipped; tokens inside a
  cube stay in raster order.  R1's raster cube order stays the default.
* R22 values may be narrower or wider than queries and keys (the separate
  hdim_v of the CK interface in [VSA-ROCm]): O_f, O_c, the gates and the
  output take V's width d_v; the softmax scale stays 1/sqrt(d) of the
  query/key width (the d_k of the SDPA formula, [VSA-ROCm] §The Attention
  Bottleneck in Video Diffusion).
* R19 grouped heads (K and V with fewer heads than Q, the head counts of the
  CK kernel interface in [VSA-ROCm]): query head h uses key/value head
  h // G with G = heads / kv_heads; equivalently every key/value head is
  repeated G times, and its gradient is the sum over its G copies.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, invariants, brute force, library special cases); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


# ---------------------------------------------------------------------------
# Step 0: problem checks (R2) and the reordering, [VSA-ROCm] §Two-Stage
# Architecture, "Pre-stage: 3D Space-Filling Curve (SFC) Token Reordering".
# ---------------------------------------------------------------------------

def check_grid(T: int, H: int, W: int, ct: int, ch: int, cw: int) -> None:
    for name, n, c in (("T", T, ct), ("H", H, ch), ("W", W, cw)):
        if n <= 0 or c <= 0:
            raise ValueError(f"{name}={n}, cube={c}: sizes must be positive")
        if n % c:
            raise ValueError(f"{name}={n} is not a multiple of the cube edge {c}")


def perm_index(T: int, H: int, W: int, ct: int, ch: int, cw: int) -> np.ndarray:
    """pi[p] = raster index of the token placed at cube-major position p.

    Cubes are visited in raster order over the (T/ct, H/ch, W/cw) cube grid;
    inside a cube, tokens are visited in raster order over (ct, ch, cw).  So
    every run of ct*ch*cw consecutive positions is exactly one cube (R1).
    Written as explicit loops so it can be read against the definition.
    """
    check_grid(T, H, W, ct, ch, cw)
    order = []
    for cube_t in range(T // ct):
        for cube_h in range(H // ch):
            for cube_w in range(W // cw):
                for lt in range(ct):
                    for lh in range(ch):
                        for lw in range(cw):
                            t = cube_t * ct + lt
                            h = cube_h * ch + lh
                            w = cube_w * cw + lw
                            order.append((t * H + h) * W + w)
    return np.asarray(order, dtype=np.int64)


def hilbert_index(t: int, h: int, w: int, bits: int) -> int:
    """Distance of cell (t, h, w) along the 3D Hilbert curve that fills the
    cube of side 2**bits (R21), by Skilling's transform ("Programming the
    Hilbert curve", AIP Conference Proceedings 707, 2004).

    Going down the levels from the coarsest, a coordinate whose bit is set
    at the current level reflects the lower bits of the first coordinate,
    otherwise the two exchange their lower bits; this undoes the rotations
    and reflections of the sub-cubes.  The three coordinates are then
    Gray-encoded together, and the distance reads their bits level by
    level, most significant level first, t before h before w."""
    x = [t, h, w]
    level = 1 << (bits - 1)
    while level > 1:
        low = level - 1
        for i in range(3):
            if x[i] & level:
                x[0] ^= low
            else:
                swap = (x[0] ^ x[i]) & low
                x[0] ^= swap
                x[i] ^= swap
        level >>= 1
    x[1] ^= x[0]
    x[2] ^= x[1]
    flip = 0
    level = 1 << (bits - 1)
    while level > 1:
        if x[2] & level:
            flip ^= level - 1
        level >>= 1
    x = [c ^ flip for c in x]
    dist = 0
    for b in range(bits - 1, -1, -1):
        for i in range(3):
            dist = (dist << 1) | ((x[i] >> b) & 1)
    return dist


def cube_sequence(gT: int, gH: int, gW: int, cube_order: str = "raster"):
    """Grid coordinates (ct_i, ch_i, cw_i) of the cubes in cube-major order:
    raster order over the cube grid (R1), or along the Hilbert curve of the
    smallest power-of-two cube that covers it, skipping cells outside the
    grid (R21)."""
    cells = [(a, b, c) for a in range(gT) for b in range(gH) for c in range(gW)]
    if cube_order == "raster":
        return cells
    if cube_order != "hilbert":
        raise ValueError(f"cube_order {cube_order!r} is not 'raster' or 'hilbert'")
    bits = 1
    while (1 << bits) < max(gT, gH, gW):
        bits += 1
    return sorted(cells, key=lambda c: hilbert_index(*c, bits))


def token_layout(T: int, H: int, W: int, ct: int, ch: int, cw: int,
                 cube_order: str = "raster") -> np.ndarray:
    """Cube-major layout of a grid that need not divide into cubes (R20):
    the grid is padded to whole cubes (ceil(T/ct)*ct, ...), cubes are
    visited in cube_sequence's order and tokens in raster order inside each
    cube, and pi[p] is the raster index (in the unpadded T x H x W grid) of
    the token at position p, or -1 where p is padding.  Equals perm_index
    when the grid divides and the cube order is raster."""
    for name, n, c in (("T", T, ct), ("H", H, ch), ("W", W, cw)):
        if n <= 0 or c <= 0:
            raise ValueError(f"{name}={n}, cube={c}: sizes must be positive")
    order = []
    for cube_t, cube_h, cube_w in cube_sequence(-(-T // ct), -(-H // ch), -(-W // cw), cube_order):
        for lt in range(ct):
            for lh in range(ch):
                for lw in range(cw):
                    t = cube_t * ct + lt
                    h = cube_h * ch + lh
                    w = cube_w * cw + lw
                    real = t < T and h < H and w < W
                    order.append((t * H + h) * W + w if real else -1)
    return np.asarray(order, dtype=np.int64)


def gather_padded(x: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """x'[..., p, :] = x[..., pi[p], :] for real positions, 0 for padding."""
    x = np.asarray(x)
    out = np.zeros(x.shape[:-2] + (len(pi), x.shape[-1]), dtype=np.float64)
    real = pi >= 0
    out[..., real, :] = x[..., pi[real], :]
    return out


def scatter_padded(xp: np.ndarray, pi: np.ndarray, n: int) -> np.ndarray:
    """out[..., pi[p], :] = x'[..., p, :] for real positions (n raster tokens)."""
    xp = np.asarray(xp, np.float64)
    out = np.zeros(xp.shape[:-2] + (n, xp.shape[-1]), dtype=np.float64)
    real = pi >= 0
    out[..., pi[real], :] = xp[..., real, :]
    return out


def pool_real(xp: np.ndarray, vol: int, real: np.ndarray) -> np.ndarray:
    """Cube mean over the real tokens of each cube only (R20); pool when
    every position is real."""
    xp = np.asarray(xp, np.float64)
    nc = xp.shape[-2] // vol
    out = np.zeros(xp.shape[:-2] + (nc, xp.shape[-1]), dtype=np.float64)
    for c in range(nc):
        sel = np.nonzero(real[c * vol:(c + 1) * vol])[0] + c * vol
        out[..., c, :] = xp[..., sel, :].sum(axis=-2) / len(sel)
    return out


def permute(x: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """x'[..., p, :] = x[..., pi[p], :] (raster -> cube-major)."""
    return x[..., pi, :]


def unpermute(xp: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """out[..., pi[p], :] = x'[..., p, :] (cube-major -> raster)."""
    out = np.empty_like(xp)
    out[..., pi, :] = xp
    return out


# ---------------------------------------------------------------------------
# Stage 1: coarse selection, [VSA-ROCm] §Two-Stage Architecture
# ("Stage 1: Coarse Selection") and §Generating Sparsity Patterns.
# ---------------------------------------------------------------------------

def pool(xp: np.ndarray, vol: int) -> np.ndarray:
    """Cube mean-pool of a cube-major tensor: xc[..., c, :] is the mean of
    rows c*vol .. c*vol+vol-1.  Accumulates in float64."""
    xp = np.asarray(xp, dtype=np.float64)
    n = xp.shape[-2]
    if n % vol:
        raise ValueError("token count is not a multiple of the cube volume")
    nc = n // vol
    out = np.zeros(xp.shape[:-2] + (nc, xp.shape[-1]), dtype=np.float64)
    for c in range(nc):
        out[..., c, :] = xp[..., c * vol:(c + 1) * vol, :].sum(axis=-2) / vol
    return out


def coarse_scores(qc: np.ndarray, kc: np.ndarray, scale: float) -> np.ndarray:
    """S[..., i, j] = scale * <Qc[i], Kc[j]> (the einsum of the LUT pseudo-code
    with the SDPA scale of §The Attention Bottleneck in Video Diffusion)."""
    return scale * np.matmul(qc, np.swapaxes(kc, -1, -2))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with max subtraction, float64."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def coarse_attention(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float):
    """Coarse cube-to-cube attention over all cubes (R3): returns (S, P_c, O_c)."""
    s = coarse_scores(qc, kc, scale)
    p = softmax_rows(s)
    return s, p, np.matmul(p, vc)


def topk_lut(s: np.ndarray, k: int):
    """Per query cube, the k key cubes with the highest scores (R6): order by
    (score descending, index ascending), keep k, store ascending.
    Returns (kv_block_idx [..., Nc, k] int32, valid_block_num [..., Nc] int32).
    """
    nc = s.shape[-1]
    if not 1 <= k <= nc:
        raise ValueError(f"top_k={k} outside [1, {nc}]")
    flat = s.reshape(-1, nc)
    lut = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        order = np.argsort(-flat[r], kind="stable")   # ties keep ascending index
        lut[r] = np.sort(order[:k])
    lut = lut.reshape(s.shape[:-1] + (k,))
    valid = np.full(s.shape[:-1], k, dtype=np.int32)
    return lut, valid


# ---------------------------------------------------------------------------
# Stage 2: fine block-sparse attention, [VSA-ROCm] §Two-Stage Architecture
# ("Stage 2: Fine Computation"), §Block-Sparse Encoding, §Sparse Traversal;
# [VSA-arXiv] Abstract.  Softmax as in §The Attention Bottleneck in Video
# Diffusion: softmax(Q K^T / sqrt(d)) V.
# ---------------------------------------------------------------------------

def fine_attention(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray,
                   kv_block_idx: np.ndarray, valid_block_num: np.ndarray,
                   scale: float, vol: int, query_cubes=None, key_valid=None):
    """Token-level attention of every query cube over its listed key cubes.

    qp/kp/vp: cube-major [B, heads, N, d] (vp may be d_v wide, R22).  For query cube i the key set is
    the concatenation of token ranges [vol*j, vol*j + vol) for the first
    valid_block_num[i] entries j of row i of the LUT (R8: in LUT order).
    Returns (O_f [B, heads, N, d], LSE [B, heads, N]) with
    LSE = log(sum_q exp(scale * q.k)) in natural-log units (R7 for empty rows).
    ``query_cubes`` (optional iterable of (b, h, i)) limits the work to those
    query cubes, for spot checks at full size; other rows stay 0 / -inf.
    ``key_valid`` (optional bool per cube-major position) drops padded key
    positions (R20).
    """
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    B, nh, N, d = qp.shape
    nc = N // vol
    of = np.zeros((B, nh, N, vp.shape[-1]), dtype=np.float64)   # V's width (R22)
    lse = np.full((B, nh, N), -np.inf, dtype=np.float64)
    todo = ((b, h, i) for b in range(B) for h in range(nh) for i in range(nc)) \
        if query_cubes is None else query_cubes
    for b, h, i in todo:
        cnt = int(valid_block_num[b, h, i])
        if cnt == 0:
            continue
        blocks = kv_block_idx[b, h, i, :cnt]
        rows = np.concatenate([np.arange(j * vol, j * vol + vol) for j in blocks])
        if key_valid is not None:
            rows = rows[key_valid[rows]]
        q = qp[b, h, i * vol:(i + 1) * vol]
        s = scale * (q @ kp[b, h, rows].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        of[b, h, i * vol:(i + 1) * vol] = (e @ vp[b, h, rows]) / den
        lse[b, h, i * vol:(i + 1) * vol] = (m + np.log(den))[:, 0]
    return of, lse


def fine_attention_bwd(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray,
                       kv_block_idx: np.ndarray, valid_block_num: np.ndarray,
                       scale: float, vol: int, of: np.ndarray, lse: np.ndarray,
                       dof: np.ndarray, key_valid=None):
    """Gradients of the fine stage ([VSA-arXiv] Abstract: the method is
    trained end to end; the forward is the block-sparse softmax attention of
    fine_attention).  For query cube i with key rows R (the listed cubes'
    tokens, in LUT order, R8), P = exp(scale * Q_i K_R^T - LSE_i) is the
    attention matrix of the forward; with D = rowsum(dO_i * O_i):
        dV_R += P^T dO_i,   dP = dO_i V_R^T,   dS = P * (dP - D),
        dQ_i  = scale * dS K_R,   dK_R += scale * dS^T Q_i.
    A cube listed twice receives both contributions; ``key_valid`` drops
    padded key positions as in fine_attention.  Returns (dq, dk, dv),
    cube-major like the inputs."""
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    of = np.asarray(of, np.float64)
    dof = np.asarray(dof, np.float64)
    B, nh, N, d = qp.shape
    nc = N // vol
    dq = np.zeros_like(qp)
    dk = np.zeros_like(kp)
    dv = np.zeros_like(vp)
    for b in range(B):
        for h in range(nh):
            for i in range(nc):
                cnt = int(valid_block_num[b, h, i])
                if cnt == 0:
                    continue
                rows = np.concatenate([np.arange(j * vol, j * vol + vol)
                                       for j in kv_block_idx[b, h, i, :cnt]])
                if key_valid is not None:
                    rows = rows[key_valid[rows]]
                qs = slice(i * vol, (i + 1) * vol)
                q, do, o = qp[b, h, qs], dof[b, h, qs], of[b, h, qs]
                p = np.exp(scale * (q @ kp[b, h, rows].T) - lse[b, h, qs][:, None])
                dmat = (do * o).sum(axis=1, keepdims=True)
                dp = do @ vp[b, h, rows].T
                ds = p * (dp - dmat)
                dq[b, h, qs] = scale * (ds @ kp[b, h, rows])
                np.add.at(dk[b, h], rows, scale * (ds.T @ q))
                np.add.at(dv[b, h], rows, p.T @ do)
    return dq, dk, dv


def fine_attention_masked(qp, kp, vp, kv_block_idx, valid_block_num, scale, vol):
    """Brute-force form of the same stage: the full N x N mask in which a
    selected cube pair (i, j) expands to a vol x vol block of allowed entries
    (the conceptual mask of [VSA-ROCm] §Two-Stage Architecture), then dense
    masked softmax.  Only for small grids; LUT rows must not repeat an entry.
    """
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    B, nh, N, d = qp.shape
    out = np.zeros_like(qp)
    for b in range(B):
        for h in range(nh):
            allowed = np.zeros((N, N), dtype=bool)
            for p in range(N):
                i = p // vol
                cnt = int(valid_block_num[b, h, i])
                for j in kv_block_idx[b, h, i, :cnt]:
                    allowed[p, j * vol:(j + 1) * vol] = True
            s = scale * (qp[b, h] @ kp[b, h].T)
            s = np.where(allowed, s, -np.inf)
            has = allowed.any(axis=1)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            o = e @ vp[b, h]
            out[b, h] = np.where(has[:, None], o / np.where(has, den, 1.0)[:, None], 0.0)
    return out


# ---------------------------------------------------------------------------
# Block relation matrix -> index list, [VSA-ROCm] §Comparison with Jenga,
# "Sparse Encoding in CK Tile": a block-mask method keeps the full M x M
# one-hot relation B (B[i][j] = 1: query block i attends key block j), VSA
# keeps per query block the selected key-block indices and their count
# (§Block-Sparse Encoding).  Both describe the same pattern.  Reading R15:
# indices are listed in ascending order; a row with more than max_kv
# selected blocks keeps its first max_kv and is counted as an overflow.
# ---------------------------------------------------------------------------

def mask_to_lut(mask: np.ndarray, max_kv: int):
    """Returns (kv_block_idx, valid_block_num, overflow_rows) for a relation
    matrix [..., M, M]; entries past a row's count are 0."""
    m = np.asarray(mask) != 0
    lead, M = m.shape[:-2], m.shape[-2]
    lut = np.zeros(lead + (M, max_kv), dtype=np.int32)
    valid = np.zeros(lead + (M,), dtype=np.int32)
    overflow = 0
    for idx in np.ndindex(*lead, M):
        cols = [j for j in range(m.shape[-1]) if m[idx][j]]
        n = min(len(cols), max_kv)
        lut[idx][:n] = cols[:n]
        valid[idx] = n
        overflow += int(len(cols) > max_kv)
    return lut, valid, overflow


# ---------------------------------------------------------------------------
# Output combination, [VSA-ROCm] §Two-Stage Architecture (learnable gates
# between coarse and fine outputs) and §Algorithmic Design; readings R4, R5.
# ---------------------------------------------------------------------------

def combine(of: np.ndarray, oc: np.ndarray, vol: int,
            gate_c: Optional[np.ndarray] = None,
            gate_f: Optional[np.ndarray] = None) -> np.ndarray:
    """out'[p] = g_f[p] * O_f[p] + g_c[p] * O_c[p // vol] (cube-major)."""
    of = np.asarray(of, np.float64)
    oc_tok = np.repeat(np.asarray(oc, np.float64), vol, axis=-2)
    out = of if gate_f is None else np.asarray(gate_f, np.float64) * of
    if gate_c is not None:
        out = out + np.asarray(gate_c, np.float64) * oc_tok
    return out


# ---------------------------------------------------------------------------
# Grouped heads (R19).
# ---------------------------------------------------------------------------

def kv_group(q: np.ndarray, k: np.ndarray) -> int:
    """G = heads of q per head of k (axis 1); k's head count must divide q's."""
    hq, hk = q.shape[1], k.shape[1]
    if hk < 1 or hq % hk:
        raise ValueError(f"{hk} key/value heads do not divide {hq} query heads")
    return hq // hk


def expand_kv_heads(x: np.ndarray, group: int) -> np.ndarray:
    """Repeat every head (axis 1) `group` times: head h of the result is head
    h // group of x."""
    return np.repeat(np.asarray(x), group, axis=1)


def reduce_kv_heads(dx: np.ndarray, group: int) -> np.ndarray:
    """Adjoint of expand_kv_heads: sum each run of `group` heads."""
    dx = np.asarray(dx, np.float64)
    B, h = dx.shape[:2]
    return dx.reshape((B, h // group, group) + dx.shape[2:]).sum(axis=2)


# ---------------------------------------------------------------------------
# The whole forward pass, steps in the pages' order.
# ---------------------------------------------------------------------------

def vsa_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                grid, cube, top_k: int,
                gate_c: Optional[np.ndarray] = None,
                gate_f: Optional[np.ndarray] = None,
                kv_block_idx: Optional[np.ndarray] = None,
                valid_block_num: Optional[np.ndarray] = None,
                cube_order: str = "raster") -> Dict[str, np.ndarray]:
    """VSA forward on raster inputs [B, heads, N, d]; returns every
    intermediate.  If a LUT is given it replaces the Top-K selection (used to
    score a kernel on exactly the LUT it was handed).  k and v may have fewer
    heads than q (R19); their intermediates are then returned expanded to
    the query heads.  A grid that does not divide into cubes is padded (R20):
    pi holds -1 at padded cube-major positions.  cube_order picks the order
    of the cubes (R1 raster, or R21 Hilbert); cube indices in a given LUT
    refer to that order."""
    T, H, W = grid
    ct, ch, cw = cube
    vol = ct * ch * cw
    q = np.asarray(q, np.float64)
    group = kv_group(q, np.asarray(k))
    k = expand_kv_heads(np.asarray(k, np.float64), group)
    v = expand_kv_heads(np.asarray(v, np.float64), group)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    pi = token_layout(T, H, W, ct, ch, cw, cube_order)   # = perm_index for a divisible raster layout
    real = pi >= 0
    n = T * H * W
    qp, kp, vp = gather_padded(q, pi), gather_padded(k, pi), gather_padded(v, pi)
    qc, kc, vc = pool_real(qp, vol, real), pool_real(kp, vol, real), pool_real(vp, vol, real)
    s, pc, oc = coarse_attention(qc, kc, vc, scale)
    if kv_block_idx is None:
        kv_block_idx, valid_block_num = topk_lut(s, top_k)
    of, lse = fine_attention(qp, kp, vp, kv_block_idx, valid_block_num, scale, vol,
                             key_valid=None if real.all() else real)
    gcp = None if gate_c is None else gather_padded(gate_c, pi)
    gfp = None if gate_f is None else gather_padded(gate_f, pi)
    outp = combine(of, oc, vol, gcp, gfp)
    out = scatter_padded(outp, pi, n)
    return dict(pi=pi, qp=qp, kp=kp, vp=vp, qc=qc, kc=kc, vc=vc, scores=s,
                p_coarse=pc, oc=oc, kv_block_idx=kv_block_idx,
                valid_block_num=valid_block_num, o_fine=of, lse=lse,
                out_cube=outp, out=out, scale=scale)


# ---------------------------------------------------------------------------
# Backward of the remaining steps, so that a whole layer can be trained end to
# end ([VSA-arXiv] Abstract); the LUT is a constant (R17).
# ---------------------------------------------------------------------------

def combine_bwd(dout: np.ndarray, of: np.ndarray, oc: np.ndarray, vol: int,
                gate_c: Optional[np.ndarray] = None,
                gate_f: Optional[np.ndarray] = None):
    """Gradients of out' = g_f * O_f + g_c * O_c[p // vol] (R4, R5) for the
    upstream gradient dout (cube-major).  Returns (dO_f, dO_c, dg_c, dg_f):
    dO_f = g_f * dout; dO_c[c] sums g_c * dout over the vol tokens of cube c
    (the adjoint of the broadcast); dg_c = dout * O_c[p // vol];
    dg_f = dout * O_f.  An absent gate has no gradient (None); an absent g_c
    gives dO_c = 0."""
    dout = np.asarray(dout, np.float64)
    of = np.asarray(of, np.float64)
    oc = np.asarray(oc, np.float64)
    dof = dout if gate_f is None else np.asarray(gate_f, np.float64) * dout
    dgf = None if gate_f is None else dout * of
    if gate_c is None:
        return dof, np.zeros_like(oc), None, dgf
    gd = np.asarray(gate_c, np.float64) * dout
    n = gd.shape[-2]
    doc = np.zeros_like(oc)
    for c in range(n // vol):
        doc[..., c, :] = gd[..., c * vol:(c + 1) * vol, :].sum(axis=-2)
    dgc = dout * np.repeat(oc, vol, axis=-2)
    return dof, doc, dgc, dgf


def coarse_attention_bwd(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                         scale: float, doc: np.ndarray):
    """Gradients of O_c = softmax(scale * Qc Kc^T) Vc over all cubes (R3)
    given dO_c.  With P the coarse probabilities and Dc = rowsum(dO_c * O_c):
        dVc = P^T dO_c,   dP = dO_c Vc^T,   dS = P * (dP - Dc),
        dQc = scale * dS Kc,   dKc = scale * dS^T Qc.
    Returns (dQc, dKc, dVc)."""
    qc = np.asarray(qc, np.float64)
    kc = np.asarray(kc, np.float64)
    vc = np.asarray(vc, np.float64)
    doc = np.asarray(doc, np.float64)
    _, p, oc = coarse_attention(qc, kc, vc, scale)
    dvc = np.matmul(np.swapaxes(p, -1, -2), doc)
    dp = np.matmul(doc, np.swapaxes(vc, -1, -2))
    dmat = (doc * oc).sum(axis=-1, keepdims=True)
    ds = p * (dp - dmat)
    dqc = scale * np.matmul(ds, kc)
    dkc = scale * np.matmul(np.swapaxes(ds, -1, -2), qc)
    return dqc, dkc, dvc


def pool_bwd(dxc: np.ndarray, vol: int) -> np.ndarray:
    """Gradient of the cube mean (pool): every one of the vol tokens of cube c
    receives dxc[c] / vol."""
    return np.repeat(np.asarray(dxc, np.float64), vol, axis=-2) / vol


def pool_real_bwd(dxc: np.ndarray, vol: int, real: np.ndarray) -> np.ndarray:
    """Gradient of pool_real: each real token of cube c receives dxc[c] / (the
    cube's real-token count); padded positions receive 0.  pool_bwd when every
    position is real."""
    dxc = np.asarray(dxc, np.float64)
    nc = dxc.shape[-2]
    counts = real.reshape(nc, vol).sum(axis=1).astype(np.float64)
    out = np.repeat(dxc / counts[:, None], vol, axis=-2)
    out[..., ~real, :] = 0.0
    return out


def vsa_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, grid, cube,
                 kv_block_idx: np.ndarray, valid_block_num: np.ndarray,
                 dout: np.ndarray, gate_c: Optional[np.ndarray] = None,
                 gate_f: Optional[np.ndarray] = None, cube_order: str = "raster") -> Dict[str, np.ndarray]:
    """Gradients of the whole layer (raster in, raster out) for the upstream
    gradient dout (raster), the LUT held fixed (R17): the forward's steps
    taken backwards -- reorder dout, combine, fine attention (through the
    LSE), coarse attention, pooling, reorder back.  Q, K and V each collect
    their fine-stage gradient plus the pooled coarse-stage gradient; with
    grouped heads (R19) dK and dV sum over each key/value head's query heads.
    Returns dict(dq, dk, dv, dgate_c, dgate_f) in raster order (absent gates
    give None)."""
    group = kv_group(np.asarray(q), np.asarray(k))
    f = vsa_forward(q, k, v, grid, cube, 0, gate_c=gate_c, gate_f=gate_f,
                    kv_block_idx=kv_block_idx, valid_block_num=valid_block_num, cube_order=cube_order)
    pi = f["pi"]
    real = pi >= 0
    kv = None if real.all() else real
    n = grid[0] * grid[1] * grid[2]
    vol = cube[0] * cube[1] * cube[2]
    scale = f["scale"]
    doutp = gather_padded(dout, pi)
    gcp = None if gate_c is None else gather_padded(gate_c, pi)
    gfp = None if gate_f is None else gather_padded(gate_f, pi)
    dof, doc, dgcp, dgfp = combine_bwd(doutp, f["o_fine"], f["oc"], vol, gcp, gfp)
    dqf, dkf, dvf = fine_attention_bwd(f["qp"], f["kp"], f["vp"], kv_block_idx, valid_block_num,
                                       scale, vol, f["o_fine"], f["lse"], dof, key_valid=kv)
    dqc, dkc, dvc = coarse_attention_bwd(f["qc"], f["kc"], f["vc"], scale, doc)
    return dict(dq=scatter_padded(dqf + pool_real_bwd(dqc, vol, real), pi, n),
                dk=reduce_kv_heads(scatter_padded(dkf + pool_real_bwd(dkc, vol, real), pi, n), group),
                dv=reduce_kv_heads(scatter_padded(dvf + pool_real_bwd(dvc, vol, real), pi, n), group),
                dgate_c=None if dgcp is None else scatter_padded(dgcp, pi, n),
                dgate_f=None if dgfp is None else scatter_padded(dgfp, pi, n))
