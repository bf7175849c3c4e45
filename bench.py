"""Benchmark of the VSA forward pass on one MI355X.

One step = one pass of the whole forward path over one batch of synthetic
input resident in HBM: pool Q, K, V into cubes (one pass per tensor over its
raster rows), coarse attention + Top-K, fine block-sparse attention (with
the coarse output combined through the gates' default) that gathers each
64-token cube of Q, K, V straight from the raster rows in its tile loads
(the reorder into cubes) and writes the output back in raster order from its
epilogue (the reorder back).  The same step with explicit cube-major copies
(the reorder fused with the pool, the fine stage reading the copies) writes
the same bits and is reported as `reorder_step`.  The default workload is the
32,768-token Wan2.1-scale layer (16x32x64 grid, 4x4x4 cubes, 12 heads,
d=128, bf16, Top-K 154 of 512 cubes = 70% sparsity).

Prints ONE JSON line.  `value` is effective TFLOP/s of the whole step, counting
only the attention FLOPs of selected (query cube, key cube) pairs
(4 * heads * N * 64 * K * d).  `roofline` reports the fine kernel against the
bf16 MFMA peak, with its launch durations measured by HIP events on the stream
the kernels run on.  `cpu_baseline` times the fp64 CPU oracle on a bounded
sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--top-k K]
                       [--no-cpu-baseline] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA, published
MI355X_HBM_PEAK_GBPS = 8000.0        # HBM3E, published
# the fine kernels' sources (pairs and quads of query cubes) and the headers they include
FINE_SOURCES = [os.path.join(ROOT, "block_sparse_video_major_amd", "csrc", n)
                for n in ("sparse_attn_fwd.hip", "sparse_attn_fwd_quad.hip", "token_map.h", "mfma_util.h",
                          "vsa_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_fwd_wan_traffic.md")


def _fine_source_hash() -> str:
    h = hashlib.sha256()
    for path in FINE_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _measured_traffic():
    """HBM bytes per fine-kernel launch from the committed rocprofv3 PMC
    summary, only if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_b or not m_h or m_h.group(1) != _fine_source_hash():
        return None
    return float(m_b.group(1))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_heads(w, seconds_budget: float, max_heads: int):
    """Whole oracle forward passes, head by head, while the budget allows.
    Returns (heads done, seconds, FLOPs counted as in `value`)."""
    import oracle
    from block_sparse_video_major_amd import workloads as wl
    heads_done, t_total, flops = 0, 0.0, 0
    for h in range(min(w.heads, max_heads)):
        x = wl.make_inputs(w, heads=[h], workers=1)
        x64 = {n: wl.as_float64(a) for n, a in x.items()}
        t0 = time.perf_counter()
        oracle.vsa_forward(x64["q"], x64["k"], x64["v"], (w.T, w.H, w.W), w.cube, w.top_k)
        t_total += time.perf_counter() - t0
        heads_done += 1
        flops += 4 * w.n_tokens * w.cube_volume * w.top_k * w.head_dim
        if t_total * (heads_done + 1) / heads_done > seconds_budget:
            break
    return heads_done, t_total, flops


def cpu_baseline(seconds_budget: float = 20.0):
    """Time the fp64 oracle on a bounded sample of the Wan workload: the whole
    forward (reorder, pool, coarse, Top-K, fine, combine, reorder back) for
    whole heads, once with every BLAS thread the host offers and once with a
    single thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from block_sparse_video_major_amd import workloads as wl
    w = wl.WAN
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    heads_done, t_total, flops = _oracle_heads(w, seconds_budget, w.heads)
    with threadpool_limits(limits=1):
        h1, t1, f1 = _oracle_heads(w, seconds_budget, 1)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        affinity = os.cpu_count() or 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads_done} of {w.heads} heads of the 32,768-token workload, full forward in fp64 "
                      f"({t_total:.1f} s with {threads} BLAS threads; same FLOP accounting as value)",
            "one_thread": {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                           "sample": f"{h1} head, full forward in fp64 ({t1:.1f} s)"},
            "nproc": os.cpu_count(), "cpus_allowed": affinity, "cpu_model": _cpu_model()}


def _stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4), "n": int(a.size)}


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--top-k", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--cube-order", choices=("raster", "hilbert"), default="raster",
                    help="order of the cubes in the timed step (the extras also time the Hilbert order)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the warm-up and timed steps (for counter runs on the step's kernels)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no communication).", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import block_sparse_video_major_amd as vsa
    from block_sparse_video_major_amd import _lib as L
    from block_sparse_video_major_amd.pipeline import gather_supported
    from block_sparse_video_major_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy()
        return 0
    L.load()

    w = wl.WAN if args.top_k is None else wl.WAN.with_top_k(args.top_k)
    p = vsa.Problem(w.batch, w.heads, w.T, w.H, w.W, *w.cube, w.head_dim, cube_order=args.cube_order)
    x = wl.make_inputs(w, with_gates=True)   # gates are drawn after V: Q, K, V do not depend on them
    dev = torch.device("cuda:0")
    q, k, v, gate_c, gate_f = (torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).to(dev)
                               for n in ("q", "k", "v", "gate_c", "gate_f"))
    del x
    f = vsa.VsaForward(p, w.top_k, dev)   # with cube-major copies: the reordering step and the extras
    gather = gather_supported(p)
    fg = vsa.VsaForward(p, w.top_k, dev, gather=True) if gather else f
    out = torch.empty_like(q)
    out_cube = torch.empty_like(q)   # cube-major output of the separate fine + unpermute breakdown
    stream = torch.cuda.Stream(device=dev)
    B = L.VSA_BF16

    def reorder_step(ev0=None, ev1=None, p=p, f=f, gates=False):
        """Reorder + pool (one fused pass per tensor), coarse + Top-K, fine
        stage on the cube-major copies with the reorder back in its epilogue."""
        L.vsa_permute_pool(p, B, q, f.qp, f.qc, stream)
        L.vsa_permute_pool(p, B, k, f.kp, f.kc, stream)
        L.vsa_permute_pool(p, B, v, f.vp, f.vc, stream)
        L.vsa_coarse_topk(p, w.top_k, f.qc, f.kc, f.vc, f.lut, f.valid, f.oc, stream)
        if ev0 is not None:
            ev0.record(stream)
        L.vsa_sparse_attn_fwd_raster(p, f.qp, f.kp, f.vp, f.lut, f.valid, out, oc=f.oc,
                                     gate_c=gate_c if gates else None, gate_f=gate_f if gates else None,
                                     stream=stream)
        if ev1 is not None:
            ev1.record(stream)

    def gather_step(ev0=None, ev1=None, p=p, f=fg, gates=False):
        """Pool from the raster rows, coarse + Top-K, fine stage gathering its
        cube tiles from the raster rows (the reorder in its loads, the reorder
        back in its epilogue): the same output bits as reorder_step."""
        L.vsa_permute_pool(p, B, q, None, f.qc, stream)
        L.vsa_permute_pool(p, B, k, None, f.kc, stream)
        L.vsa_permute_pool(p, B, v, None, f.vc, stream)
        L.vsa_coarse_topk(p, w.top_k, f.qc, f.kc, f.vc, f.lut, f.valid, f.oc, stream)
        if ev0 is not None:
            ev0.record(stream)
        L.vsa_sparse_attn_fwd_gather(p, q, k, v, f.lut, f.valid, out, oc=f.oc,
                                     gate_c=gate_c if gates else None, gate_f=gate_f if gates else None,
                                     stream=stream)
        if ev1 is not None:
            ev1.record(stream)

    step = gather_step if gather else reorder_step

    def new_events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def timed_steps(n, gates=False, flush=None, fn=None):
        """n steps (of `fn`, by default the timed step), each bracketed by its
        own events (and its fine kernel by another pair); with `flush`, a
        device write of that buffer (larger than the 256 MB Infinity Cache)
        runs before every step, outside the events.  Returns per-step and
        per-fine-kernel ms."""
        st, fe = new_events(n), new_events(n)
        for i in range(n):
            if flush is not None:
                flush.fill_(i & 0x7F)
            st[i][0].record(stream)
            (fn or step)(*fe[i], gates=gates)
            st[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in st], [a.elapsed_time(b) for a, b in fe]

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev, sev = new_events(args.steps), new_events(args.steps)
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for i in range(args.steps):
            sev[i][0].record(stream)
            step(*ev[i])
            sev[i][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_total = t_start.elapsed_time(t_end)
        fine_ms = [a.elapsed_time(b) for a, b in ev]
        step_ms = [a.elapsed_time(b) for a, b in sev]
        g_step = g_fine = c_step = c_fine = r_step = r_fine = None
        if not args.skip_extras:
            # the same step with the gated combination of the fine and the
            # coarse outputs (seeded gates in raster order), warm cache
            timed_steps(3, gates=True)
            g_step, g_fine = timed_steps(args.steps, gates=True)
            # cold cache: a 1 GiB device write before every step
            flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            timed_steps(2, flush=flush)
            c_step, c_fine = timed_steps(max(10, args.steps // 2), flush=flush)
            del flush
            if gather:
                # the step with explicit cube-major copies of q, k and v (the
                # reorder fused with the pool), for comparison
                timed_steps(3, fn=reorder_step)
                r_step, r_fine = timed_steps(args.steps, fn=reorder_step)

        def extras():
            # per-stage breakdown (separate, untimed pass); the step runs the
            # fused permute_pool, the separate permute and pool are timed too
            names = ["permute_qkv", "pool_qkv", "permute_pool_qkv", "coarse_topk", "sparse_attn_fwd", "unpermute",
                     "sparse_attn_fwd_raster"] + (["pool_from_raster_qkv", "sparse_attn_fwd_gather"] if gather else [])
            reps = max(3, min(10, args.steps))
            acc = {n: 0.0 for n in names}
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                e[0].record(stream)
                for t, dst in ((q, f.qp), (k, f.kp), (v, f.vp)):
                    L.vsa_permute(p, B, t, dst, stream)
                e[1].record(stream)
                for src, dst in ((f.qp, f.qc), (f.kp, f.kc), (f.vp, f.vc)):
                    L.vsa_pool(p, B, src, dst, stream)
                e[2].record(stream)
                for t, dst, dc in ((q, f.qp, f.qc), (k, f.kp, f.kc), (v, f.vp, f.vc)):
                    L.vsa_permute_pool(p, B, t, dst, dc, stream)
                e[3].record(stream)
                L.vsa_coarse_topk(p, w.top_k, f.qc, f.kc, f.vc, f.lut, f.valid, f.oc, stream)
                e[4].record(stream)
                L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, out_cube, oc=f.oc, stream=stream)
                e[5].record(stream)
                L.vsa_unpermute(p, B, out_cube, out, stream)
                e[6].record(stream)
                L.vsa_sparse_attn_fwd_raster(p, f.qp, f.kp, f.vp, f.lut, f.valid, out, oc=f.oc, stream=stream)
                e[7].record(stream)
                if gather:
                    for t, dc in ((q, fg.qc), (k, fg.kc), (v, fg.vc)):
                        L.vsa_permute_pool(p, B, t, None, dc, stream)
                    e[8].record(stream)
                    L.vsa_sparse_attn_fwd_gather(p, q, k, v, f.lut, f.valid, out, oc=f.oc, stream=stream)
                    e[9].record(stream)
                torch.cuda.synchronize()
                for i, n in enumerate(names):
                    acc[n] += e[i].elapsed_time(e[i + 1]) / reps
            # the practical HBM ceiling for these passes: a plain device copy
            # (torch's copy kernel) of the bytes the three reorders read and write
            csrc = torch.empty(3 * q.numel(), dtype=torch.bfloat16, device=dev).fill_(0.5)
            cdst = torch.empty_like(csrc)
            cdst.copy_(csrc)
            acc["copy_qkv"] = 0.0
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                cdst.copy_(csrc)
                e1.record(stream)
                torch.cuda.synchronize()
                acc["copy_qkv"] += e0.elapsed_time(e1) / reps
            del csrc, cdst
            # second workload: a block relation matrix (union of importance,
            # condition and adjacency masks; a different count per row) converted
            # by vsa_mask_to_lut and run through the fine kernel
            mask = wl.block_relation_mask(w, 48, 4)
            maxk = int(mask.astype(np.int64).sum(axis=-1).max())
            mask_d = torch.from_numpy(mask).to(dev)
            lut_m = torch.zeros((w.batch, w.heads, w.n_cubes, maxk), dtype=torch.int32, device=dev)
            valid_m = torch.empty((w.batch, w.heads, w.n_cubes), dtype=torch.int32, device=dev)
            over_m = torch.empty((1,), dtype=torch.int32, device=dev)
            mt = {"mask_to_lut": 0.0, "fine": 0.0}
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record(stream)
                L.vsa_mask_to_lut(p, mask_d, lut_m, valid_m, over_m, stream)
                e[1].record(stream)
                L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, lut_m, valid_m, out_cube, oc=f.oc, stream=stream)
                e[2].record(stream)
                torch.cuda.synchronize()
                mt["mask_to_lut"] += e[0].elapsed_time(e[1]) / reps
                mt["fine"] += e[1].elapsed_time(e[2]) / reps
            pairs_m = int(valid_m.sum().item())

            # sparsity sweep (a diffusion run changes the sparsity from step to
            # step): coarse stage + fine kernel at each Top-K on the same inputs
            sweep = {}
            for kk in wl.SWEEP_TOPK:
                lut_s = torch.empty((w.batch, w.heads, w.n_cubes, kk), dtype=torch.int32, device=dev)
                valid_s = torch.empty((w.batch, w.heads, w.n_cubes), dtype=torch.int32, device=dev)
                L.vsa_coarse_topk(p, kk, f.qc, f.kc, f.vc, lut_s, valid_s, f.oc, stream)
                L.vsa_sparse_attn_fwd_raster(p, f.qp, f.kp, f.vp, lut_s, valid_s, out, oc=f.oc, stream=stream)
                tsum = 0.0
                for _ in range(reps):
                    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    e[0].record(stream)
                    L.vsa_sparse_attn_fwd_raster(p, f.qp, f.kp, f.vp, lut_s, valid_s, out, oc=f.oc, stream=stream)
                    e[1].record(stream)
                    torch.cuda.synchronize()
                    tsum += e[0].elapsed_time(e[1]) / reps
                fl = w.selected_flops(kk)
                sweep[str(kk)] = {"sparsity": round(1 - kk / w.n_cubes, 3), "fine_ms": round(tsum, 4),
                                  "fine_tflops": round(fl / (tsum * 1e-3) / 1e12, 2)}
            flops_m = 4 * 64 * 64 * w.head_dim * pairs_m   # per selected (query cube, key cube) pair

            # backward of the fine stage (training): dQ, dK, dV from the forward's
            # O_f and log-sum-exp on the same LUT, with a seeded output gradient
            o_f = torch.empty_like(q)
            lse_f = torch.empty((w.batch, w.heads, w.n_tokens), dtype=torch.float32, device=dev)
            L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse=lse_f, stream=stream)
            gen = torch.Generator(device=dev).manual_seed(5)
            d_o = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            grads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3)]
            ws = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(p, w.top_k), dtype=torch.uint8, device=dev)

            def bwd():
                L.vsa_sparse_attn_bwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse_f, d_o, *grads, ws, stream)
            bwd()
            torch.cuda.synchronize()
            t_bwd = 0.0
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                bwd()
                e[1].record(stream)
                torch.cuda.synchronize()
                t_bwd += e[0].elapsed_time(e[1]) / reps
            # the whole layer's backward (VsaBackward) with seeded gates: reorder
            # dout and gates, combine backward, fine backward, coarse backward,
            # reorder back with the pooled gradients added
            bw = vsa.VsaBackward(p, w.top_k, dev)
            gate_c = torch.rand(q.shape, generator=gen, device=dev).to(torch.bfloat16)
            gate_f = torch.rand(q.shape, generator=gen, device=dev).to(torch.bfloat16)
            lgrads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(5)]

            def layer_bwd(ev=None):
                def mark(i):
                    if ev is not None:
                        ev[i].record(stream)
                mark(0)
                for src, dst in ((d_o, bw.doutp), (gate_c, bw.gcp), (gate_f, bw.gfp)):
                    L.vsa_permute(p, B, src, dst, stream)
                mark(1)
                L.vsa_combine_bwd(p, bw.doutp, bw.d_of, bw.d_oc, o_f=o_f, oc=f.oc, gate_c=bw.gcp, gate_f=bw.gfp,
                                  d_gate_c=bw.dgcp, d_gate_f=bw.dgfp, stream=stream)
                mark(2)
                L.vsa_sparse_attn_bwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse_f, bw.d_of, bw.dqf, bw.dkf,
                                      bw.dvf, bw.ws_fine, stream)
                mark(3)
                L.vsa_coarse_bwd(p, f.qc, f.kc, f.vc, f.oc, bw.d_oc, bw.dqc, bw.dkc, bw.dvc, bw.ws_coarse, stream)
                mark(4)
                for src, sc, dst in ((bw.dqf, bw.dqc, lgrads[0]), (bw.dkf, bw.dkc, lgrads[1]),
                                     (bw.dvf, bw.dvc, lgrads[2]), (bw.dgcp, None, lgrads[3]),
                                     (bw.dgfp, None, lgrads[4])):
                    L.vsa_pool_unpermute_bwd(p, src, sc, dst, stream)
                mark(5)
            layer_bwd()
            torch.cuda.synchronize()
            lnames = ["reorder_dout_gates", "combine_bwd", "sparse_attn_bwd", "coarse_bwd", "pool_unpermute_bwd"]
            lt = {n: 0.0 for n in lnames}
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
                layer_bwd(e)
                torch.cuda.synchronize()
                for i, n in enumerate(lnames):
                    lt[n] += e[i].elapsed_time(e[i + 1]) / reps

            # the differentiable layer (vsa_attention) with the same gates and
            # output gradient: its training forward (reorders and pools, coarse
            # stage, fine stage without gates keeping O_f and LSE, vsa_combine)
            # and its backward through autograd, buffers allocated per call
            leaves = [t.detach().clone().requires_grad_(True) for t in (q, k, v, gate_c, gate_f)]

            def train_layer(ev=None):
                with torch.cuda.stream(stream):
                    if ev is not None:
                        ev[0].record(stream)
                    o = vsa.vsa_attention(leaves[0], leaves[1], leaves[2], p, w.top_k,
                                          gate_c=leaves[3], gate_f=leaves[4])
                    if ev is not None:
                        ev[1].record(stream)
                    o.backward(d_o)
                    if ev is not None:
                        ev[2].record(stream)
                for t in leaves:
                    t.grad = None
            train_layer()
            torch.cuda.synchronize()
            tr = {"forward": 0.0, "backward": 0.0}
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                train_layer(e)
                torch.cuda.synchronize()
                tr["forward"] += e[0].elapsed_time(e[1]) / reps
                tr["backward"] += e[1].elapsed_time(e[2]) / reps
            del bw, lgrads, gate_c, gate_f, leaves

            # the same step and fine backward with the cubes in Hilbert order
            # (same inputs; the LUT is the Hilbert-order coarse stage's own)
            ph = dataclasses.replace(p, cube_order="hilbert")
            fh = vsa.VsaForward(ph, w.top_k, dev)
            for _ in range(2):
                step(p=ph, f=fh)
            torch.cuda.synchronize()
            hs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            h0.record(stream)
            for i in range(reps):
                step(*hs[i], p=ph, f=fh)
            h1.record(stream)
            torch.cuda.synchronize()
            h_step = h0.elapsed_time(h1) / reps
            h_fine = float(np.mean([a.elapsed_time(b) for a, b in hs]))
            L.vsa_sparse_attn_fwd(ph, fh.qp, fh.kp, fh.vp, fh.lut, fh.valid, o_f, lse=lse_f, stream=stream)

            def hbwd():
                L.vsa_sparse_attn_bwd(ph, fh.qp, fh.kp, fh.vp, fh.lut, fh.valid, o_f, lse_f, d_o, *grads, ws, stream)
            hbwd()
            torch.cuda.synchronize()
            h_bwd = 0.0
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                hbwd()
                e[1].record(stream)
                torch.cuda.synchronize()
                h_bwd += e[0].elapsed_time(e[1]) / reps
            hil = {"step_ms": h_step, "fine_ms": h_fine, "bwd_ms": h_bwd,
                   "pairs": int(fh.valid.sum().item())}
            del grads, ws, d_o, o_f, lse_f, fh

            # a value head size different from the query/key head size (its
            # own four-wavefront kernel): the step's cube-major tensors cut to
            # the widths, the step's Top-K LUT, raster output with O_c
            dvres = {}
            for dq_, dv_ in ((128, 64), (64, 128)):
                pv = dataclasses.replace(p, head_dim=dq_, head_dim_v=dv_)
                qx, kx = f.qp[..., :dq_].contiguous(), f.kp[..., :dq_].contiguous()
                vx, ocx = f.vp[..., :dv_].contiguous(), f.oc[..., :dv_].contiguous()
                ox = torch.empty(q.shape[:-1] + (dv_,), dtype=torch.bfloat16, device=dev)

                def run_dv():
                    L.vsa_sparse_attn_fwd_raster(pv, qx, kx, vx, f.lut, f.valid, ox, oc=ocx, stream=stream)
                run_dv()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    run_dv()
                e1.record(stream)
                torch.cuda.synchronize()
                t_fwd = e0.elapsed_time(e1) / reps
                # its fine backward on the same LUT (cube-major O_f and LSE of that forward)
                of_x = torch.empty(q.shape[:-1] + (dv_,), dtype=torch.bfloat16, device=dev)
                lse_x = torch.empty((w.batch, w.heads, w.n_tokens), dtype=torch.float32, device=dev)
                L.vsa_sparse_attn_fwd(pv, qx, kx, vx, f.lut, f.valid, of_x, lse=lse_x, stream=stream)
                do_x = torch.randn(of_x.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                gx = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in (qx, kx, vx)]
                wsx = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(pv, w.top_k), dtype=torch.uint8, device=dev)

                def run_dv_bwd():
                    L.vsa_sparse_attn_bwd(pv, qx, kx, vx, f.lut, f.valid, of_x, lse_x, do_x, *gx, wsx, stream)
                run_dv_bwd()
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    run_dv_bwd()
                e1.record(stream)
                torch.cuda.synchronize()
                dvres[(dq_, dv_)] = (t_fwd, e0.elapsed_time(e1) / reps)
                del qx, kx, vx, ocx, ox, of_x, lse_x, do_x, gx, wsx

            # the latent grid of an 832 x 480, 81-frame video (21 x 30 x 52 =
            # 32,760 tokens), which does not divide into 4 x 4 x 4 cubes: padded
            # to 24 x 32 x 52 positions (624 cubes), Top-K 187 (70% sparsity)
            pp = dataclasses.replace(p, T=21, H=30, W=52, cube_order="raster")
            kp_ = int(0.3 * pp.n_cubes)
            gpad = torch.Generator(device=dev).manual_seed(7)
            # seeded locality inputs (the Wan layer's recipe, field stride 8) on the padded grid
            wpad = dataclasses.replace(w, name="padded", T=21, H=30, W=52, top_k=kp_, seed=6)
            xpad = wl.make_inputs(wpad, workers=min(16, os.cpu_count() or 1))
            xs = [torch.from_numpy(xpad[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")]
            del xpad
            fpad = vsa.VsaForward(pp, kp_, dev)
            opad = torch.empty_like(xs[0])

            def pstep(ev=None):
                L.vsa_permute_pool(pp, B, xs[0], fpad.qp, fpad.qc, stream)
                L.vsa_permute_pool(pp, B, xs[1], fpad.kp, fpad.kc, stream)
                L.vsa_permute_pool(pp, B, xs[2], fpad.vp, fpad.vc, stream)
                L.vsa_coarse_topk(pp, kp_, fpad.qc, fpad.kc, fpad.vc, fpad.lut, fpad.valid, fpad.oc, stream)
                if ev is not None:
                    ev[0].record(stream)
                L.vsa_sparse_attn_fwd_raster(pp, fpad.qp, fpad.kp, fpad.vp, fpad.lut, fpad.valid, opad, oc=fpad.oc,
                                             stream=stream)
                if ev is not None:
                    ev[1].record(stream)
            pstep()
            torch.cuda.synchronize()
            pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            for i in range(reps):
                pstep(pe[i])
            p1.record(stream)
            torch.cuda.synchronize()
            pad_step = p0.elapsed_time(p1) / reps
            pad_fine = float(np.mean([a.elapsed_time(b) for a, b in pe]))
            of_p = torch.empty_like(fpad.qp)
            lse_p = torch.empty((w.batch, w.heads, pp.n_positions), dtype=torch.float32, device=dev)
            L.vsa_sparse_attn_fwd(pp, fpad.qp, fpad.kp, fpad.vp, fpad.lut, fpad.valid, of_p, lse=lse_p, stream=stream)
            do_p = torch.randn(of_p.shape, generator=gpad, device=dev).to(torch.bfloat16)
            gp = [torch.empty(of_p.shape, dtype=torch.float32, device=dev) for _ in range(3)]
            wsp = torch.empty(L.vsa_sparse_attn_bwd_workspace_size(pp, kp_), dtype=torch.uint8, device=dev)

            def pbwd():
                L.vsa_sparse_attn_bwd(pp, fpad.qp, fpad.kp, fpad.vp, fpad.lut, fpad.valid, of_p, lse_p, do_p, *gp, wsp,
                                      stream)
            pbwd()
            torch.cuda.synchronize()
            p0.record(stream)
            for _ in range(reps):
                pbwd()
            p1.record(stream)
            torch.cuda.synchronize()
            pad_bwd = p0.elapsed_time(p1) / reps
            pad = {"grid": "21x30x52", "tokens": pp.n_tokens, "positions": pp.n_positions, "cubes": pp.n_cubes,
                   "top_k": kp_, "pairs": w.batch * w.heads * pp.n_cubes * kp_, "step_ms": pad_step,
                   "fine_ms": pad_fine, "bwd_ms": pad_bwd}
            del xs, fpad, opad, of_p, lse_p, do_p, gp, wsp

            # the large layer: grid 32 x 48 x 80 (122,880 tokens), 40 heads,
            # Top-K 192 of 1,920 cubes; seeded device inputs, the step timed
            wL = wl.WORKLOADS["large"]
            pl = vsa.Problem(wL.batch, wL.heads, wL.T, wL.H, wL.W, *wL.cube, wL.head_dim)
            # the seeded locality inputs of this workload (Q and K share a smooth
            # field of stride 8, V ~ N(0, 1)), drawn on the host head by head
            xlh = wl.make_inputs(wL, workers=min(16, os.cpu_count() or 1))
            xl = []
            for n in ("q", "k", "v"):
                xl.append(torch.from_numpy(xlh[n].view(np.int16)).view(torch.bfloat16).to(dev))
                del xlh[n]
            del xlh
            fl_ = vsa.VsaForward(pl, wL.top_k, dev)
            ol = torch.empty_like(xl[0])

            def lstep(ev=None):
                def mark(i):
                    if ev is not None:
                        ev[i].record(stream)
                mark(0)
                for t, a, c in ((xl[0], fl_.qp, fl_.qc), (xl[1], fl_.kp, fl_.kc), (xl[2], fl_.vp, fl_.vc)):
                    L.vsa_permute_pool(pl, B, t, a, c, stream)
                mark(1)
                L.vsa_coarse_topk(pl, wL.top_k, fl_.qc, fl_.kc, fl_.vc, fl_.lut, fl_.valid, fl_.oc, stream)
                mark(2)
                L.vsa_sparse_attn_fwd_raster(pl, fl_.qp, fl_.kp, fl_.vp, fl_.lut, fl_.valid, ol, oc=fl_.oc,
                                             stream=stream)
                mark(3)
            lstep()
            torch.cuda.synchronize()
            nl = 5
            le = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nl)]
            p0.record(stream)
            for i in range(nl):
                lstep(le[i])
            p1.record(stream)
            torch.cuda.synchronize()
            lst = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in le]))
                   for j, n in enumerate(("permute_pool_qkv", "coarse_topk", "sparse_attn_fwd_raster"))}
            large = {"step_ms": p0.elapsed_time(p1) / nl, "fine_ms": float(np.mean([e[2].elapsed_time(e[3]) for e in le])),
                     "stages_ms": lst, "flops": wL.selected_flops(), "top_k": wL.top_k, "cubes": wL.n_cubes,
                     "heads": wL.heads, "tokens": wL.n_tokens}
            del xl, fl_, ol
            return acc, mt, pairs_m, over_m, sweep, flops_m, t_bwd, lt, tr, hil, dvres, pad, large
        ex = None if args.skip_extras else extras()
    torch.cuda.synchronize()

    flops = w.selected_flops()
    ms_step = ms_total / args.steps
    fine_avg = float(np.mean(fine_ms))
    elem = w.batch * w.heads * w.n_tokens * w.head_dim
    permute_bytes = 3 * 2 * elem * 2
    pool_bytes = 3 * (elem * 2 + w.batch * w.heads * w.n_cubes * w.head_dim * 4)
    unpermute_bytes = 2 * elem * 2
    permute_pool_bytes = 3 * (2 * elem * 2 + w.batch * w.heads * w.n_cubes * w.head_dim * 4)
    achieved = flops / (fine_avg * 1e-3) / 1e12
    rec = {
        "metric": "VSA fwd ms/call + effective TFLOP/s (% bf16 peak), 32K tokens @70% sparsity",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"wan2.1-scale layer: grid 16x32x64 (32768 tokens), cube 4x4x4, 12 heads, "
                               f"d=128, Top-K {w.top_k} of 512 cubes ({w.sparsity:.1%} sparsity)",
                   "batch": w.batch, "heads": w.heads, "tokens": w.n_tokens, "head_dim": w.head_dim,
                   "top_k": w.top_k, "n_cubes": w.n_cubes, "cube_order": args.cube_order},
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "fine_ms_per_call": round(fine_avg, 4),
        "fine_tflops": round(achieved, 2),
        "fine_pct_bf16_peak": round(100 * achieved / MI355X_BF16_PEAK_TFLOPS, 2),
        "timing": {"note": f"{args.steps} timed steps, each with its own HIP events on the kernels' stream",
                   "step_ms": _stats(step_ms), "fine_ms": _stats(fine_ms)},
    }
    if g_step is not None:
        rec.update({
        "gated_step": {"note": "the same step with gate_c and gate_f (seeded U(0,1), raster order): "
                               "out = g_f * O_f + g_c * O_c broadcast per cube, in the fine kernel's epilogue",
                       "step_ms": _stats(g_step), "fine_ms": _stats(g_fine),
                       "tflops_per_step": round(flops / (float(np.median(g_step)) * 1e-3) / 1e12, 2),
                       "fine_tflops": round(flops / (float(np.median(g_fine)) * 1e-3) / 1e12, 2)},
        "cold_cache": {"note": "a 1 GiB device write (beyond the 256 MB Infinity Cache) before every step, "
                               "outside the timed events",
                       "steps": len(c_step), "step_ms": _stats(c_step), "fine_ms": _stats(c_fine),
                       "tflops_per_step": round(flops / (float(np.median(c_step)) * 1e-3) / 1e12, 2)},
        })
    if r_step is not None:
        rec["reorder_step"] = {
            "note": "the step with explicit cube-major copies: reorder + pool of q, k, v in one pass per tensor, "
                    "coarse + Top-K, the fine stage on the copies (vsa_sparse_attn_fwd_raster); the same output "
                    "bits as the timed step, which pools from the raster rows and gathers the cube tiles in the "
                    "fine kernel's loads (vsa_sparse_attn_fwd_gather)",
            "step_ms": _stats(r_step), "fine_ms": _stats(r_fine),
            "tflops_per_step": round(flops / (float(np.median(r_step)) * 1e-3) / 1e12, 2)}
    rec.update({
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MI355X_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4),
                     "traffic": _measured_traffic()},
    })
    cus, khz, peak_rt = L.vsa_device_peak(torch.cuda.current_device())
    rec["device"] = {"name": torch.cuda.get_device_properties(0).name, "compute_units": cus,
                     "max_sclk_mhz": round(khz / 1e3, 1),
                     "bf16_peak_tflops_runtime": round(peak_rt, 1),
                     "bf16_peak_tflops_spec": MI355X_BF16_PEAK_TFLOPS,
                     "fine_frac_of_runtime_peak": round(achieved / peak_rt, 4) if peak_rt > 0 else None,
                     "note": "runtime peak = compute units x peak shader clock x 4096 bf16 flop per clock "
                             "per CU, from HIP's device attributes; roofline.peak is the published figure"}
    if ex is not None:
        acc, mt, pairs_m, over_m, sweep, flops_m, t_bwd, lt, tr, hil, dvres, pad, large = ex
        pad_fl = 4 * 64 * 64 * w.head_dim * pad["pairs"]   # per selected pair, padded positions included
        rec.update({
            "stages_ms": {n: round(t, 4) for n, t in acc.items()},
            "stages_gbps": {"permute_qkv": round(permute_bytes / (acc["permute_qkv"] * 1e-3) / 1e9, 1),
                            "pool_qkv": round(pool_bytes / (acc["pool_qkv"] * 1e-3) / 1e9, 1),
                            "permute_pool_qkv": round(permute_pool_bytes / (acc["permute_pool_qkv"] * 1e-3) / 1e9,
                                                      1),
                            "unpermute": round(unpermute_bytes / (acc["unpermute"] * 1e-3) / 1e9, 1),
                            **({"pool_from_raster_qkv": round(pool_bytes / (acc["pool_from_raster_qkv"] * 1e-3) / 1e9,
                                                              1)} if gather else {}),
                            "copy_ceiling": round(permute_bytes / (acc["copy_qkv"] * 1e-3) / 1e9, 1),
                            "note": "copy_ceiling: torch's device copy of the bytes the three reorders move, "
                                    "timed in the same run; HBM peak 8000 GB/s"},
            "topk_sweep": sweep,
            "mask_workload": {"pattern": "union of 48 random + 4 fixed + 3x3x3-neighbour key cubes per query cube",
                              "mean_key_cubes_per_query_cube": round(pairs_m / (w.batch * w.heads * w.n_cubes), 1),
                              "overflow_rows": int(over_m.item()),
                              "mask_to_lut_ms": round(mt["mask_to_lut"], 4), "fine_ms": round(mt["fine"], 4),
                              "fine_tflops": round(flops_m / (mt["fine"] * 1e-3) / 1e12, 2)},
            "backward": {"ms_per_call": round(t_bwd, 4),
                         "tflops": round(2.5 * flops / (t_bwd * 1e-3) / 1e12, 2),
                         "pct_bf16_peak": round(100 * 2.5 * flops / (t_bwd * 1e-3) / 1e12 / MI355X_BF16_PEAK_TFLOPS,
                                                2),
                         "flop_accounting": "5 products of 2*64*64*d per selected pair (S, dP, dQ, dK, dV)",
                         "layer_ms": round(sum(lt.values()), 4),
                         "layer_stages_ms": {n: round(t, 4) for n, t in lt.items()},
                         "layer_note": "whole-layer backward with gates (VsaBackward steps), LUT fixed"},
            "training_layer": {"note": "vsa_attention with gates: its forward keeps O_f and LSE for the backward "
                                       "and forms the output with vsa_combine; backward through autograd, "
                                       "gradients cast to bf16; buffers allocated on every call",
                               "forward_ms": round(tr["forward"], 4), "backward_ms": round(tr["backward"], 4),
                               "total_ms": round(tr["forward"] + tr["backward"], 4)},
            "hilbert_order": {"note": "the same step and fine backward with the cubes in 3D Hilbert order",
                              "ms_per_step": round(hil["step_ms"], 4),
                              "tflops_per_step": round(flops / (hil["step_ms"] * 1e-3) / 1e12, 2),
                              "fine_ms_per_call": round(hil["fine_ms"], 4),
                              "fine_tflops": round(flops / (hil["fine_ms"] * 1e-3) / 1e12, 2),
                              "bwd_ms_per_call": round(hil["bwd_ms"], 4),
                              "bwd_tflops": round(2.5 * flops / (hil["bwd_ms"] * 1e-3) / 1e12, 2)},
            "padded_grid": {"note": "latent grid of an 832x480, 81-frame video: 21x30x52 tokens padded to whole "
                                    "4x4x4 cubes; FLOPs per selected cube pair as for the main line",
                            "grid": pad["grid"], "tokens": pad["tokens"], "positions": pad["positions"],
                            "cubes": pad["cubes"], "top_k": pad["top_k"],
                            "ms_per_step": round(pad["step_ms"], 4),
                            "fine_ms_per_call": round(pad["fine_ms"], 4),
                            "fine_tflops": round(pad_fl / (pad["fine_ms"] * 1e-3) / 1e12, 2),
                            "bwd_ms_per_call": round(pad["bwd_ms"], 4),
                            "bwd_tflops": round(2.5 * pad_fl / (pad["bwd_ms"] * 1e-3) / 1e12, 2)},
            "large_workload": {"note": "grid 32x48x80, 40 heads, d=128, seeded locality inputs (field stride 8)",
                               "tokens": large["tokens"], "heads": large["heads"], "cubes": large["cubes"],
                               "top_k": large["top_k"], "ms_per_step": round(large["step_ms"], 3),
                               "fine_ms_per_call": round(large["fine_ms"], 3),
                               "stages_ms_median": {n: round(t, 3) for n, t in large["stages_ms"].items()},
                               "fine_tflops": round(large["flops"] / (large["fine_ms"] * 1e-3) / 1e12, 2),
                               # the coarse stage's products: S = Qc Kc^T and O_c = P Vc, 2 Nc^2 d each per head,
                               # against the 157.3 TFLOP/s fp32 matrix peak
                               "coarse_tflops": round(4.0 * large["cubes"] ** 2 * 128 * large["heads"]
                                                      / (large["stages_ms"]["coarse_topk"] * 1e-3) / 1e12, 2),
                               "coarse_pct_fp32_peak": round(100.0 * 4.0 * large["cubes"] ** 2 * 128 * large["heads"]
                                                             / (large["stages_ms"]["coarse_topk"] * 1e-3) / 157.3e12, 2)},
            "value_head_size": {
                "note": "fine stage with d_v != d (its own forward kernel), the step's Top-K LUT, raster output "
                        "with O_c; FLOPs 2*64*64*(d + d_v) per selected pair; fine backward on the same LUT, "
                        "FLOPs 2*64*64*(3 d + 2 d_v) per pair (S, dP, dQ, dK, dV)",
                **{f"d{a}_dv{b}": {"fine_ms_per_call": round(t[0], 4),
                                   "tflops": round(flops * (a + b) / 256 / (t[0] * 1e-3) / 1e12, 2),
                                   "bwd_ms_per_call": round(t[1], 4),
                                   "bwd_tflops": round(flops * (3 * a + 2 * b) / 256 / (t[1] * 1e-3) / 1e12, 2)}
                   for (a, b), t in dvres.items()}},
        })
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
