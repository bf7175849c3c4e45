"""Concurrent callers: four host threads run whole forward passes at once,
each on its own stream with its own Top-K (so the fine kernel's dynamic LDS
size differs between them), and each result must equal the same pass run
alone, bit for bit.  The library keeps only per-device launch settings
(granted LDS sizes, the CU count), updated under a lock; ctypes releases
the interpreter lock during each call, so the launches really overlap on
the host."""
import threading

import numpy as np
import pytest
import torch

from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaForward
from gpu_helpers import bits, dev, inputs, problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def test_concurrent_forward_passes_equal_sequential():
    w = wl.SMALL
    print("\n[case] four threads, four streams, Top-K 4/8/16/32", flush=True)
    p = problem(w)
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    ks = (4, 8, 16, 32)
    fwd = {kk: VsaForward(p, kk) for kk in ks}
    want = {}
    for kk in ks:
        out = torch.empty_like(q)
        fwd[kk](q, k, v, out, gc, gf)
        torch.cuda.synchronize()
        want[kk] = bits(out).copy()
    outs = {kk: torch.full_like(q, float("nan")) for kk in ks}
    streams = {kk: torch.cuda.Stream() for kk in ks}
    errors = []
    start = threading.Barrier(len(ks))

    def worker(kk):
        try:
            start.wait()
            for _ in range(5):
                fwd[kk](q, k, v, outs[kk], gc, gf, stream=streams[kk])
            streams[kk].synchronize()
        except Exception as e:   # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(kk,)) for kk in ks]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for kk in ks:
        assert np.array_equal(bits(outs[kk]), want[kk]), f"Top-K {kk}: concurrent result differs"


def test_vsa_forward_reuses_buffers_per_stream():
    """vsa_forward keeps its intermediates per (problem, Top-K, stream,
    thread): repeated calls with other inputs give the same bits as a fresh
    VsaForward, and a second stream gets buffers of its own."""
    import block_sparse_video_major_amd as vsa
    from block_sparse_video_major_amd import pipeline
    w = wl.SMALL
    print("\n[case] vsa_forward cache, small grid, Top-K 8", flush=True)
    p = problem(w)
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    q2 = torch.flip(q, dims=[2]).contiguous()
    vsa.clear_forward_cache()
    want = {}
    for name, qq in (("a", q), ("b", q2)):
        out = torch.empty_like(q)
        VsaForward(p, 8)(qq, k, v, out, gc, gf)
        torch.cuda.synchronize()
        want[name] = bits(out).copy()
    got = []
    for qq in (q, q2, q):
        got.append(vsa.vsa_forward(qq, k, v, p, 8, gc, gf))
    torch.cuda.synchronize()
    assert np.array_equal(bits(got[0]), want["a"])
    assert np.array_equal(bits(got[1]), want["b"])
    assert np.array_equal(bits(got[2]), want["a"])
    assert len(pipeline._forward_cache.entries) == 1
    s2 = torch.cuda.Stream()
    o2 = vsa.vsa_forward(q2, k, v, p, 8, gc, gf, stream=s2)
    s2.synchronize()
    assert np.array_equal(bits(o2), want["b"])
    assert len(pipeline._forward_cache.entries) == 2
    vsa.clear_forward_cache()
