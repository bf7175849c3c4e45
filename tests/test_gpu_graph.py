"""The whole forward pass and the whole layer backward captured in a HIP
graph: no entry point allocates, synchronises or clears memory with a memset,
so the sequence of library calls can be captured once and replayed.  Each
graph is replayed several times with eager work and synchronisations of the
program in between, and every replay must give exactly the eager result
(the kernels are deterministic: bit-exact).  The eager result itself is
checked against the oracle by the other GPU tests."""
import numpy as np
import pytest
import torch

from block_sparse_video_major_amd import _lib as L
from block_sparse_video_major_amd import workloads as wl
from block_sparse_video_major_amd.pipeline import VsaBackward, VsaForward
from gpu_helpers import bits, dev, inputs, problem

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


@pytest.mark.parametrize("name,layout,order", [("small", "bhnd", "raster"), ("small", "bnhd", "hilbert"),
                                                ("wan", "bhnd", "raster")])
def test_forward_graph_replays_equal_eager(name, layout, order):
    import dataclasses
    w = wl.WORKLOADS[name]
    _log(f"forward graph {name} {layout} {order}")
    p = dataclasses.replace(problem(w), cube_order=order)
    x = inputs(name)
    tens = [dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f")]
    if layout == "bnhd":
        tens = [t.permute(0, 2, 1, 3).contiguous() for t in tens]
    q, k, v, gc, gf = tens
    f = VsaForward(p, w.top_k, layout=layout)
    out = torch.empty_like(q)
    f(q, k, v, out, gc, gf)          # eager: also grants LDS and uploads the cube table once
    torch.cuda.synchronize()
    want = bits(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        f(q, k, v, out, gc, gf)
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device="cuda")
    for r in range(3):
        out.fill_(float("nan"))
        scratch.normal_()            # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), want), f"replay {r} differs from the eager pass"


def test_layer_backward_graph_replays_equal_eager():
    w = wl.SMALL
    _log("layer backward graph small")
    p = problem(w)
    x = inputs(w.name)
    q, k, v, gc, gf = (dev(x[n]) for n in ("q", "k", "v", "gate_c", "gate_f"))
    rng = np.random.default_rng(131)
    dout = dev(wl.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32)))
    f = VsaForward(p, w.top_k)
    out = torch.empty_like(q)
    f(q, k, v, out, gc, gf)
    saved = f.intermediates()
    o_f = torch.empty_like(f.qp)
    lse = torch.empty((1, w.heads, p.n_positions), device="cuda")
    L.vsa_sparse_attn_fwd(p, f.qp, f.kp, f.vp, f.lut, f.valid, o_f, lse=lse)
    bw = VsaBackward(p, w.top_k)
    grads = [torch.empty(q.shape, device="cuda") for _ in range(5)]

    def run():
        bw(saved, o_f, lse, dout, *grads[:3], gate_c=gc, gate_f=gf, dgate_c=grads[3], dgate_f=grads[4])
    run()
    torch.cuda.synchronize()
    want = [bits(t).copy() for t in grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        for t in grads:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(grads):
            assert np.array_equal(bits(t), want[i]), f"replay {r}, gradient {i} differs from the eager pass"
