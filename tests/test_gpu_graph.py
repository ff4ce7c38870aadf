"""The step captured in a HIP graph and replayed.

The library only enqueues kernels on the caller's stream: it allocates
nothing, clears nothing with memset and never synchronises, so one step (the
forward with the hard mask fused in, over several tensors, then the backward
of each from the saved soft index) can be captured once and replayed.  Kernel
arguments, the sample parameters (seed, step, kappa, tau) among them, are
fixed at capture; the arrays are read at replay, so logits rewritten in place
between replays are used.  Every replay is checked against the same calls made
eagerly (bit for bit; the fp64 regulariser, summed with atomics in no fixed
order, to 1e-12 relative), with eager work and synchronisations between the
replays and the outputs overwritten before each one.
"""
import math

import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

SHAPES = [(96, 256), (37, 72), (64, 1024)]
REPLAYS = 3


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


def _buffers(mg, n, m, seed):
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    K = math.comb(m, n)
    ts = []
    for i, (rows, cols) in enumerate(SHAPES):
        t = mg.Tensor(n, m, rows, cols, 13 * i + 1, i)
        B = t.nblocks
        d = dict(t=t,
                 w=(torch.randn(rows, cols, generator=g, device=dev) * 0.02).to(torch.bfloat16),
                 z=torch.randn(B, K, generator=g, device=dev),
                 G=(torch.randn(rows, cols, generator=g, device=dev) * 1e-3).to(torch.bfloat16),
                 out=torch.empty(rows, cols, dtype=torch.bfloat16, device=dev),
                 y=torch.empty(B, K, device=dev), dz=torch.empty(B, K, device=dev),
                 idx=torch.empty(B, dtype=torch.uint8, device=dev),
                 bits=torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev))
        if m == 4:
            d["vals"] = torch.empty(2 * B, dtype=torch.bfloat16, device=dev)
            d["vidx"] = torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
        ts.append(d)
    reg = torch.zeros(1, dtype=torch.float64, device=dev)
    return ts, reg


OUTS = ("out", "y", "dz", "idx", "bits", "vals", "vidx")


def _step(mg, ts, reg, p):
    reg.zero_()
    for d in ts:
        mg.maskgs_fwd_hard(d["t"], p, d["w"], d["z"], d["out"], d["y"], reg, d["idx"],
                           d["bits"], d.get("vals"), d.get("vidx"))
    for d in ts:
        mg.maskgs_bwd(d["t"], p, d["w"], None, d["y"], d["G"], 1e-5, d["dz"])


def _scramble(ts, reg):
    """Overwrites every output, so that a replay has to write all of them."""
    import torch
    for d in ts:
        for k in OUTS:
            if k in d:
                x = d[k]
                if x.dtype == torch.uint8:
                    x.fill_(0xA5)
                else:
                    x.fill_(float("nan"))
    reg.fill_(-1.0)


def _snapshot(ts, reg):
    import torch
    torch.cuda.synchronize()
    return [{k: to_np(d[k]).copy() for k in OUTS if k in d} for d in ts], float(reg.item())


def _same(a, b, what):
    (ta, ra), (tb, rb) = a, b
    for i, (x, y) in enumerate(zip(ta, tb)):
        for k in x:
            assert np.array_equal(x[k].view(np.uint8), y[k].view(np.uint8)), (what, SHAPES[i], k)
    assert abs(ra - rb) <= 1e-12 * abs(rb), (what, ra, rb)


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_step_graph_replays_match_eager(mg, nm):
    import torch
    n, m = nm
    ts, reg = _buffers(mg, n, m, seed=500 + m)
    p = mg.sample_params(17, 6, 100.0, 4.0 if m == 4 else 2.0)

    _step(mg, ts, reg, p)
    eager = _snapshot(ts, reg)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(mg, ts, reg, p)          # warm-up on the capture stream's device
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(mg, ts, reg, p)

    busy = torch.randn(512, 512, device="cuda:0")
    for r in range(REPLAYS):
        _scramble(ts, reg)
        graph.replay()
        _same(_snapshot(ts, reg), eager, f"replay {r}")
        busy = torch.tanh(busy @ busy.T * 1e-3)    # the program's own eager work
        torch.cuda.synchronize()

    # new logits written in place are read at replay
    g = torch.Generator(device="cuda:0")
    g.manual_seed(900 + m)
    for d in ts:
        d["z"].copy_(torch.randn(d["z"].shape, generator=g, device="cuda:0"))
    _step(mg, ts, reg, p)
    eager2 = _snapshot(ts, reg)
    assert not np.array_equal(eager2[0][0]["y"], eager[0][0]["y"])
    for r in range(REPLAYS):
        _scramble(ts, reg)
        graph.replay()
        _same(_snapshot(ts, reg), eager2, f"replay {r} after new logits")
    del graph
