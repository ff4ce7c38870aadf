"""Concurrent launches on several HIP streams.

The library keeps no state between calls and writes only the caller's
buffers, so independent tensors launched on two streams at once (the way
bench.py overlaps one tensor's kernel with the next) must give exactly the
outputs of the same calls made one after another on one stream.  Checked for
the step's two kernels (forward with the hard mask fused, backward) and the
linear-space pair, 2:4 and 4:8, with every launch of one phase alternating
between two streams.
"""
import math

import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

SHAPES = [(96, 256), (37, 72), (256, 128), (64, 1024)]


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


def _tensors(mg, n, m):
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(100 + m)
    K = math.comb(m, n)
    ts = []
    for i, (rows, cols) in enumerate(SHAPES):
        t = mg.Tensor(n, m, rows, cols, 11 * i, i)
        B = t.nblocks
        ts.append(dict(
            t=t,
            w=(torch.randn(rows, cols, generator=g, device=dev) * 0.02).to(torch.bfloat16),
            z=torch.randn(B, K, generator=g, device=dev),
            G=(torch.randn(rows, cols, generator=g, device=dev) * 1e-3).to(torch.bfloat16),
            pi=torch.randn(B, m, generator=g, device=dev)))
    return ts


def _outputs(mg, ts, n, m, streams):
    """Runs the forward phase, then the backward phase, then the linear-space
    pair; launch i of a phase goes to streams[i % len(streams)]."""
    import torch
    main = torch.cuda.current_stream()
    p = mg.sample_params(5, 3, 100.0, 2.0)
    dp = mg.draw_params(7, 2)
    res = []
    for d in ts:
        t = d["t"]
        B = t.nblocks
        dev = d["w"].device
        res.append(dict(
            out=torch.empty_like(d["w"]), y=torch.empty_like(d["z"]), dz=torch.empty_like(d["z"]),
            bits=torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev),
            idx=torch.empty(B, dtype=torch.uint8, device=dev),
            mp_out=torch.empty_like(d["w"]), dpi=torch.empty_like(d["pi"]),
            order=torch.empty(B, dtype=torch.uint8 if m == 4 else torch.int16, device=dev)))

    def phase(fn):
        ev = torch.cuda.Event()
        ev.record(main)
        for s in streams:
            s.wait_event(ev)
        for i, (d, r) in enumerate(zip(ts, res)):
            fn(d, r, streams[i % len(streams)])
        for s in streams:
            e = torch.cuda.Event()
            e.record(s)
            main.wait_event(e)

    phase(lambda d, r, s: mg.maskgs_fwd_hard(d["t"], p, d["w"], d["z"], r["out"], r["y"], None,
                                             r["idx"], r["bits"], stream=s))
    phase(lambda d, r, s: mg.maskgs_bwd(d["t"], p, d["w"], d["z"], r["y"], d["G"], 1e-5, r["dz"],
                                        stream=s))
    phase(lambda d, r, s: mg.maskpro_fwd(d["t"], dp, d["pi"], d["w"], r["mp_out"],
                                         order=r["order"], stream=s))
    phase(lambda d, r, s: mg.maskpro_bwd(d["t"], dp, d["pi"], 0.25, r["dpi"], order=r["order"],
                                         stream=s))
    torch.cuda.synchronize()
    return [{k: to_np(v) for k, v in r.items()} for r in res]


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_two_streams_match_in_order(mg, nm):
    import torch
    n, m = nm
    ts = _tensors(mg, n, m)
    dev = torch.device("cuda:0")
    one = _outputs(mg, ts, n, m, [torch.cuda.Stream(device=dev)])
    two = _outputs(mg, ts, n, m, [torch.cuda.Stream(device=dev) for _ in range(2)])
    for i, (a, b) in enumerate(zip(one, two)):
        for k in a:
            assert np.array_equal(a[k], b[k]), (nm, SHAPES[i], k)
