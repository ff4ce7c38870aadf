"""Tensors whose logit arrays hold more than 2^31 floats.

A 4:8 tensor of 16384 x 16384 weights has 33.5M blocks and 2.35G logits (9.4
GB); a 2:4 tensor of 32768 x 45056 weights has 369M blocks and 2.21G logits.
Every index and byte offset past 2^31 must be carried in 64 bits: the
forward with the hard mask fused in and the backward run on the whole tensor
in the benchmark's launch configuration (with the soft index saved, and
recomputed as the benchmark's step does), and the oracle checks the first,
middle and last rows (noise keyed on their global block indices), the hard
mask of those rows, and the backward; likewise the linear-space draw and
policy gradient on [B, M] logits past 2^31 floats.  At most 36 GB of device
memory per test.
"""
import math

import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import assert_bf16_ulp, assert_close, to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

CASES = [(4, 8, 16384, 16384), (2, 4, 32768, 45056)]


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


@pytest.mark.parametrize("case", CASES)
def test_logit_arrays_past_2_31(mg, orc, case):
    import torch
    n, m, rows, cols = case
    K = math.comb(m, n)
    bpr = cols // m
    B = rows * bpr
    assert B * K > 2**31
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(rows + m)
    w = (torch.randn(rows, cols, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    G = (torch.randn(rows, cols, generator=g, device=dev) * 1e-3).to(torch.bfloat16)
    z = torch.randn(B, K, generator=g, device=dev)
    t = mg.Tensor(n, m, rows, cols, 0, 9)
    p = mg.sample_params(21, 3, 100.0, 4.0)
    lam = 1e-5
    out = torch.empty_like(w)
    y = torch.empty_like(z)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev)
    dz = torch.empty_like(z)
    rows_checked = (0, 1, rows // 2, rows - 2, rows - 1)
    ref = {}
    # the soft index saved by the forward and read by the backward, then the
    # benchmark's step: the forward saving nothing and the backward drawing
    # the soft index again from z (outputs overwritten between the two)
    for saved in (True, False):
        mg.maskgs_fwd_hard(t, p, w, z, out, y if saved else None, None, idx, bits)
        mg.maskgs_bwd(t, p, w, None if saved else z, y if saved else None, G, lam, dz)
        torch.cuda.synchronize()
        for r in rows_checked:
            b0, b1 = r * bpr, (r + 1) * bpr
            wn = widen(to_np(w[r:r + 1]))
            zn = to_np(z[b0:b1])
            kw = dict(kappa=p.kappa, tau=p.tau, seed=p.seed, step=p.step, tensor_id=9,
                      block_offset=b0)
            if r not in ref:
                ref[r] = (orc.fwd(n, m, wn, zn, **kw), orc.hard_extract(n, m, zn, 1, cols),
                          orc.bwd(n, m, wn, zn, widen(to_np(G[r:r + 1])), lam=lam, **kw))
            f, h, d = ref[r]
            what = f"{n}:{m} row {r} ({'saved' if saved else 'recomputed'} soft index)"
            if saved:
                assert_close(to_np(y[b0:b1]), f["y"], f"{what} y")
            assert_bf16_ulp(to_np(out[r:r + 1]), f["out"], f"{what} out")
            assert np.array_equal(to_np(idx[b0:b1]), h["idx"]), what
            if m == 8:
                assert np.array_equal(to_np(bits[b0:b1]), h["bits"]), what
            else:
                assert np.array_equal(to_np(bits[b0 // 2:b1 // 2]), h["bits"]), what
            assert_close(to_np(dz[b0:b1]), d, f"{what} dz")
    del w, G, z, out, y, dz, idx, bits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_linear_space_logits_past_2_31(mg, orc, nm):
    """The linear-space draw and policy gradient on a tensor whose [B, M]
    logits hold more than 2^31 floats (2:4: 32768 x 65568 weights, 537M
    blocks; 4:8: 16384 x 131104, 268M blocks), first, middle and last rows
    against the oracle."""
    import torch
    from test_gpu_maskpro import _order_tensor, assert_pg, order_np, pack_order
    n, m = nm
    rows, cols = (32768, 65568) if m == 4 else (16384, 131104)
    bpr = cols // m
    B = rows * bpr
    assert B * m > 2**31
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(cols + m)
    w = (torch.randn(rows, cols, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    pi = torch.randn(B, m, generator=g, device=dev)
    t = mg.Tensor(n, m, rows, cols, 0, 4)
    p = mg.draw_params(77, 5)
    out = torch.empty_like(w)
    order = _order_tensor(B, m, dev)
    mg.maskpro_fwd(t, p, pi, w, out, order=order)
    dpi = torch.empty_like(pi)
    adv = -0.4
    mg.maskpro_bwd(t, p, pi, adv, dpi, order=order)
    torch.cuda.synchronize()
    for r in (0, rows // 2, rows - 1):
        b0, b1 = r * bpr, (r + 1) * bpr
        pin = to_np(pi[b0:b1])
        kw = dict(seed=p.seed, step=p.step, tensor_id=4, block_offset=b0)
        f = orc.maskpro_fwd(n, m, widen(to_np(w[r:r + 1])), pin, **kw)
        assert np.array_equal(order_np(order[b0:b1], m), pack_order(f["order"], m)), r
        assert np.array_equal(to_np(out[r:r + 1]), f["out"]), r
        ref = orc.maskpro_grad(n, m, pin, 1, cols, advantage=adv, order=f["order"])
        assert_pg(to_np(dpi[b0:b1]), ref, adv, n, f"{n}:{m} row {r}")
    del w, pi, out, order, dpi
    torch.cuda.empty_cache()
