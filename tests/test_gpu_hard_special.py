"""GPU parity of the hard decisions on logits with special values.

The hard mask of a block is the candidate of the first largest logit, found
by a strict ">" scan from the first candidate (MaskLLM summary, section 3.2
inference flow; section 3.4, Algorithm 1 step 3).  The oracle's scan decides
every case below, so indices, packed bits, the compacted 2:4 values and the
masked weights of the hard Gumbel-max sample must match it bit for bit:
ties (also between +0 and -0), +inf, -inf, a NaN first logit (nothing compares
greater than it, so candidate 0 stays), NaN elsewhere (never taken), all NaN,
and subnormal logits (the kernels keep fp32 subnormals).
"""
import math

import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

KINDS = 10


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


def special_logits(B, K, seed):
    """[B, K] fp32 logits; block b gets special pattern b % KINDS."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, K)).astype(np.float32)
    for b in range(B):
        j = int(rng.integers(1, K))
        kind = b % KINDS
        if kind == 1:                       # many ties
            z[b] = np.round(z[b] * 2.0) / 2.0
        elif kind == 2:                     # +inf, twice: the first one wins
            z[b, j] = np.inf
            z[b, K - 1] = np.inf
        elif kind == 3:                     # NaN first: candidate 0 stays
            z[b, 0] = np.nan
        elif kind == 4:                     # NaN elsewhere: never taken
            z[b, j] = np.nan
        elif kind == 5:
            z[b] = np.nan
        elif kind == 6:
            z[b] = -np.inf
        elif kind == 7:                     # subnormal logits, some tied
            z[b] = (np.round(z[b] * 4.0) * np.float32(1e-41)).astype(np.float32)
        elif kind == 8:                     # +0 / -0 ties
            z[b] = np.where(rng.random(K) < 0.5, np.float32(0.0), np.float32(-0.0))
        elif kind == 9:                     # -inf everywhere but one NaN
            z[b] = -np.inf
            z[b, j] = np.nan
    assert np.any(z[7::KINDS] != 0) and np.all(np.abs(z[7::KINDS]) < np.float32(1.2e-38))
    return z


CASES = [(2, 4, 37, 72), (4, 8, 37, 72), (4, 8, 16, 128)]


@pytest.mark.parametrize("case", CASES)
def test_hard_extract_special_values(mg, orc, case):
    import torch
    n, m, rows, cols = case
    K = math.comb(m, n)
    B = rows * cols // m
    dev = torch.device("cuda:0")
    zn = special_logits(B, K, seed=B + m)
    z = torch.from_numpy(zn).to(dev)
    w = (torch.arange(rows * cols, device=dev, dtype=torch.float32).reshape(rows, cols)
         * 1e-3 - 0.5).to(torch.bfloat16)
    t = mg.Tensor(n, m, rows, cols, 0, 0)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev)
    kw = {}
    if (n, m) == (2, 4):
        kw = dict(values=torch.empty(2 * B, dtype=torch.bfloat16, device=dev),
                  val_idx=torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev))
    mg.maskgs_hard_extract(t, z, w if kw else None, idx, bits, **kw)
    torch.cuda.synchronize()
    h = orc.hard_extract(n, m, zn, rows, cols, to_np(w) if kw else None)
    for kind in range(KINDS):
        sel = np.arange(kind, B, KINDS)
        assert np.array_equal(to_np(idx)[sel], h["idx"][sel]), (case, kind)
    assert np.array_equal(to_np(idx), h["idx"]), case
    assert np.array_equal(to_np(bits), h["bits"]), case
    assert np.all(h["idx"][3::KINDS] == 0) and np.all(h["idx"][5::KINDS] == 0)
    if kw:
        assert np.array_equal(to_np(kw["values"]), h["values"]), case
        assert np.array_equal(to_np(kw["val_idx"]), h["val_idx"]), case


@pytest.mark.parametrize("case", CASES)
def test_fwd_hard_special_values(mg, orc, case):
    """The hard mask fused into the forward: the same decisions as the
    extraction (the soft outputs of non-finite blocks are NaN and not compared)."""
    import torch
    n, m, rows, cols = case
    K = math.comb(m, n)
    B = rows * cols // m
    dev = torch.device("cuda:0")
    zn = special_logits(B, K, seed=3 * B + m)
    z = torch.from_numpy(zn).to(dev)
    w = torch.full((rows, cols), 0.25, dtype=torch.bfloat16, device=dev)
    t = mg.Tensor(n, m, rows, cols, 5, 1)
    p = mg.sample_params(3, 1, 100.0, 2.0)
    out = torch.empty_like(w)
    y = torch.empty_like(z)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev)
    mg.maskgs_fwd_hard(t, p, w, z, out, y, None, idx, bits)
    torch.cuda.synchronize()
    h = orc.hard_extract(n, m, zn, rows, cols)
    assert np.array_equal(to_np(idx), h["idx"]), case
    assert np.array_equal(to_np(bits), h["bits"]), case


@pytest.mark.parametrize("case", CASES)
def test_hard_sample_special_values(mg, orc, case):
    """The hard Gumbel-max sample on the perturbed logits of special values:
    the masked weights are W at the sampled candidate's positions, bit for bit."""
    import torch
    n, m, rows, cols = case
    K = math.comb(m, n)
    B = rows * cols // m
    dev = torch.device("cuda:0")
    zn = special_logits(B, K, seed=5 * B + m)
    z = torch.from_numpy(zn).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(B)
    w = (torch.randn(rows, cols, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    t = mg.Tensor(n, m, rows, cols, 7, 2)
    p = mg.sample_params(9, 4, 100.0, 2.0, mg.MASKGS_HARD_SAMPLE)
    out = torch.empty_like(w)
    mg.maskgs_fwd(t, p, w, z, out, None)
    torch.cuda.synchronize()
    f = orc.fwd(n, m, widen(to_np(w)), zn, kappa=100.0, tau=2.0, seed=9, step=4, tensor_id=2,
                block_offset=7, flags=orc.HARD_SAMPLE)
    assert np.array_equal(to_np(out), f["out"]), case
