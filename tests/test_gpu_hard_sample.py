"""GPU parity of the hard Gumbel-max sample with a straight-through gradient
(flag MASKGS_HARD_SAMPLE; MaskLLM summary, section 3.4, Eq. 5: the first
argmax of the perturbed logits is a draw from softmax(kappa z)).

The applied mask is an integer decision on the bit-exact fp32 perturbed logits
of the noise contract, so the masked weights are compared bit for bit; y, dz,
R and the AdamW update follow the usual bars.  The Gumbel-max property itself
is checked on the GPU: blocks with identical logits draw their hard masks with
frequencies softmax(kappa z) (chi^2).
"""
import math

import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import assert_close, to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


def _rand(shape, std, dtype, seed):
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=dev) * std).to(dtype)


CASES = [
    # n, m, rows, cols, w dtype, out dtype, block_offset, tensor_id, seed, step, kappa, tau
    (2, 4, 64, 256, "bf16", "bf16", 0, 0, 0, 0, 100.0, 4.0),
    (2, 4, 37, 72, "f32", "f32", 5, 3, 11, 2, 1.0, 2.0),      # noise-dominated, odd offset
    (4, 8, 37, 72, "bf16", "bf16", 3, 4, 11, 2, 100.0, 2.0),  # ragged tile
    (4, 8, 16, 128, "f32", "f32", 1, 1, 7, 5, 10.0, 0.5),
    (2, 4, 37, 72, "bf16", "bf16", 2**56 - 333, 2, 2**63 + 1, 9, 10.0, 2.0),  # high counters
    (4, 8, 37, 72, "bf16", "bf16", 2**56 - 333, 2, 2**63 + 1, 9, 10.0, 2.0),
]


@pytest.mark.parametrize("case", CASES)
def test_hard_sample_fwd_bwd(mg, orc, case):
    import torch
    n, m, rows, cols, wdt, odt, off, tid, seed, step, kappa, tau = case
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    K = math.comb(m, n)
    B = rows * cols // m
    w = _rand((rows, cols), 0.02, dt[wdt], 90 + tid)
    z = _rand((B, K), 1.0, torch.float32, 91 + tid)
    G = _rand((rows, cols), 1e-3, dt[wdt], 92 + tid)
    t = mg.Tensor(n, m, rows, cols, off, tid)
    p = mg.sample_params(seed, step, kappa, tau, mg.MASKGS_HARD_SAMPLE)
    out = torch.empty((rows, cols), dtype=dt[odt], device=w.device)
    y = torch.empty_like(z)
    reg = torch.zeros(1, dtype=torch.float64, device=w.device)
    mg.maskgs_fwd(t, p, w, z, out, y, reg)
    dz = torch.empty_like(z)
    mg.maskgs_bwd(t, p, w, z, None, G, 0.5, dz)
    reg2 = torch.zeros_like(reg)
    mg.maskgs_reg_reduce(t, p, w, z, None, reg2)
    torch.cuda.synchronize()
    kw = dict(kappa=kappa, tau=tau, seed=seed, step=step, tensor_id=tid, block_offset=off,
              flags=orc.HARD_SAMPLE)
    wf = widen(to_np(w))
    f = orc.fwd(n, m, wf, to_np(z), out_dtype=odt, **kw)
    what = str(case)
    assert np.array_equal(to_np(out), f["out"]), what          # the kept weights, exactly
    assert_close(to_np(y), f["y"], f"{what} y")
    for r in (reg, reg2):
        assert abs(r.item() - f["reg"]) <= 1e-5 * f["reg"], (what, r.item(), f["reg"])
    d = orc.bwd(n, m, wf, to_np(z), widen(to_np(G)), lam=0.5, **kw)
    assert_close(to_np(dz), d, f"{what} dz straight-through")
    with pytest.raises(mg.MaskgsError):
        mg.maskgs_bwd(t, p, w, z, y, G, 0.5, dz)


def test_hard_sample_adamw(mg, orc):
    import torch
    rows, cols = 40, 64
    B = rows * cols // 4
    w = _rand((rows, cols), 0.02, torch.bfloat16, 95)
    z = _rand((B, 6), 1.0, torch.float32, 96)
    G = _rand((rows, cols), 1e-3, torch.bfloat16, 97)
    t = mg.Tensor(2, 4, rows, cols, 3, 2)
    p = mg.sample_params(4, 1, 100.0, 4.0, mg.MASKGS_HARD_SAMPLE)
    m1 = torch.zeros_like(z)
    m2 = torch.zeros_like(z)
    z0 = to_np(z).copy()
    mg.maskgs_bwd_adamw(t, p, w, z, None, G, 1e-5, m1, m2, lr=5e-4, step_t=1)
    torch.cuda.synchronize()
    kw = dict(kappa=100.0, tau=4.0, seed=4, step=1, tensor_id=2, block_offset=3,
              flags=orc.HARD_SAMPLE)
    d = orc.bwd(2, 4, widen(to_np(w)), z0, widen(to_np(G)), lam=1e-5, **kw).astype(np.float32)
    hp = {k: float(np.float32(v)) for k, v in
          dict(lr=5e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1).items()}
    zr, _, _ = orc.adamw(z0, d, np.zeros_like(z0), np.zeros_like(z0), t=1, **hp)
    assert_close(to_np(z), zr, "hard-sample AdamW z")


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_gumbel_max_frequencies_on_gpu(mg, orc, nm):
    """Section 3.4, Eq. 5: blocks with the same logits and their own noise draw
    hard masks with frequencies softmax(kappa z), at any temperature."""
    import torch
    from scipy import stats
    n, m = nm
    K = math.comb(m, n)
    rng = np.random.default_rng(79)
    zrow = rng.normal(0, 1.0, size=K).astype(np.float32)
    rows, cols = 400, m * 1000
    B = rows * cols // m
    dev = torch.device("cuda:0")
    z = torch.from_numpy(np.tile(zrow, (B, 1))).to(dev)
    w = torch.ones((rows, cols), dtype=torch.float32, device=dev)
    out = torch.empty_like(w)
    t = mg.Tensor(n, m, rows, cols, 0, 0)
    mg.maskgs_fwd(t, mg.sample_params(12, 3, 1.0, 5.0, mg.MASKGS_HARD_SAMPLE), w, z, out)
    kept = (to_np(out).reshape(B, m) != 0)
    codes = (kept * (1 << np.arange(m))).sum(1)
    index = {int(c): i for i, c in enumerate(orc.candidates(n, m))}
    counts = np.bincount([index[int(c)] for c in codes], minlength=K)
    p = np.exp(zrow.astype(np.float64) - zrow.max())
    p /= p.sum()
    chi2 = ((counts - B * p) ** 2 / (B * p)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, K - 1), chi2
