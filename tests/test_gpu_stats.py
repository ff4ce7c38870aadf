"""GPU parity of maskgs_mask_stats, the training diagnostics of the pages
(MaskLLM summary, section 3.4 kappa discussion / Figure 5: mask change between
steps and maximum probability; Figure 6: kept-weight norm against magnitude
pruning; Figure 8: mask difference; Table 14: logit gradient norm), through
the C ABI, against the oracle's sums.

Bars: block and change counts exact (the hard masks, sampled ones included,
are integer decisions on bit-exact fp32 values); the maximum-probability sum
within 1e-5 relative (the kernel's exponentials are fp32); the |w| and dz^2
sums within 1e-12 relative (fp64 sums of exact values in a different order).
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import to_np, widen

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


def _compare(got, ref, what):
    assert got["blocks"] == ref["blocks"], what
    assert got["changed"] == ref["changed"], (what, got["changed"], ref["changed"])
    assert abs(got["max_prob"] - ref["max_prob"]) <= 1e-5 * ref["max_prob"], (what, got, ref)
    for k in ("kept_l1", "magnitude_l1", "grad_sq"):
        assert abs(got[k] - ref[k]) <= 1e-12 * abs(ref[k]) + 1e-300, (what, k, got[k], ref[k])


CASES = [
    # n, m, rows, cols, w dtype, block_offset, tensor_id, kappa, sampled (tau)
    (2, 4, 64, 256, "bf16", 0, 0, 100.0, None),
    (2, 4, 37, 72, "f32", 5, 3, 1.0, 4.0),          # odd offset, ragged, sampled
    (2, 4, 41, 20, "bf16", 1, 1, 1e5, 0.05),         # near one-hot, sampled
    (4, 8, 37, 72, "bf16", 3, 4, 100.0, None),       # 333 blocks: ragged tile
    (4, 8, 130, 64, "f32", 2, 2, 10.0, 2.0),         # sampled
    (2, 4, 37, 72, "f32", 2**56 - 333, 5, 1.0, 4.0),  # sampled, Philox counters' high word
    (4, 8, 37, 72, "bf16", 2**56 - 333, 6, 10.0, 2.0),
]


@pytest.mark.parametrize("case", CASES)
def test_mask_stats_small(mg, orc, case):
    import torch
    n, m, rows, cols, wdt, off, tid, kappa, tau = case
    dt = torch.float32 if wdt == "f32" else torch.bfloat16
    K = 6 if m == 4 else 70
    B = rows * cols // m
    w = _rand((rows, cols), 0.02, dt, 80 + tid)
    z = _rand((B, K), 1.0, torch.float32, 81 + tid)
    z_prev = _rand((B, K), 1.0, torch.float32, 82 + tid)
    dz = _rand((B, K), 1e-3, torch.float32, 83 + tid)
    t = mg.Tensor(n, m, rows, cols, off, tid)
    ref_bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=w.device)
    mg.maskgs_hard_extract(t, z_prev, None, None, ref_bits)
    sample = None if tau is None else mg.sample_params(9, 4, kappa, tau)
    st = mg.new_stats(w.device)
    mg.maskgs_mask_stats(t, z, kappa, st, sample=sample, ref_bits=ref_bits, w=w, dz=dz)
    got = mg.read_stats(st)
    sm = None if tau is None else dict(tau=tau, seed=9, step=4, tensor_id=tid, block_offset=off)
    ref = orc.mask_stats(n, m, to_np(z), rows, cols, kappa=kappa, ref_bits=to_np(ref_bits),
                         w=widen(to_np(w)), dz=to_np(dz), sample=sm)
    _compare(got, ref, str(case))
    # accumulation: a second call adds the same sums again
    mg.maskgs_mask_stats(t, z, kappa, st, sample=sample, ref_bits=ref_bits, w=w, dz=dz)
    twice = mg.read_stats(st)
    assert twice["blocks"] == 2 * B and twice["changed"] == 2 * ref["changed"]
    # only max_prob is computed when the optional inputs are absent
    st2 = mg.new_stats(w.device)
    mg.maskgs_mask_stats(t, z, kappa, st2)
    only = mg.read_stats(st2)
    assert only["changed"] == 0 and only["kept_l1"] == 0.0 and only["grad_sq"] == 0.0
    assert abs(only["max_prob"] - ref["max_prob"]) <= 1e-5 * ref["max_prob"]


def test_mask_stats_mlp_tensor(mg, orc):
    """LLaMA-2-7B up_proj 11008x4096 bf16 at full size: the sampled masks of two
    consecutive steps (Figure 5's mask change) and the rest of the sums."""
    import torch
    from workloads import WORKLOADS, tensor_inputs
    wl = WORKLOADS["llama7b_all_linear"]
    spec = [s for s in wl.tensors if s.rows == 11008][0]
    dev = torch.device("cuda:0")
    w, z, G = tensor_inputs(wl, spec, dev)
    B = spec.rows * spec.cols // 4
    t = mg.Tensor(2, 4, spec.rows, spec.cols, 0, spec.tensor_id)
    # step-0 sampled masks as reference bits (from the oracle: the decision is exact)
    zn = to_np(z)
    a0 = orc.sample_logits(2, 4, zn, spec.rows, spec.cols, kappa=wl.kappa, tau=wl.tau, seed=0,
                           step=0, tensor_id=spec.tensor_id)
    cands = orc.candidates(2, 4)
    masks = cands[np.argmax(a0, axis=1)]
    bits = np.packbits(((masks[:, None] >> np.arange(4)) & 1).astype(np.uint8).reshape(-1),
                       bitorder="little")
    del a0
    ref_bits = torch.from_numpy(bits).to(dev)
    st = mg.new_stats(dev)
    mg.maskgs_mask_stats(t, z, wl.kappa, st, sample=mg.sample_params(0, 1, wl.kappa, wl.tau),
                         ref_bits=ref_bits, w=w)
    got = mg.read_stats(st)
    ref = orc.mask_stats(2, 4, zn, spec.rows, spec.cols, kappa=wl.kappa, ref_bits=bits,
                         w=widen(to_np(w)),
                         sample=dict(tau=wl.tau, seed=0, step=1, tensor_id=spec.tensor_id))
    _compare(got, ref, "up_proj")
    assert 0 < got["changed"] < B
