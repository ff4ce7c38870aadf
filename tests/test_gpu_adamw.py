"""GPU parity of maskgs_bwd_adamw: the backward to the logits fused with
their AdamW update (MaskLLM summary, section 3.4, Algorithm 1 "update logits";
training details: AdamW, lr 5e-4, weight decay 0.1), through the C ABI.

Two checks per case:
  - end to end against the oracle (oracle backward, rounded to fp32 as
    maskgs_bwd stores it, then the oracle AdamW), z within 1e-6 + 1e-5|ref|;
  - the update arithmetic alone: the GPU's own maskgs_bwd gradient (the fp32
    values the fused kernel computes internally) through the oracle AdamW,
    z within one fp32 ulp plus a few fp32 roundings of the step lr (upd + wd z),
    the moments within a few fp32 ulps of the sum of their terms.
Small shapes span several tiles with a ragged last one and odd block offsets;
one full-size MLP tensor is checked on sampled rows.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import assert_close, to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

HP = dict(lr=5e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
# the C ABI carries the hyperparameters as fp32: the oracle gets the same values
HP32 = {k: float(np.float32(v)) for k, v in HP.items()}
U32 = 2.0 ** -24


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


def _moments(B, K, t, seed):
    import torch
    if t == 1:
        z = torch.zeros((B, K), dtype=torch.float32, device="cuda:0")
        return z, z.clone()
    m = _rand((B, K), 1e-5, torch.float32, seed)
    v = _rand((B, K), 1e-5, torch.float32, seed + 1) ** 2
    return m, v


def _check_update(got, z0, g, m0, v0, t, what):
    """GPU fused (z, m, v) against the oracle AdamW applied to the GPU's own
    maskgs_bwd gradient g."""
    import oracle as orc
    zr, mr, vr = orc.adamw(z0, g, m0, v0, t=t, **HP32)
    zg, mgot, vg = (np.asarray(a, dtype=np.float64) for a in got)
    b1, b2 = HP32["beta1"], HP32["beta2"]
    g64, m64, v64 = (a.astype(np.float64) for a in (g, m0, v0))
    # z: one ulp of the result plus a few fp32 roundings of the step lr*(upd + wd*z)
    mh = (b1 * m64 + (1 - b1) * g64) / (1 - b1 ** t)
    vh = (b2 * v64 + (1 - b2) * g64 * g64) / (1 - b2 ** t)
    upd = np.abs(mh) / (np.sqrt(vh) + HP32["eps"])
    step = HP32["lr"] * (upd + HP32["weight_decay"] * np.abs(z0.astype(np.float64)))
    tol_z = np.spacing(np.abs(zr).astype(np.float32)).astype(np.float64) + 8 * U32 * step + 1e-12
    tol_m = 4 * U32 * (np.abs(mr) + b1 * np.abs(m64) + (1 - b1) * np.abs(g64)) + 1e-38
    tol_v = 4 * U32 * (np.abs(vr) + b2 * v64 + (1 - b2) * g64 * g64) + 1e-38
    for a, r, tol, nm in [(zg, zr, tol_z, "z"), (mgot, mr, tol_m, "m"), (vg, vr, tol_v, "v")]:
        d = np.abs(a - r.astype(np.float64))
        bad = d > tol
        assert not bad.any(), (what, nm, int(bad.sum()), float(d.max()),
                               np.argwhere(bad)[0].tolist())


CASES = [
    # n, m, rows, cols, w dtype, block_offset, tensor_id, seed, step, kappa, tau, t, saved
    (2, 4, 64, 256, "bf16", 0, 0, 0, 0, 100.0, 4.0, 1, True),
    (2, 4, 37, 72, "bf16", 5, 3, 11, 2, 100.0, 4.0, 5, False),   # 666 blocks, odd offset
    (2, 4, 41, 20, "f32", 1, 1, 2, 7, 500.0, 0.05, 3, True),     # ragged, cold tau
    (2, 4, 300, 1024, "bf16", 7, 2, 3, 1, 100.0, 4.0, 2000, False),
    (4, 8, 37, 72, "bf16", 3, 4, 11, 2, 100.0, 2.0, 1, True),    # 333 blocks: ragged tile
    (4, 8, 16, 128, "f32", 0, 0, 0, 0, 100.0, 2.0, 4, False),
    (4, 8, 130, 64, "bf16", 2, 3, 5, 1, 10.0, 8.0, 9, True),
    (2, 4, 37, 72, "bf16", 2**56 - 333, 7, 2**40, 3, 100.0, 4.0, 2, False),  # high counters
    (4, 8, 37, 72, "bf16", 2**56 - 333, 7, 2**40, 3, 100.0, 2.0, 2, False),
]


@pytest.mark.parametrize("case", CASES)
def test_bwd_adamw_small(mg, orc, case):
    import torch
    n, m, rows, cols, wdt, off, tid, seed, step, kappa, tau, t, saved = case
    dt = torch.float32 if wdt == "f32" else torch.bfloat16
    K = 6 if m == 4 else 70
    B = rows * cols // m
    w = _rand((rows, cols), 0.02, dt, 60 + tid)
    z = _rand((B, K), 1.0, torch.float32, 61 + tid)
    G = _rand((rows, cols), 1.0 if wdt == "f32" else 1e-3, dt, 62 + tid)
    m1, m2 = _moments(B, K, t, 63 + tid)
    ten = mg.Tensor(n, m, rows, cols, off, tid)
    p = mg.sample_params(seed, step, kappa, tau)
    lam = 1e-5
    y = None
    if saved:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=w.device)
        y = torch.empty_like(z)
        mg.maskgs_fwd(ten, p, w, z, out, y)
    dz = torch.empty_like(z)
    mg.maskgs_bwd(ten, p, w, z, y, G, lam, dz)
    z0, m0, v0 = to_np(z).copy(), to_np(m1).copy(), to_np(m2).copy()
    zu, mu, vu = z.clone(), m1.clone(), m2.clone()
    mg.maskgs_bwd_adamw(ten, p, w, zu, y, G, lam, mu, vu, step_t=t, **HP)
    torch.cuda.synchronize()
    what = str(case)
    got = (to_np(zu), to_np(mu), to_np(vu))
    _check_update(got, z0, to_np(dz), m0, v0, t, what)
    # end to end: oracle backward (fp32 as stored) then oracle AdamW
    kw = dict(kappa=kappa, tau=tau, seed=seed, step=step, tensor_id=tid, block_offset=off)
    d = orc.bwd(n, m, widen(to_np(w)), z0, widen(to_np(G)), lam=lam, **kw).astype(np.float32)
    zr, mr, vr = orc.adamw(z0, d, m0, v0, t=t, **HP32)
    assert_close(got[0], zr, f"{what} z")


def test_bwd_adamw_mlp_tensor_sampled_rows(mg, orc):
    """LLaMA-2-7B up_proj 11008x4096 bf16 (the benchmark's largest 2:4 launch):
    fused update from a saved soft index at t = 3, oracle on sampled rows."""
    import torch
    from workloads import WORKLOADS, tensor_inputs
    from gpu_helpers import sample_rows
    wl = WORKLOADS["llama7b_all_linear"]
    spec = [s for s in wl.tensors if s.rows == 11008][0]
    dev = torch.device("cuda:0")
    w, z, G = tensor_inputs(wl, spec, dev)
    B = spec.rows * spec.cols // 4
    m1, m2 = _moments(B, 6, 3, 77)
    ten = mg.Tensor(2, 4, spec.rows, spec.cols, 0, spec.tensor_id)
    p = mg.sample_params(0, 0, wl.kappa, wl.tau)
    out = torch.empty_like(w)
    y = torch.empty_like(z)
    mg.maskgs_fwd(ten, p, w, z, out, y)
    bpr = spec.cols // 4
    rows = sample_rows(spec.rows)
    sel = torch.tensor(rows, device=dev)
    bsel = (sel[:, None] * bpr + torch.arange(bpr, device=dev)[None, :]).reshape(-1)
    z0 = to_np(z.index_select(0, bsel))
    m0, v0 = to_np(m1.index_select(0, bsel)), to_np(m2.index_select(0, bsel))
    wn, Gn = to_np(w.index_select(0, sel)), to_np(G.index_select(0, sel))
    mg.maskgs_bwd_adamw(ten, p, w, z, y, G, wl.lam, m1, m2, step_t=3, **HP)
    torch.cuda.synchronize()
    zg = to_np(z.index_select(0, bsel)).reshape(len(rows), bpr, 6)
    mgot = to_np(m1.index_select(0, bsel)).reshape(len(rows), bpr, 6)
    z0, m0, v0 = (a.reshape(len(rows), bpr, 6) for a in (z0, m0, v0))
    for i, r in enumerate(rows):
        kw = dict(kappa=p.kappa, tau=p.tau, seed=p.seed, step=p.step,
                  tensor_id=spec.tensor_id, block_offset=r * bpr)
        d = orc.bwd(2, 4, widen(wn[i:i + 1]), z0[i], widen(Gn[i:i + 1]), lam=wl.lam,
                    **kw).astype(np.float32)
        zr, mr, _ = orc.adamw(z0[i], d, m0[i], v0[i], t=3, **HP32)
        assert_close(zg[i], zr.reshape(bpr, 6), f"row {r} z")
        # m = b1 m0 + (1 - b1) g cancels: bound it by the gradient's tolerance
        # applied to its terms, 1e-5 relative plus an absolute term; the
        # absolute term is 1e-6 of the row's largest gradient (an fp32
        # gradient that crosses zero keeps an error of that order), far below
        # the 1e-6 absolute the gradient tolerance allows at these magnitudes
        b1 = HP32["beta1"]
        d64 = np.abs(d.astype(np.float64))
        tol = (1e-5 * ((1 - b1) * d64 + b1 * np.abs(m0[i].astype(np.float64))) +
               (1 - b1) * 1e-6 * d64.max() + 1e-12)
        dm = np.abs(mgot[i].astype(np.float64) - mr.reshape(bpr, 6))
        assert (dm <= tol).all(), (r, float(dm.max()))
