"""GPU parity of the calls the benchmark times, at the sizes it times them.

The benchmark's step is, for every linear weight of a 32-layer LLaMA-2-7B-shaped
model, maskgs_fwd_hard (W (.) M~, regulariser, argmax, packed bits, 2:4 values
and 2-bit indices; the soft index saved or not) and then maskgs_bwd (from the
saved soft index, or recomputing it from z).  The shapes 4096x4096,
11008x4096 and 4096x11008 take several grid-stride passes of the launch grid,
so every pass of the fused kernels is covered here; the launch geometry depends
only on the tensor shape and the device, so it is the benchmark's.

Bars (MaskLLM summary page, section 3.4 Algorithm 1 and the inference flow of
section 3.2):
  - argmax indices, packed bits, 2:4 values and 2-bit indices: in full,
    bit-exact against the oracle;
  - the regulariser of the whole tensor: within 1e-5 relative;
  - soft index, masked weight and logit gradient: on every 61st row plus the
    first and last rows (fp32 within 1e-6 + 1e-5|ref|, bf16 within one ulp).
The all-linear sweep then checks every one of the 224 tensors the same way on
sampled rows (integer outputs in full), in groups of four layers, and the
Nemotron-4-15B-shaped 4:8 layer set goes through its step (the same two calls)
with the same bars.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import check_rows, to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return mg


def _step(mg, wl, spec, w, z, G, p, save_y):
    """One tensor of the benchmark's step: the fused forward with every output,
    then the backward (saved or recomputed soft index)."""
    import torch
    dev = w.device
    B = spec.rows * spec.cols // 4
    t = mg.Tensor(2, 4, spec.rows, spec.cols, 0, spec.tensor_id)
    out = torch.empty_like(w)
    y = torch.empty_like(z) if save_y else None
    reg = torch.zeros(1, dtype=torch.float64, device=dev)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B * 4 + 7) // 8, dtype=torch.uint8, device=dev)
    vals = torch.empty(2 * B, dtype=w.dtype, device=dev)
    vidx = torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
    dz = torch.empty_like(z)
    mg.maskgs_fwd_hard(t, p, w, z, out, y, reg, idx, bits, vals, vidx)
    mg.maskgs_bwd(t, p, w, None if save_y else z, y, G, wl.lam, dz)
    torch.cuda.synchronize()
    return dict(out=out, y=y, reg=reg, idx=idx, bits=bits, vals=vals, vidx=vidx, dz=dz)


def _check_hard(orc, spec, z, w, r, what):
    h = orc.hard_extract(2, 4, to_np(z), spec.rows, spec.cols, w_raw=to_np(w))
    for name, key in (("idx", "idx"), ("bits", "bits"), ("vals", "values"),
                      ("vidx", "val_idx")):
        got = to_np(r[name])
        if not np.array_equal(got, h[key]):
            bad = np.flatnonzero(got.reshape(-1) != h[key].reshape(-1))
            raise AssertionError(f"{what} {name}: {bad.size} of {got.size} differ, first at "
                                 f"{bad[0]}")


@pytest.mark.parametrize("save_y", [False, True], ids=["recompute_y", "saved_y"])
@pytest.mark.parametrize("which", ["q_proj", "gate_proj", "down_proj"])
def test_timed_step_full_size(mg, orc, which, save_y):
    """Layer 0's 4096x4096, 11008x4096 and 4096x11008 tensors through the
    benchmark's step, every output of the fused forward against the oracle."""
    import torch
    from workloads import WORKLOADS, llama7b_layer, tensor_inputs
    wl = WORKLOADS["llama7b_all_linear"]
    spec = next(s for s in llama7b_layer(0) if s.name.endswith(which))
    dev = torch.device("cuda:0")
    w, z, G = tensor_inputs(wl, spec, dev)
    p = mg.sample_params(0, 3, wl.kappa, wl.tau)
    r = _step(mg, wl, spec, w, z, G, p, save_y)
    print(f"{spec.name} {spec.rows}x{spec.cols} save_y={save_y}: GPU step done", flush=True)
    _check_hard(orc, spec, z, w, r, spec.name)
    f = orc.fwd(2, 4, widen(to_np(w)), to_np(z), kappa=p.kappa, tau=p.tau, seed=p.seed,
                step=p.step, tensor_id=spec.tensor_id)
    assert abs(r["reg"].item() - f["reg"]) <= 1e-5 * f["reg"], (r["reg"].item(), f["reg"])
    del f
    check_rows(orc, 2, 4, spec, p, w, z, G, wl.lam, r["y"], r["out"], r["dz"], spec.name)


@pytest.mark.parametrize("first_layer", range(0, 32, 4))
def test_all_linear_sweep_sampled(mg, orc, first_layer):
    """Four layers (28 tensors) of the 224-tensor sweep: the step's fused
    forward and recomputing backward; integer outputs in full, the rest on
    sampled rows; the saved-soft-index step gives the same outputs bit for
    bit."""
    import torch
    from workloads import WORKLOADS, llama7b_layer, tensor_inputs
    wl = WORKLOADS["llama7b_all_linear"]
    dev = torch.device("cuda:0")
    p = mg.sample_params(0, 0, wl.kappa, wl.tau)
    for layer in range(first_layer, first_layer + 4):
        for spec in llama7b_layer(layer):
            w, z, G = tensor_inputs(wl, spec, dev)
            r = _step(mg, wl, spec, w, z, G, p, save_y=False)
            rs = _step(mg, wl, spec, w, z, G, p, save_y=True)
            for k in ("out", "idx", "bits", "vals", "vidx", "dz"):
                assert torch.equal(r[k], rs[k]), (spec.name, k)
            del rs
            _check_hard(orc, spec, z, w, r, spec.name)
            check_rows(orc, 2, 4, spec, p, w, z, G, wl.lam, None, r["out"], r["dz"], spec.name)
            del w, z, G, r
        print(f"layer {layer}: 7 tensors match the oracle", flush=True)
        torch.cuda.empty_cache()


def _oracle_reg(orc, n, m, spec, p, w, z, chunk_rows=1024):
    """The oracle regulariser of a whole tensor, summed over row ranges (a row
    range is a tensor with a block offset, so the noise is the whole
    tensor's), to keep the oracle's fp64 soft index of a range small."""
    bpr = spec.cols // m
    total = 0.0
    for r0 in range(0, spec.rows, chunk_rows):
        r1 = min(spec.rows, r0 + chunk_rows)
        f = orc.fwd(n, m, widen(to_np(w[r0:r1])), to_np(z[r0 * bpr:r1 * bpr]), kappa=p.kappa,
                    tau=p.tau, seed=p.seed, step=p.step, tensor_id=spec.tensor_id,
                    block_offset=r0 * bpr)
        total += f["reg"]
        del f
    return total


def test_nemotron_step_sampled_rows(mg, orc):
    """The six Nemotron-shaped 4:8 tensors through the benchmark's step: the
    fused forward saving no soft index (masked weights, regulariser, argmax,
    packed bits), then the backward drawing the soft index again; indices and
    bits in full, the regulariser of each whole tensor within 1e-5, masked
    weights and dz on sampled rows; the step with the soft index saved gives
    the same outputs bit for bit."""
    import torch
    from workloads import WORKLOADS, tensor_inputs
    wl = WORKLOADS["nemotron15b_layer_48"]
    dev = torch.device("cuda:0")
    p = mg.sample_params(0, 5, wl.kappa, wl.tau)
    for spec in wl.tensors:
        w, z, G = tensor_inputs(wl, spec, dev)
        B = spec.rows * spec.cols // 8
        t = mg.Tensor(4, 8, spec.rows, spec.cols, 0, spec.tensor_id)
        res = {}
        for save_y in (False, True):
            out = torch.empty_like(w)
            y = torch.empty_like(z) if save_y else None
            reg = torch.zeros(1, dtype=torch.float64, device=dev)
            idx = torch.empty(B, dtype=torch.uint8, device=dev)
            bits = torch.empty(B, dtype=torch.uint8, device=dev)
            dz = torch.empty_like(z)
            mg.maskgs_fwd_hard(t, p, w, z, out, y, reg, idx, bits)
            mg.maskgs_bwd(t, p, w, None if save_y else z, y, G, wl.lam, dz)
            torch.cuda.synchronize()
            res[save_y] = dict(out=out, reg=reg, idx=idx, bits=bits, dz=dz)
            del y
        r, rs = res[False], res[True]
        for k in ("out", "idx", "bits", "dz"):
            assert torch.equal(r[k], rs[k]), (spec.name, k)
        del res, rs
        print(f"{spec.name} {spec.rows}x{spec.cols}: GPU step done", flush=True)
        h = orc.hard_extract(4, 8, to_np(z), spec.rows, spec.cols)
        assert np.array_equal(to_np(r["idx"]), h["idx"]), spec.name
        assert np.array_equal(to_np(r["bits"]), h["bits"]), spec.name
        del h
        ref = _oracle_reg(orc, 4, 8, spec, p, w, z)
        assert abs(r["reg"].item() - ref) <= 1e-5 * ref, (spec.name, r["reg"].item(), ref)
        check_rows(orc, 4, 8, spec, p, w, z, G, wl.lam, None, r["out"], r["dz"], spec.name)
        del w, z, G, r
        torch.cuda.empty_cache()
