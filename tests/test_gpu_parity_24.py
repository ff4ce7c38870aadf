"""GPU parity of the 2:4 path: libmaskgs (through its C ABI) against the CPU oracle.

Same seeded inputs on both sides (generated on the device, copied to the host
for the oracle).  Bars: Philox words, Gumbel noise, argmax indices, packed bits,
compacted values and indices bit-exact; soft index, logit gradient, prior logits
and regulariser within |d| <= 1e-6 + 1e-5|ref|; bf16 masked weights within one
bf16 ulp.  Small shapes are compared in full (several workgroups and a ragged
tail); the full-size workloads are compared on sampled rows.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_helpers import assert_bf16_ulp, assert_close, assert_out, to_np, widen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

LAM = 1e-5


@pytest.fixture(scope="module")
def dev():
    import torch
    import sparsity_masks_weights_amd as mg
    mg.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def mg():
    import sparsity_masks_weights_amd as mg
    return mg


def _rand(shape, std, dtype, dev, seed):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=dev) * std
    return x.to(dtype)


def _run_all(mg, t, p, w, z, G, lam=LAM):
    """fwd (with y and reg) + bwd (recompute and saved-y) + hard extract on GPU."""
    import torch
    dev = w.device
    B, K = t.nblocks, t.k
    out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, K), dtype=torch.float32, device=dev)
    reg = torch.zeros(1, dtype=torch.float64, device=dev)
    mg.maskgs_fwd(t, p, w, z, out, y, reg)
    dz_r = torch.empty((B, K), dtype=torch.float32, device=dev)
    mg.maskgs_bwd(t, p, w, z, None, G, lam, dz_r)
    dz_s = torch.empty_like(dz_r)
    mg.maskgs_bwd(t, p, w, None, y, G, lam, dz_s)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B * 4 + 7) // 8, dtype=torch.uint8, device=dev)
    vals = torch.empty(B * 2, dtype=w.dtype, device=dev)
    vidx = torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
    mg.maskgs_hard_extract(t, z, w, idx, bits, vals, vidx)
    torch.cuda.synchronize()
    return dict(out=to_np(out), y=to_np(y), reg=float(reg.item()), dz_r=to_np(dz_r),
                dz_s=to_np(dz_s), idx=to_np(idx), bits=to_np(bits), vals=to_np(vals),
                vidx=to_np(vidx))


def _oracle_all(orc, t, p, w, z, G, lam=LAM):
    wn, zn, Gn = to_np(w), to_np(z), to_np(G)
    wf = widen(wn)
    kw = dict(kappa=p.kappa, tau=p.tau, seed=p.seed, step=p.step, tensor_id=t.tensor_id,
              block_offset=t.block_offset, flags=p.flags)
    f = orc.fwd(2, 4, wf, zn, out_dtype="bf16", **kw)
    dz = orc.bwd(2, 4, wf, zn, widen(Gn), lam=lam, **kw)
    h = orc.hard_extract(2, 4, zn, t.rows, t.cols, w_raw=wn)
    return f, dz, h


def _compare(res, f, dz, h, what):
    assert_close(res["y"], f["y"], f"{what} y")
    assert_bf16_ulp(res["out"], f["out"], f"{what} out")
    assert abs(res["reg"] - f["reg"]) <= 1e-5 * abs(f["reg"]) + 1e-30, (what, res["reg"], f["reg"])
    assert_close(res["dz_r"], dz, f"{what} dz (recompute)")
    assert_close(res["dz_s"], dz, f"{what} dz (saved y)")
    assert np.array_equal(res["dz_r"], res["dz_s"]), f"{what}: saved-y and recompute differ"
    assert np.array_equal(res["idx"], h["idx"]), f"{what} idx"
    assert np.array_equal(res["bits"], h["bits"]), f"{what} bits"
    assert np.array_equal(res["vals"], h["values"]), f"{what} values"
    assert np.array_equal(res["vidx"], h["val_idx"]), f"{what} val_idx"


# --------------------------------------------------------------------------
# Noise stream
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,step,tid,n0,count", [
    (0, 0, 0, 0, 4096), (0x0123456789ABCDEF, 7, 3, 5, 1000),
    (2**64 - 1, 2**32 - 1, 2**32 - 1, 2**34 - 6, 77), (42, 1, 2, (2**32 - 3) * 4, 64)])
def test_philox_words_bit_exact(dev, mg, orc, seed, step, tid, n0, count):
    import torch
    words = torch.empty(count, dtype=torch.int32, device=dev)
    mg.maskgs_debug_philox(seed, step, tid, n0, words)
    got = to_np(words).view(np.uint32)
    assert np.array_equal(got, orc.philox_words(seed, step, tid, n0, count))


def test_gumbel_exhaustive_bit_exact(dev, mg, orc):
    """Every one of the 2^23 uniforms (random low bits, which the map ignores)."""
    import torch
    k = np.arange(1 << 23, dtype=np.uint64)
    x = ((k << 9) | ((k * 2654435761) & 0x1FF)).astype(np.uint32)
    words = torch.from_numpy(x.view(np.int32)).to(dev)
    g = torch.empty(1 << 23, dtype=torch.float32, device=dev)
    mg.maskgs_debug_gumbel(words, g)
    got = to_np(g)
    ref = orc.gumbel_all()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# Small shapes in full
# --------------------------------------------------------------------------
CASES = [
    # rows, cols, w dtype, block_offset, tensor_id, seed, step, kappa, tau, zstd
    (256, 256, "f32", 0, 0, 0, 0, 100.0, 4.0, 1.0),      # the 256x256 fp32 workload
    (37, 36, "bf16", 0, 5, 9, 3, 100.0, 4.0, 1.0),       # odd block count: ragged pair
    (37, 36, "bf16", 7, 5, 9, 3, 100.0, 4.0, 1.0),       # odd global offset: 4-call pairs
    (64, 1024, "bf16", 123456789, 11, 2**40 + 3, 5, 500.0, 0.05, 1.0),   # annealed end
    (64, 1024, "f32", 5, 12, 7, 5, 500.0, 0.05, 1.0),    # annealed end, large dL/dM
    (300, 512, "bf16", 2, 224, 1, 9, 250.0, 1.0, 0.01),  # small logits, many workgroups
    (1, 4, "f32", 0, 0, 0, 0, 100.0, 4.0, 1.0),          # a single block
    (3, 8, "f32", 1, 0, 0, 0, 100.0, 4.0, 1.0),
    # global blocks near the 2^56 limit: Philox counters with a non-zero high word
    (37, 36, "bf16", 2**56 - 333, 6, 2**63 + 5, 2**32 - 1, 100.0, 4.0, 1.0),   # odd
    (64, 1024, "f32", 2**55 + 2, 13, 1, 1, 100.0, 4.0, 1.0),                # even
]


@pytest.mark.parametrize("case", CASES)
def test_small_shapes_full(dev, mg, orc, case):
    import torch
    rows, cols, wdt, off, tid, seed, step, kappa, tau, zstd = case
    dt = torch.float32 if wdt == "f32" else torch.bfloat16
    w = _rand((rows, cols), 0.02, dt, dev, 1 + tid)
    z = _rand((rows * cols // 4, 6), zstd, torch.float32, dev, 2 + tid)
    G = _rand((rows, cols), 1.0 if wdt == "f32" else 1e-3, dt, dev, 3 + tid)
    t = mg.Tensor(2, 4, rows, cols, off, tid)
    p = mg.sample_params(seed, step, kappa, tau)
    res = _run_all(mg, t, p, w, z, G)
    _compare(res, *_oracle_all(orc, t, p, w, z, G), what=str(case))


def test_fp32_output_and_no_noise(dev, mg, orc):
    import torch
    rows, cols = 33, 64
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 5)
    z = _rand((rows * cols // 4, 6), 1.0, torch.float32, dev, 6)
    t = mg.Tensor(2, 4, rows, cols, 3, 1)
    for flags in (0, mg.MASKGS_NO_NOISE):
        p = mg.sample_params(5, 2, 100.0, 4.0, flags)
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
        y = torch.empty((t.nblocks, 6), dtype=torch.float32, device=dev)
        mg.maskgs_fwd(t, p, w, z, out, y)
        f = orc.fwd(2, 4, widen(to_np(w)), to_np(z), kappa=100.0, tau=4.0, seed=5, step=2,
                    tensor_id=1, block_offset=3, flags=flags, out_dtype="f32")
        assert_close(to_np(y), f["y"], "y")
        assert_out(to_np(out), f["out"], "fp32 out")


def test_bwd_accumulate_and_lambda(dev, mg, orc):
    import torch
    rows, cols = 40, 96
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 7)
    z = _rand((rows * cols // 4, 6), 1.0, torch.float32, dev, 8)
    G = _rand((rows, cols), 1e-3, torch.float32, dev, 9)
    t = mg.Tensor(2, 4, rows, cols, 0, 2)
    p = mg.sample_params(1, 1, 100.0, 4.0)
    prev = _rand((t.nblocks, 6), 1e-3, torch.float32, dev, 10)
    for lam in (0.0, 1e-5, 0.5):
        dz = prev.clone()
        mg.maskgs_bwd(t, p, w, z, None, G, lam, dz, accumulate=True)
        ref = orc.bwd(2, 4, widen(to_np(w)), to_np(z), to_np(G), kappa=100.0, tau=4.0,
                      lam=lam, seed=1, step=1, tensor_id=2, dz_prev=to_np(prev))
        assert_close(to_np(dz), ref, f"accumulate lambda={lam}")


def test_reg_reduce_matches_fwd(dev, mg, orc):
    import torch
    rows, cols = 129, 256
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 11)
    z = _rand((rows * cols // 4, 6), 1.0, torch.float32, dev, 12)
    t = mg.Tensor(2, 4, rows, cols, 5, 4)
    p = mg.sample_params(3, 4, 300.0, 0.5)
    y = torch.empty((t.nblocks, 6), dtype=torch.float32, device=dev)
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    r1 = torch.zeros(1, dtype=torch.float64, device=dev)
    r2 = torch.zeros_like(r1)
    r3 = torch.zeros_like(r1)
    mg.maskgs_fwd(t, p, w, z, out, y, r1)
    mg.maskgs_reg_reduce(t, p, w, z, None, r2)
    mg.maskgs_reg_reduce(t, p, w, None, y, r3)
    f = orc.fwd(2, 4, widen(to_np(w)), to_np(z), kappa=300.0, tau=0.5, seed=3, step=4,
                tensor_id=4, block_offset=5)
    for r in (r1, r2, r3):
        assert abs(r.item() - f["reg"]) <= 1e-5 * f["reg"]


@pytest.mark.parametrize("mode,source", [(0, "bits"), (1, "bits"), (0, "w_bf16"), (0, "w_f32"),
                                         (1, "w_bf16")])
def test_prior_init(dev, mg, orc, mode, source):
    import torch
    rows, cols = 45, 64
    B = rows * cols // 4
    wdt = torch.float32 if source == "w_f32" else torch.bfloat16
    w = _rand((rows, cols), 0.02, wdt, dev, 13)
    w[0, :4] = 0.5  # magnitude ties keep the lower positions
    w[1, :4] = -0.5
    z = _rand((B, 6), 0.01, torch.float32, dev, 14)
    t = mg.Tensor(2, 4, rows, cols)
    zz = z.clone()
    if source == "bits":
        rng = np.random.default_rng(3)
        S = np.array(orc.candidates(2, 4))
        masks = S[rng.integers(0, 6, size=B)]
        masks[::17] = 0b0111  # invalid priors: no equal candidate
        nib = np.zeros((B + 1) // 2 * 2, dtype=np.uint8)
        nib[:B] = masks
        bits_np = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
        bits = torch.from_numpy(bits_np).to(dev)
        mg.maskgs_prior_init(t, zz, 3.0, mode, prior_bits=bits)
        ref = orc.prior_init(2, 4, to_np(z), rows, cols, alpha=3.0, mode=mode,
                             prior_bits=bits_np)
    else:
        mg.maskgs_prior_init(t, zz, 3.0, mode, w=w)
        ref = orc.prior_init(2, 4, to_np(z), rows, cols, alpha=3.0, mode=mode,
                             w=widen(to_np(w)))
    assert_close(to_np(zz), ref, f"prior mode {mode} {source}")


def test_empty_and_repeat_determinism(dev, mg, orc):
    import torch
    t0 = mg.Tensor(2, 4, 0, 64)
    e = torch.empty(0, device=dev)
    mg.maskgs_fwd(t0, mg.sample_params(), e.bfloat16(), e, e.bfloat16())
    rows, cols = 512, 1024
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 15)
    z = _rand((rows * cols // 4, 6), 1.0, torch.float32, dev, 16)
    G = _rand((rows, cols), 1e-3, torch.bfloat16, dev, 17)
    t = mg.Tensor(2, 4, rows, cols, 0, 3)
    p = mg.sample_params(2, 6, 180.0, 2.0)
    a = _run_all(mg, t, p, w, z, G)
    b = _run_all(mg, t, p, w, z, G)
    for k in a:
        if k == "reg":
            assert abs(a[k] - b[k]) <= 1e-12 * abs(a[k])
        else:
            assert np.array_equal(a[k], b[k]), k


def test_row_sharding_is_invariant(dev, mg):
    """Row ranges with matching block offsets reproduce the whole-tensor call."""
    import torch
    rows, cols = 96, 512
    bpr = cols // 4
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 18)
    z = _rand((rows * bpr, 6), 1.0, torch.float32, dev, 19)
    G = _rand((rows, cols), 1e-3, torch.bfloat16, dev, 20)
    p = mg.sample_params(4, 2, 100.0, 4.0)
    full = _run_all(mg, mg.Tensor(2, 4, rows, cols, 0, 6), p, w, z, G)
    for r0, r1 in [(0, 31), (31, 32), (32, 96)]:
        t = mg.Tensor(2, 4, r1 - r0, cols, r0 * bpr, 6)
        part = _run_all(mg, t, p, w[r0:r1], z[r0 * bpr:r1 * bpr], G[r0:r1])
        sl = slice(r0 * bpr, r1 * bpr)
        assert np.array_equal(part["y"], full["y"][sl])
        assert np.array_equal(part["out"], full["out"][r0:r1])
        assert np.array_equal(part["dz_s"], full["dz_s"][sl])


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[4], CASES[5]])
def test_fwd_hard_equals_fwd_then_extract(dev, mg, orc, case):
    """The fused forward + hard mask gives bit-identical outputs to maskgs_fwd
    followed by maskgs_hard_extract, and the oracle's."""
    import torch
    rows, cols, wdt, off, tid, seed, step, kappa, tau, zstd = case
    dt = torch.float32 if wdt == "f32" else torch.bfloat16
    w = _rand((rows, cols), 0.02, dt, dev, 1 + tid)
    z = _rand((rows * cols // 4, 6), zstd, torch.float32, dev, 2 + tid)
    G = _rand((rows, cols), 1e-3, dt, dev, 3 + tid)
    t = mg.Tensor(2, 4, rows, cols, off, tid)
    p = mg.sample_params(seed, step, kappa, tau)
    ref = _run_all(mg, t, p, w, z, G)
    B = t.nblocks
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, 6), dtype=torch.float32, device=dev)
    reg = torch.zeros(1, dtype=torch.float64, device=dev)
    idx = torch.empty(B, dtype=torch.uint8, device=dev)
    bits = torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
    vals = torch.empty(2 * B, dtype=dt, device=dev)
    vidx = torch.empty((B + 1) // 2, dtype=torch.uint8, device=dev)
    mg.maskgs_fwd_hard(t, p, w, z, out, y, reg, idx, bits, vals, vidx)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), ref["out"])
    assert np.array_equal(to_np(y), ref["y"])
    assert abs(reg.item() - ref["reg"]) <= 1e-12 * abs(ref["reg"])
    for name, got in (("idx", idx), ("bits", bits), ("vals", vals), ("vidx", vidx)):
        assert np.array_equal(to_np(got), ref[name]), name
    h = orc.hard_extract(2, 4, to_np(z), rows, cols, w_raw=to_np(w))
    assert np.array_equal(to_np(bits), h["bits"]) and np.array_equal(to_np(vals), h["values"])


@pytest.mark.parametrize("save_y,flags", [(True, 0), (False, 0), (True, 2), (False, 2)])
def test_autograd_pairing_matches_the_abi_calls(mg, save_y, flags):
    """masked_weight (torch.autograd.Function over maskgs_fwd / maskgs_bwd)
    gives exactly the outputs of the direct calls, also under the hard sample
    (flags 2), where the backward recomputes the soft index whatever save_y
    asks."""
    import torch
    assert flags in (0, mg.MASKGS_HARD_SAMPLE)
    rows, cols = 37, 72
    B = rows * cols // 4
    dev = torch.device("cuda:0")
    w = _rand((rows, cols), 0.02, torch.bfloat16, dev, 90)
    z0 = _rand((B, 6), 1.0, torch.float32, dev, 91)
    G = _rand((rows, cols), 1e-3, torch.bfloat16, dev, 92)
    t = mg.Tensor(2, 4, rows, cols, 5, 3)
    p = mg.sample_params(11, 2, 100.0, 4.0, flags)
    z = z0.clone().requires_grad_(True)
    out, reg = mg.masked_weight(z, w, t, p, lam=1e-5, save_y=save_y)
    out.backward(G)
    ref_out = torch.empty_like(w)
    ref_reg = torch.zeros(1, dtype=torch.float64, device=w.device)
    mg.maskgs_fwd(t, p, w, z0, ref_out, None, ref_reg)
    ref_dz = torch.empty_like(z0)
    mg.maskgs_bwd(t, p, w, z0, None, G, 1e-5, ref_dz)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(reg, ref_reg)
    assert not reg.requires_grad
    assert torch.equal(z.grad, ref_dz)
