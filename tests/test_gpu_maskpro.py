"""GPU parity of the linear-space mask learner (include/maskpro.h; MaskPro
summary page, "Approach" and "Limitations") against the CPU oracle, through
the C ABI.

Bars:
  - the draw (order, packed mask) and the masked weights: bit-exact (the keys
    fp32(pi + g) decide the draw on both sides in the same precision; the
    masked weight is a copy of the kept weight);
  - the initial logits: bit-exact;
  - the policy gradient dpi = A * dlogp: |d| <= 1e-6 * max(1, |A|) + 1e-5 |ref|.
    Each of the N rounds adds or subtracts a term e/Z in [0, 1] that the fp32
    kernel forms with a few roundings (exp, the sum Z of at most M terms, the
    reciprocal, the product); the error of dlogp measured at most 4.6e-7 of
    its unit scale, within the 1e-6 absolute bound, and A scales it.
Small shapes in full (several workgroups and a ragged tail, odd and
even global block offsets), the draw's Plackett-Luce frequencies, then one
full-size tensor per pattern on sampled rows.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

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


def pack_order(order, m):
    """Oracle draw order [B, N] -> the kernel's packed format."""
    o = order.astype(np.uint32)
    bits = 2 if m == 4 else 3
    v = np.zeros(o.shape[0], dtype=np.uint32)
    for k in range(o.shape[1]):
        v |= o[:, k] << (bits * k)
    return v.astype(np.uint8 if m == 4 else np.uint16)


def order_np(order, m):
    a = to_np(order)
    return a if m == 4 else a.view(np.uint16)


def _order_tensor(B, m, dev):
    import torch
    return torch.empty(B, dtype=torch.uint8 if m == 4 else torch.int16, device=dev)


def assert_pg(got, ref, adv, n, what):
    # dlogp is a unit-scale quantity and A multiplies it, so the absolute bound
    # 1e-6 holds for |A| <= 1 and scales with |A| beyond
    assert_close(got, ref, what, rtol=1e-5, atol=1e-6 * max(1.0, abs(adv)))


CASES = [
    # n, m, rows, cols, w dtype, out dtype, block_offset, tensor_id, seed, step, advantage
    (2, 4, 64, 256, "bf16", "bf16", 0, 0, 0, 0, 1.0),
    (2, 4, 37, 72, "bf16", "bf16", 5, 3, 11, 2, -0.37),   # 666 blocks, odd offset
    (2, 4, 41, 20, "f32", "bf16", 1, 1, 2, 7, 2.5),       # 205 blocks: odd count
    (2, 4, 300, 1024, "f32", "f32", 7, 2, 2 ** 33 + 1, 1, 0.125),
    (4, 8, 37, 72, "bf16", "bf16", 3, 4, 11, 2, 1.0),     # 333 blocks: ragged
    (4, 8, 16, 128, "f32", "f32", 0, 0, 0, 0, -3.0),
    (4, 8, 130, 512, "bf16", "f32", 2, 3, 5, 1, 0.5),
    # global block offsets past 2^40 and the largest step: the Philox counter's
    # high word and the step word both in play
    (2, 4, 33, 64, "bf16", "bf16", 2 ** 40 + 3, 7, 12345, 2 ** 32 - 1, 0.75),
    (4, 8, 9, 64, "bf16", "bf16", 2 ** 45 + 1, 2, 99, 123456, 1.5),
]


@pytest.mark.parametrize("case", CASES)
def test_small_shapes_full(mg, orc, case):
    import torch
    n, m, rows, cols, wdt, odt, off, tid, seed, step, adv = case
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    B = rows * cols // m
    w = _rand((rows, cols), 0.02, dt[wdt], 70 + tid)
    pi = _rand((B, m), 1.0, torch.float32, 71 + tid)
    t = mg.Tensor(n, m, rows, cols, off, tid)
    p = mg.draw_params(seed, step)
    dev = w.device
    out = torch.empty((rows, cols), dtype=dt[odt], device=dev)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev)
    order = _order_tensor(B, m, dev)
    mg.maskpro_fwd(t, p, pi, w, out, bits, order)
    d_saved = torch.empty_like(pi)
    mg.maskpro_bwd(t, p, pi, adv, d_saved, order=order)
    d_rec = torch.empty_like(pi)
    mg.maskpro_bwd(t, p, pi, adv, d_rec)
    torch.cuda.synchronize()

    kw = dict(seed=seed, step=step, tensor_id=tid, block_offset=off)
    pin = to_np(pi)
    f = orc.maskpro_fwd(n, m, widen(to_np(w)), pin, out_dtype=odt, **kw)
    what = str(case)
    assert np.array_equal(order_np(order, m), pack_order(f["order"], m)), what
    assert np.array_equal(to_np(bits), f["bits"]), what
    assert np.array_equal(to_np(out), f["out"]), what
    ref = orc.maskpro_grad(n, m, pin, rows, cols, advantage=adv, order=f["order"])
    assert_pg(to_np(d_saved), ref, adv, n, f"{what} saved order")
    assert np.array_equal(to_np(d_rec), to_np(d_saved)), what
    err = np.abs(to_np(d_saved).astype(np.float64) - ref).max() / abs(adv)
    print(f"{what}: max |d|/|A| = {err:.3g}")


def test_outputs_optional_and_accumulate(mg, orc):
    import torch
    n, m, rows, cols = 2, 4, 9, 64
    B = rows * cols // m
    pi = _rand((B, m), 1.0, torch.float32, 80)
    t = mg.Tensor(n, m, rows, cols, 3, 2)
    p = mg.draw_params(4, 1)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=pi.device)
    mg.maskpro_fwd(t, p, pi, mask_bits=bits)             # no weights, no out
    f = orc.maskpro_fwd(n, m, np.ones((rows, cols), np.float32), to_np(pi), seed=4, step=1,
                        tensor_id=2, block_offset=3)
    assert np.array_equal(to_np(bits), f["bits"])
    prev = _rand((B, m), 0.3, torch.float32, 81)
    d = prev.clone()
    mg.maskpro_bwd(t, p, pi, 0.8, d, accumulate=True)
    ref = orc.maskpro_grad(n, m, to_np(pi), rows, cols, advantage=0.8, dpi_prev=to_np(prev),
                           seed=4, step=1, tensor_id=2, block_offset=3)
    assert_pg(to_np(d), ref, 0.8, n, "accumulate")


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_no_noise_draw_and_extreme_logits(mg, orc, n, m):
    """Without noise the draw is the top-N of pi; logits spread over hundreds of
    units within a block keep the gradient accurate (each round is formed
    against its own largest logit)."""
    import torch
    rng = np.random.default_rng(m)
    rows, cols = 8, 16 * m
    B = rows * cols // m
    pin = rng.standard_normal((B, m)).astype(np.float32)
    pin[::3] *= 150.0                                    # spreads of several hundred
    pin[1::7] = np.round(pin[1::7])                      # ties
    pi = torch.from_numpy(pin).cuda()
    t = mg.Tensor(n, m, rows, cols, 0, 1)
    order = _order_tensor(B, m, pi.device)
    for flags in (mg.MASKGS_NO_NOISE, 0):
        p = mg.draw_params(9, 3, flags)
        mg.maskpro_fwd(t, p, pi, order=order)
        d = torch.empty_like(pi)
        mg.maskpro_bwd(t, p, pi, 1.0, d)
        torch.cuda.synchronize()
        kw = dict(seed=9, step=3, tensor_id=1, flags=flags)
        f = orc.maskpro_fwd(n, m, np.ones((rows, cols), np.float32), pin, **kw)
        assert np.array_equal(order_np(order, m), pack_order(f["order"], m)), flags
        if flags:
            top = np.argsort(-pin, axis=1, kind="stable")[:, :n]
            assert np.array_equal(f["order"], top)
        ref = orc.maskpro_grad(n, m, pin, rows, cols, advantage=1.0, **kw)
        assert_pg(to_np(d), ref, 1.0, n, f"flags {flags}")


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_draw_special_keys(mg, orc, n, m):
    """The draw where keys are NaN, infinite, signed zeros or equal: the order
    is the oracle's scan (strict '>' from the lowest open position, so equal
    keys and a NaN at the first open position keep the lower position) bit for
    bit, with and without noise, and the gradient drawing again equals the one
    from the saved order (NaN where the logits make it NaN)."""
    import torch
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    rng = np.random.default_rng(40 + m)
    pats = [[nan] + [1.0] * (m - 1), [1.0, 2.0, nan] + [0.5] * (m - 3), [nan] * m,
            [inf] + [0.0] * (m - 1), [0.0, inf, 1.0, inf] + [2.0] * (m - 4), [-inf] * m,
            [-inf, 0.0] + [-inf] * (m - 2), [inf, -inf] * (m // 2), [inf] * m,
            [-0.0, 0.0, -0.0, 0.0] + [-1.0] * (m - 4), [0.0, -0.0] * (m // 2),
            [-0.0] * m, [3.0] * m, [1.0, 3.0, 3.0, 1.0] * (m // 4)]
    # every pattern in several rotations, then ordinary blocks
    blocks = [np.roll(np.array(p, np.float32), r) for p in pats for r in range(0, m, 3)]
    blocks += list(rng.standard_normal((64, m)).astype(np.float32))
    pin = np.stack(blocks).astype(np.float32)
    pad = (-len(pin)) % 4
    pin = np.concatenate([pin, rng.standard_normal((pad, m)).astype(np.float32)])
    B = len(pin)
    rows, cols = B // 4, 4 * m
    pi = torch.from_numpy(pin).cuda()
    t = mg.Tensor(n, m, rows, cols, 0, 2)
    for flags in (mg.MASKGS_NO_NOISE, 0):
        p = mg.draw_params(13, 5, flags)
        order = _order_tensor(B, m, pi.device)
        bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=pi.device)
        mg.maskpro_fwd(t, p, pi, mask_bits=bits, order=order)
        d_saved = torch.empty_like(pi)
        d_redrawn = torch.empty_like(pi)
        mg.maskpro_bwd(t, p, pi, 1.0, d_saved, order=order)
        mg.maskpro_bwd(t, p, pi, 1.0, d_redrawn)
        torch.cuda.synchronize()
        kw = dict(seed=13, step=5, tensor_id=2, flags=flags)
        f = orc.maskpro_fwd(n, m, np.ones((rows, cols), np.float32), pin, **kw)
        assert np.array_equal(order_np(order, m), pack_order(f["order"], m)), flags
        assert np.array_equal(to_np(bits), f["bits"]), flags
        np.testing.assert_array_equal(to_np(d_redrawn), to_np(d_saved))
        fin = np.isfinite(pin).all(axis=1)
        ref = orc.maskpro_grad(n, m, pin, rows, cols, advantage=1.0, **kw)
        assert_pg(to_np(d_redrawn)[fin], ref[fin], 1.0, n, f"finite blocks, flags {flags}")


@pytest.mark.parametrize("n,m,source", [(2, 4, "bits"), (2, 4, "w_bf16"), (4, 8, "w_f32"),
                                        (4, 8, "bits"), (2, 4, "w_f32")])
def test_init(mg, orc, n, m, source):
    import torch
    rows, cols = 21, 8 * m
    B = rows * cols // m
    wdt = torch.float32 if source == "w_f32" else torch.bfloat16
    w = _rand((rows, cols), 0.015, wdt, 82)
    w[0, :m] = 0.25                                      # ties keep the lower positions
    t = mg.Tensor(n, m, rows, cols)
    pi = torch.full((B, m), 7.0, device=w.device)
    if source == "bits":
        bits_np = orc.magnitude_mask(n, m, widen(to_np(_rand((rows, cols), 1.0, torch.float32,
                                                                83))))
        mg.maskpro_init(t, pi, 3.5, prior_bits=torch.from_numpy(bits_np).cuda())
        ref = orc.maskpro_init(n, m, rows, cols, c=3.5, prior_bits=bits_np)
    else:
        mg.maskpro_init(t, pi, 3.5, w=w)
        ref = orc.maskpro_init(n, m, rows, cols, c=3.5, w=widen(to_np(w)))
    assert np.array_equal(to_np(pi), ref), source


def _pl_prob(pi, order):
    p = np.exp(pi - pi.max())
    p = p / p.sum()
    prob, used = 1.0, 0.0
    for j in order:
        prob *= p[j] / (1.0 - used)
        used += p[j]
    return prob


def _chi2_p(counts, probs):
    exp = probs * counts.sum()
    keep = exp > 0
    chi2 = (((counts - exp) ** 2)[keep] / exp[keep]).sum()
    return stats.chi2.sf(chi2, keep.sum() - 1)


def test_draw_frequencies_are_plackett_luce(mg):
    """Blocks with identical logits draw ordered positions with the
    Plackett-Luce probabilities of softmax(pi) (sequential draws without
    replacement): 2:4 over the 12 ordered pairs, 4:8 over the first position
    and the 70 unordered sets."""
    import torch
    for n, m, B, pi_row in [(2, 4, 600_000, [0.8, -0.4, 0.1, 1.3]),
                            (4, 8, 400_000, [0.5, -0.2, 1.0, 0.0, -1.1, 0.3, 0.7, -0.5])]:
        pin = np.tile(np.array(pi_row, dtype=np.float32), (B, 1))
        pi = torch.from_numpy(pin).cuda()
        t = mg.Tensor(n, m, 1, B * m, 1234, 6)
        order = _order_tensor(B, m, pi.device)
        mg.maskpro_fwd(t, mg.draw_params(77, 5), pi, order=order)
        v = order_np(order, m).astype(np.int64)
        bits = 2 if m == 4 else 3
        od = np.stack([(v >> (bits * k)) & (m - 1) for k in range(n)], axis=1)
        x = np.array(pi_row, dtype=np.float64)
        if m == 4:
            code = od[:, 0] * 4 + od[:, 1]
            probs = np.zeros(16)
            for d in itertools.permutations(range(4), 2):
                probs[d[0] * 4 + d[1]] = _pl_prob(x, d)
            assert _chi2_p(np.bincount(code, minlength=16), probs) > 1e-4
        else:
            p1 = np.exp(x - x.max())
            assert _chi2_p(np.bincount(od[:, 0], minlength=8), p1 / p1.sum()) > 1e-4
            sets = list(itertools.combinations(range(8), 4))
            index = {s: i for i, s in enumerate(sets)}
            probs = np.array([sum(_pl_prob(x, d) for d in itertools.permutations(s))
                              for s in sets])
            key = np.array([index[tuple(sorted(r))] for r in od.tolist()])
            assert _chi2_p(np.bincount(key, minlength=70), probs) > 1e-4


@pytest.mark.parametrize("wl_key,name", [("llama7b_all_linear", "layers.0.up_proj"),
                                         ("nemotron15b_layer_48", "up_proj")])
def test_full_size_tensor_sampled_rows(mg, orc, wl_key, name):
    """A full-size tensor in the launch configuration the benchmark times: the
    whole tensor on the GPU, the oracle on every 61st row and the last."""
    import torch
    from workloads import WORKLOADS, linear_logits, tensor_inputs
    from gpu_helpers import sample_rows
    wl = WORKLOADS[wl_key]
    spec = [s for s in wl.tensors if s.name == name][0]
    n, m = wl.n, wl.m
    dev = torch.device("cuda:0")
    w, _, _ = tensor_inputs(wl, spec, dev)
    pi = linear_logits(wl, spec, dev)
    t = mg.Tensor(n, m, spec.rows, spec.cols, 0, spec.tensor_id)
    p = mg.draw_params(2024, 3)
    B = t.nblocks
    out = torch.empty_like(w)
    bits = torch.empty((B * m + 7) // 8, dtype=torch.uint8, device=dev)
    order = _order_tensor(B, m, dev)
    mg.maskpro_fwd(t, p, pi, w, out, bits, order)
    dpi = torch.empty_like(pi)
    adv = 0.3
    mg.maskpro_bwd(t, p, pi, adv, dpi, order=order)
    torch.cuda.synchronize()
    bpr = spec.cols // m
    rows = sample_rows(spec.rows)
    sel = torch.tensor(rows, device=dev)
    bsel = (sel[:, None] * bpr + torch.arange(bpr, device=dev)[None, :]).reshape(-1)
    pin = to_np(pi.index_select(0, bsel)).reshape(len(rows), bpr, m)
    wn = widen(to_np(w.index_select(0, sel)))
    outg = to_np(out.index_select(0, sel))
    ordg = order_np(order.index_select(0, bsel), m).reshape(len(rows), bpr)
    dg = to_np(dpi.index_select(0, bsel)).reshape(len(rows), bpr, m)
    for i, r in enumerate(rows):
        kw = dict(seed=p.seed, step=p.step, tensor_id=spec.tensor_id, block_offset=r * bpr)
        f = orc.maskpro_fwd(n, m, wn[i:i + 1], pin[i], **kw)
        assert np.array_equal(ordg[i], pack_order(f["order"], m)), r
        assert np.array_equal(outg[i:i + 1], f["out"]), r
        ref = orc.maskpro_grad(n, m, pin[i], 1, spec.cols, advantage=adv, order=f["order"])
        assert_pg(dg[i], ref, adv, n, f"row {r}")
    # the packed mask is the set of the drawn positions, for every block
    v = order_np(order, m).astype(np.int64)
    bw = 2 if m == 4 else 3
    keep = np.zeros(B, dtype=np.int64)
    for k in range(n):
        keep |= 1 << ((v >> (bw * k)) & (m - 1))
    got = orc.unpack_masks(to_np(bits), B, m).astype(np.int64)
    assert np.array_equal(got, keep)
