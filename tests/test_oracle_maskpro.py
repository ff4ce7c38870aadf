"""Pins of the MaskPro oracle (oracle/maskpro_oracle.c) against what the
mathematics fixes, independent of the oracle's own code.

Summary page "MaskPro: Linear-Space Probabilistic Learning for Strict
(N:M)-Sparsity on LLMs" (atlas.scime.ai), "Approach": one categorical per
block of M weights, N positions drawn without replacement, policy gradient on
the loss residual with a moving-average baseline; "Limitations": logits start
from an initial mask and a magnitude C.

  - the likelihood of an ordered draw is the Plackett-Luce product
    prod_k p_{j_k} / (1 - sum_{i<k} p_{j_i}), p = softmax(pi), written here
    from that closed form;
  - its gradient against central differences of that closed form;
  - the score-function (REINFORCE) identity, exactly, by enumerating every
    ordered draw: sum_d p(d) L(d) dlogp(d) = d/dpi sum_d p(d) L(d);
  - the Gumbel-top-k draws of the oracle have the Plackett-Luce frequencies
    (chi-square over many blocks sharing one set of logits);
  - the closed form of the moving-average baseline and of the initial logits.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle as orc


def _pl_prob(pi, order):
    """Plackett-Luce probability of an ordered draw, from softmax(pi), fp64."""
    p = np.exp(pi - pi.max())
    p = p / p.sum()
    prob, used = 1.0, 0.0
    for j in order:
        prob *= p[j] / (1.0 - used)
        used += p[j]
    return prob


def _draws(n, m):
    return list(itertools.permutations(range(m), n))


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4), (4, 4), (3, 8)])
def test_logp_is_plackett_luce_and_sums_to_one(n, m):
    rng = np.random.default_rng(n * 10 + m)
    pi = (rng.standard_normal(m) * 1.5).astype(np.float32)
    draws = _draws(n, m)
    order = np.array(draws, dtype=np.uint8)
    lp = orc.maskpro_logp(n, m, np.tile(pi, (len(draws), 1)), order)
    ref = np.array([_pl_prob(pi.astype(np.float64), d) for d in draws])
    assert np.allclose(np.exp(lp), ref, rtol=1e-12, atol=0)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12


def _grad(n, m, pi, order, adv=1.0):
    B = order.shape[0]
    return orc.maskpro_grad(n, m, np.tile(pi, (B, 1)), 1, B * m, advantage=adv, order=order)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4), (4, 4)])
def test_grad_matches_finite_differences_of_closed_form(n, m):
    rng = np.random.default_rng(7 + m)
    pi = (rng.standard_normal(m) * 2.0).astype(np.float32)
    draws = _draws(n, m)
    sel = [draws[i] for i in rng.choice(len(draws), size=min(12, len(draws)), replace=False)]
    order = np.array(sel, dtype=np.uint8)
    g = _grad(n, m, pi, order, adv=1.0)
    h = 1e-6
    x = pi.astype(np.float64)
    for r, d in enumerate(sel):
        fd = np.zeros(m)
        for j in range(m):
            xp, xm = x.copy(), x.copy()
            xp[j] += h
            xm[j] -= h
            fd[j] = (np.log(_pl_prob(xp, d)) - np.log(_pl_prob(xm, d))) / (2 * h)
        assert np.allclose(g[r], fd, atol=1e-8), (d, g[r], fd)


def test_grad_special_cases():
    pi = np.array([0.3, -1.0, 2.0, 0.5], dtype=np.float32)
    p = np.exp(pi.astype(np.float64) - pi.max())
    p /= p.sum()
    # N = 1: the textbook categorical score, onehot - softmax
    for j in range(4):
        g = _grad(1, 4, pi, np.array([[j]], dtype=np.uint8))[0]
        assert np.allclose(g, np.eye(4)[j] - p, atol=1e-14)
    # every score sums to zero (softmax is shift invariant), and it scales with A
    order = np.array(_draws(2, 4), dtype=np.uint8)
    g = _grad(2, 4, pi, order, adv=1.0)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-14)
    assert np.allclose(_grad(2, 4, pi, order, adv=-2.5), -2.5 * g, rtol=1e-15)
    # N = M: the unordered draw is certain, so the score averages to zero over
    # the M! orders and each order's score is the Plackett-Luce one
    order = np.array(_draws(4, 4), dtype=np.uint8)
    g = _grad(4, 4, pi, order)
    w = np.array([_pl_prob(pi.astype(np.float64), d) for d in _draws(4, 4)])
    assert np.allclose((w[:, None] * g).sum(axis=0), 0.0, atol=1e-14)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_reinforce_identity_exact(n, m):
    """sum_d p(d) L(d) dlogp(d) equals the gradient of E[L] (finite differences
    of the closed form), and subtracting a constant baseline changes nothing
    in expectation: the estimator is unbiased."""
    rng = np.random.default_rng(3 * m)
    pi = (rng.standard_normal(m) * 1.2).astype(np.float32)
    draws = _draws(n, m)
    loss_of_set = {s: rng.standard_normal() for s in
                   {frozenset(d) for d in draws}}
    L = np.array([loss_of_set[frozenset(d)] for d in draws])
    order = np.array(draws, dtype=np.uint8)
    x = pi.astype(np.float64)
    p = np.array([_pl_prob(x, d) for d in draws])
    B = len(draws)
    pg = orc.maskpro_grad(n, m, np.tile(pi, (B, 1)), 1, B * m, advantage=1.0, order=order)
    est = (p[:, None] * L[:, None] * pg).sum(axis=0)

    def expected_loss(v):
        return sum(_pl_prob(v, d) * L[i] for i, d in enumerate(draws))

    h = 1e-6
    fd = np.zeros(m)
    for j in range(m):
        xp, xm = x.copy(), x.copy()
        xp[j] += h
        xm[j] -= h
        fd[j] = (expected_loss(xp) - expected_loss(xm)) / (2 * h)
    assert np.allclose(est, fd, atol=1e-8)
    base = 0.7
    est_b = (p[:, None] * (L - base)[:, None] * pg).sum(axis=0)
    assert np.allclose(est_b, fd, atol=1e-8)


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    keep = exp > 0
    chi2 = (((counts - exp) ** 2)[keep] / exp[keep]).sum()
    return stats.chi2.sf(chi2, keep.sum() - 1)


def test_gumbel_top_k_draws_have_plackett_luce_frequencies_24():
    pi = np.array([0.8, -0.4, 0.1, 1.3], dtype=np.float32)
    B = 200_000
    w = np.ones((1, B * 4), dtype=np.float32)
    f = orc.maskpro_fwd(2, 4, w, np.tile(pi, (B, 1)), seed=12345, step=3, tensor_id=2,
                        block_offset=17)
    draws = _draws(2, 4)
    code = f["order"][:, 0].astype(np.int64) * 4 + f["order"][:, 1]
    counts = np.bincount(code, minlength=16)
    assert counts[[j * 4 + j for j in range(4)]].sum() == 0   # never the same position twice
    probs = np.zeros(16)
    for d in draws:
        probs[d[0] * 4 + d[1]] = _pl_prob(pi.astype(np.float64), d)
    assert _chi2_pvalue(counts, probs) > 1e-4


def test_gumbel_top_k_draws_have_plackett_luce_frequencies_48():
    rng = np.random.default_rng(5)
    pi = (rng.standard_normal(8) * 0.8).astype(np.float32)
    B = 150_000
    w = np.ones((1, B * 8), dtype=np.float32)
    f = orc.maskpro_fwd(4, 8, w, np.tile(pi, (B, 1)), seed=99, step=1, tensor_id=5)
    order = f["order"].astype(np.int64)
    x = pi.astype(np.float64)
    # first position: softmax(pi)
    p1 = np.exp(x - x.max())
    p1 /= p1.sum()
    assert _chi2_pvalue(np.bincount(order[:, 0], minlength=8), p1) > 1e-4
    # unordered kept set: sum of the 24 orders of each set
    sets = list(itertools.combinations(range(8), 4))
    index = {s: i for i, s in enumerate(sets)}
    probs = np.array([sum(_pl_prob(x, d) for d in itertools.permutations(s)) for s in sets])
    key = [index[tuple(sorted(r))] for r in order.tolist()]
    counts = np.bincount(np.array(key), minlength=len(sets))
    assert abs(probs.sum() - 1.0) < 1e-12
    assert _chi2_pvalue(counts, probs) > 1e-4


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_fwd_invariants_and_masked_weight(n, m):
    rng = np.random.default_rng(m)
    rows, cols = 7, 6 * m
    B = rows * cols // m
    # bf16-representable weights: the masked weight is the kept weight, exactly
    w = orc.widen_bf16((rng.integers(0, 1 << 16, size=(rows, cols)) & 0xBFFF).astype(np.uint16))
    w = np.where(np.isfinite(w), w, 1.0).astype(np.float32)
    pi = rng.standard_normal((B, m)).astype(np.float32)
    f = orc.maskpro_fwd(n, m, w, pi, seed=4, step=2, tensor_id=1, block_offset=9)
    order = f["order"].astype(np.int64)
    assert all(len(set(r)) == n for r in order.tolist())
    keep = np.zeros((B, m), dtype=bool)
    np.put_along_axis(keep, order, True, axis=1)
    assert np.array_equal(orc.unpack_masks(f["bits"], B, m),
                          (keep.astype(np.uint32) << np.arange(m, dtype=np.uint32)).sum(1))
    expect = np.where(keep.reshape(rows, cols), w, 0.0).astype(np.float32)
    assert np.array_equal(orc.widen_bf16(f["out"]), expect)
    f32 = orc.maskpro_fwd(n, m, w, pi, seed=4, step=2, tensor_id=1, block_offset=9,
                          out_dtype="f32")
    assert np.array_equal(f32["out"], expect)


def test_no_noise_draw_is_descending_top_n():
    pi = np.array([[0.5, 2.0, 2.0, -1.0], [1.0, 1.0, 1.0, 1.0], [3.0, 0.0, 4.0, 5.0]],
                  dtype=np.float32)
    w = np.ones((1, 12), dtype=np.float32)
    f = orc.maskpro_fwd(2, 4, w, pi, flags=orc.MP_NO_NOISE)
    # descending, ties to the lower position
    assert f["order"].tolist() == [[1, 2], [0, 1], [3, 2]]


def test_block_offset_shifts_the_noise_stream():
    """A tensor that starts at global block o draws as rows of a larger
    tensor that starts at 0 (the noise depends on the global block only)."""
    rng = np.random.default_rng(1)
    rows, cols = 6, 32
    w = rng.standard_normal((rows, cols)).astype(np.float32)
    pi = rng.standard_normal((rows * cols // 8, 8)).astype(np.float32)
    full = orc.maskpro_fwd(4, 8, w, pi, seed=3, step=1, tensor_id=4)
    bpr = cols // 8
    part = orc.maskpro_fwd(4, 8, w[2:], pi[2 * bpr:], seed=3, step=1, tensor_id=4,
                           block_offset=2 * bpr)
    assert np.array_equal(part["order"], full["order"][2 * bpr:])


def test_grad_recomputed_draw_and_accumulation():
    rng = np.random.default_rng(2)
    for n, m in [(2, 4), (4, 8)]:
        rows, cols = 5, 4 * m
        B = rows * cols // m
        w = np.ones((rows, cols), dtype=np.float32)
        pi = rng.standard_normal((B, m)).astype(np.float32)
        kw = dict(seed=8, step=6, tensor_id=3, block_offset=11)
        f = orc.maskpro_fwd(n, m, w, pi, **kw)
        g1 = orc.maskpro_grad(n, m, pi, rows, cols, advantage=0.37, order=f["order"])
        g2 = orc.maskpro_grad(n, m, pi, rows, cols, advantage=0.37, **kw)
        assert np.array_equal(g1, g2)
        prev = rng.standard_normal((B, m)).astype(np.float32)
        g3 = orc.maskpro_grad(n, m, pi, rows, cols, advantage=0.37, dpi_prev=prev, **kw)
        assert np.allclose(g3, prev.astype(np.float64) + g1, rtol=0, atol=1e-15)


def test_init_logits():
    rng = np.random.default_rng(3)
    for n, m in [(2, 4), (4, 8)]:
        rows, cols = 4, 4 * m
        B = rows * cols // m
        w = rng.standard_normal((rows, cols)).astype(np.float32)
        pi = orc.maskpro_init(n, m, rows, cols, c=3.5, w=w)
        aw = np.abs(w).reshape(B, m)
        top = np.argsort(-aw, axis=1, kind="stable")[:, :n]
        expect = np.zeros((B, m), dtype=np.float32)
        np.put_along_axis(expect, top, np.float32(3.5), axis=1)
        assert np.array_equal(pi, expect)
        bits = orc.magnitude_mask(n, m, w)
        assert np.array_equal(orc.maskpro_init(n, m, rows, cols, c=3.5, prior_bits=bits), expect)
        # at these logits the noiseless draw is the initial mask
        f = orc.maskpro_fwd(n, m, w, pi, flags=orc.MP_NO_NOISE)
        assert np.array_equal(f["bits"], bits)


def test_baseline_closed_form():
    mu, r = 0.9, 2.0
    adv, b = orc.maskpro_baseline([r] * 5, mu=mu)
    # b_0 = 0, A_t = r - b_t, b_{t+1} = mu b_t + (1 - mu) r  =>  A_t = r mu^t
    assert np.allclose(adv, r * mu ** np.arange(5), rtol=1e-15)
    assert abs(b - r * (1 - mu ** 5)) < 1e-15
    # the advantage of step t does not see residual t in the baseline
    res = np.array([0.3, -1.2, 0.8, 2.0])
    a1, _ = orc.maskpro_baseline(res, mu=0.5)
    res2 = res.copy()
    res2[2] += 10.0
    a2, _ = orc.maskpro_baseline(res2, mu=0.5)
    assert np.allclose(a2[:2], a1[:2]) and abs(a2[2] - a1[2] - 10.0) < 1e-12
    assert abs(a2[3] - a1[3] + 0.5 * 10.0) < 1e-12
    with pytest.raises(ValueError):
        orc.maskpro_baseline([1.0], mu=1.5)
