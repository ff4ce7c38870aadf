"""Pins of the CPU oracle against what the MaskLLM pages and mathematics fix.

Each test checks the oracle against something other than itself: literal values
printed on the MaskLLM summary page (``tests/golden``), closed forms, invariants,
limits stated on the page, brute force on tiny inputs, finite differences, and
independent Philox implementations (PyTorch's and rocRAND's, called, never
copied).  A plausible mistake in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong candidate order) fails at least one test.
"""
import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from conftest import REPO

GOLDEN = os.path.join(REPO, "tests", "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Candidate set S (MaskLLM summary, section 3.2 and Eq. 7)
# --------------------------------------------------------------------------
def test_candidates_2_4_page_order(orc):
    g = _golden("candidates_2_4.json")
    S = orc.candidate_matrix(2, 4)
    assert S.tolist() == g["rows"]


@pytest.mark.parametrize("m", range(1, 9))
def test_candidates_counts_and_balance(orc, m):
    for n in range(1, m + 1):
        c = orc.candidates(n, m)
        assert len(c) == math.comb(m, n)
        assert len(set(c.tolist())) == len(c)
        assert all(bin(int(v)).count("1") == n for v in c)
        assert all(int(v) < (1 << m) for v in c)
        S = orc.candidate_matrix(n, m)
        # every position is kept by C(M-1, N-1) candidates
        assert (S.sum(axis=0) == math.comb(m - 1, n - 1)).all()


def test_candidates_4_8_lexicographic(orc):
    c = orc.candidates(4, 8)
    want = [sum(1 << p for p in t) for t in itertools.combinations(range(8), 4)]
    assert c.tolist() == want
    assert len(c) == 70


def test_candidates_invalid(orc):
    with pytest.raises(ValueError):
        orc.candidates(3, 2)
    with pytest.raises(ValueError):
        orc.candidates(1, 9)


def test_storage_bits_per_parameter(orc):
    # section 1: about 0.65 bits per parameter for a 2:4 mask index
    g = _golden("table7_hyperparameters.json")
    bits = math.log2(len(orc.candidates(2, 4))) / 4
    assert round(bits, 2) == g["mask_bits_per_param_2_4"]


# --------------------------------------------------------------------------
# Philox4x32-10 against independent implementations
# --------------------------------------------------------------------------
def _cases():
    rng = np.random.default_rng(1234)
    cases = [(0, 0, 0), (2**64 - 1, 2**64 - 1, 4 * (2**64 // 4 - 1)), (7, 5, 8)]
    for _ in range(60):
        cases.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                      int(rng.integers(0, 2**63)), 4 * int(rng.integers(0, 2**40))))
    return cases


def _run_harness(exe, cases):
    inp = "".join(f"{s} {ss} {off}\n" for s, ss, off in cases)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [[int(x, 16) for x in line.split()] for line in out.strip().splitlines()]


def _oracle_words(orc, cases):
    res = []
    for seed, ss, off in cases:
        q = off // 4
        ctr = [q & 0xFFFFFFFF, q >> 32, ss & 0xFFFFFFFF, ss >> 32]
        res.append(orc.philox4x32_10(ctr, [seed & 0xFFFFFFFF, seed >> 32]).tolist())
    return res


def test_philox_vs_torch_engine(orc, tmp_path):
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path / "torch_philox")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I" + inc,
                    os.path.join(REPO, "tests", "xcheck", "torch_philox.cpp"), "-o", exe],
                   check=True)
    # torch's offset argument counts 128-bit outputs, not words
    cases = _cases()
    tcases = [(s, ss, off // 4) for s, ss, off in cases]
    assert _run_harness(exe, tcases) == _oracle_words(orc, cases)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_philox_vs_rocrand(orc, tmp_path):
    exe = str(tmp_path / "rocrand_philox")
    subprocess.run(["hipcc", "-O1", os.path.join(REPO, "tests", "xcheck", "rocrand_philox.cpp"),
                    "-o", exe], check=True, capture_output=True)
    cases = _cases()
    assert _run_harness(exe, cases) == _oracle_words(orc, cases)


def test_philox_word_layout(orc):
    # word n of the stream is output n % 4 of call n // 4 with counter
    # (lo32(q), hi32(q), step, tensor_id) and key (lo32(seed), hi32(seed))
    seed, step, tid = 0x1122334455667788, 7, 3
    n0 = (1 << 34) - 6
    words = orc.philox_words(seed, step, tid, n0, 16)
    for t in range(16):
        n = n0 + t
        q = n >> 2
        blk = orc.philox4x32_10([q & 0xFFFFFFFF, q >> 32, step, tid],
                                [seed & 0xFFFFFFFF, seed >> 32])
        assert words[t] == blk[n & 3]


# --------------------------------------------------------------------------
# Uniform and Gumbel noise (section 3.4, Eq. 5)
# --------------------------------------------------------------------------
def test_uniform_exact_open_interval(orc):
    assert orc.uniform(0) == 2.0 ** -24
    assert orc.uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    rng = np.random.default_rng(5)
    for x in rng.integers(0, 2**32, size=2000, dtype=np.uint64):
        x = int(x)
        e = orc.uniform(x)
        assert e == (2 * (x >> 9) + 1) * 2.0 ** -24
        # symmetric: complementing the word reflects the uniform exactly
        assert orc.uniform(x ^ 0xFFFFFFFF) == 1.0 - e
        assert 0.0 < e < 1.0


@pytest.fixture(scope="module")
def gumbel_table(orc):
    return orc.gumbel_all().astype(np.float64)


def test_gumbel_exhaustive_accuracy(gumbel_table):
    """All 2^23 noise values against -ln(-ln eps) in fp64 (section 3.4, Eq. 5):
    within 1.25 ulp of max(|g|, 1) everywhere, the bound the segment-cubic
    contract is built to (the Taylor remainder at |d| <= 1/64 is below 0.15
    ulp; the rest is the rounding of the coefficients and the three fused
    multiply-adds)."""
    k = np.arange(1 << 23, dtype=np.float64)
    eps = (2 * k + 1) * 2.0 ** -24
    ref = -np.log(-np.log(eps))
    # 1 - eps is exact in fp64, so the upper half uses log1p for -ln(eps)
    hi = eps > 0.5
    ref[hi] = -np.log(-np.log1p(-(1.0 - eps[hi])))
    err = np.abs(gumbel_table - ref)
    u1 = np.spacing(np.maximum(np.abs(ref), 1.0).astype(np.float32)).astype(np.float64)
    assert (err <= 1.25 * u1).all(), float((err / u1).max())
    # the noise is monotone in the uniform (inverse CDF of the Gumbel law)
    assert (np.diff(gumbel_table) >= 0).all()


def test_gumbel_moments(gumbel_table):
    """The 2^23 equally spaced uniforms are a midpoint rule for the Gumbel law:
    mean -> Euler-Mascheroni gamma, variance -> pi^2/6."""
    gamma = 0.5772156649015329
    assert abs(gumbel_table.mean() - gamma) < 2e-6
    assert abs(gumbel_table.var() - math.pi ** 2 / 6) < 2e-5


def test_gumbel_coefficients_are_taylor_coefficients(orc):
    """c1, c2, c3 of every segment against central finite differences of the
    exact g(d) = -ln(-ln eps(d)) in fp64 (an independent route to the
    derivatives: a wrong sign, factor or power in a coefficient fails it), and
    c0 against g at the segment centre."""
    co = orc.gumbel_coef().astype(np.float64)
    h = 1.0 / 256.0
    # the segments some uniform falls in: binades 0..22 on both sides, and on
    # side 1 the single value 1 - eps = 1/2 (binade 23, segment 0)
    for side, b, nq in [(s_, b_, 32) for s_ in (0, 1) for b_ in range(23)] + [(1, 23, 1)]:
        q = np.arange(nq, dtype=np.float64)
        vc = 2.0 ** b * (1.0 + (q + 0.5) / 32.0)

        def g(d):
            x = (vc + 2.0 ** b * d) * 2.0 ** -24
            t = -np.log(x) if side == 0 else -np.log1p(-x)
            return -np.log(t)

        f = [g(j * h) for j in (-2, -1, 0, 1, 2)]
        d1 = (f[3] - f[1]) / (2 * h) - (f[4] - 2 * f[3] + 2 * f[1] - f[0]) / (12 * h)
        d2 = (f[3] - 2 * f[2] + f[1]) / h ** 2
        d3 = (f[4] - 2 * f[3] + 2 * f[1] - f[0]) / (2 * h ** 3)
        c = co[side, b, :nq]
        assert np.allclose(c[:, 0], f[2], rtol=1e-7, atol=1e-7), (side, b)
        assert np.allclose(c[:, 1], d1, rtol=1e-4, atol=1e-9), (side, b)
        assert np.allclose(c[:, 2], d2 / 2, rtol=2e-3, atol=1e-9), (side, b)
        assert np.allclose(c[:, 3], d3 / 6, rtol=5e-2, atol=1e-6), (side, b)


# --------------------------------------------------------------------------
# Soft index, soft mask, masked weight (section 3.4, Eqs. 5-7, Algorithm 1)
# --------------------------------------------------------------------------
def _rand_inputs(rows, cols, n, m, seed=0, zstd=1.0):
    rng = np.random.default_rng(seed)
    K = math.comb(m, n)
    w = rng.normal(0, 0.02, size=(rows, cols)).astype(np.float32)
    z = rng.normal(0, zstd, size=(rows * cols // m, K)).astype(np.float32)
    g = rng.normal(0, 1e-3, size=(rows, cols)).astype(np.float32)
    return w, z, g


@pytest.mark.parametrize("nm", [(2, 4), (4, 8), (1, 4), (3, 8)])
def test_softmax_and_soft_mask_invariants(orc, nm):
    n, m = nm
    w, z, _ = _rand_inputs(8, 64, n, m)
    r = orc.fwd(n, m, w, z, kappa=100.0, tau=4.0, seed=3, step=1)
    y, mk = r["y"], r["m"]
    assert (y >= 0).all() and np.allclose(y.sum(1), 1.0, atol=1e-12)
    assert np.allclose(mk.sum(1), n, atol=1e-12)
    assert (mk >= -1e-15).all() and (mk <= 1 + 1e-12).all()


def test_soft_mask_worked_example(orc):
    """Section 3.4, Step 3: 0.7 on [1,1,0,0] and 0.3 on [1,0,1,0] give the
    soft mask [1.0, 0.7, 0.3, 0.0]."""
    g = _golden("soft_mask_example.json")
    kappa, tau = 100.0, 4.0
    p = np.array(g["soft_index"])
    with np.errstate(divide="ignore"):
        logit = np.where(p > 0, np.log(np.maximum(p, 1e-300)), -1e4)
    z = (logit * tau / kappa).astype(np.float32).reshape(1, 6)
    w = np.ones((1, 4), dtype=np.float32)
    r = orc.fwd(2, 4, w, z, kappa=kappa, tau=tau, flags=orc.NO_NOISE, out_dtype="f32")
    assert np.allclose(r["y"][0], p, atol=1e-6)
    assert np.allclose(r["m"][0], g["soft_mask"], atol=1e-6)
    assert np.allclose(r["out"][0], g["soft_mask"], atol=1e-6)


def _perturbed_argmax(orc, n, m, z, kappa, tau, seed, step, tid, block_offset=0):
    """Argmax of the perturbed logits kappa*z + g (the Gumbel-max sample)."""
    B, K = z.shape
    words = orc.philox_words(seed, step, tid, block_offset * K, B * K).reshape(B, K)
    g = np.vectorize(orc.gumbel, otypes=[np.float32])(words)
    a = (np.float32(kappa) * z.astype(np.float64) + g).astype(np.float64)
    return np.argmax(a, axis=1)


def test_tau_to_zero_is_one_hot(orc):
    """Section 3.4: as tau -> 0 the soft index becomes the one-hot Gumbel-max
    sample argmax_i (kappa*pi_i + g_i)."""
    w, z, _ = _rand_inputs(4, 64, 2, 4, seed=9)
    r = orc.fwd(2, 4, w, z, kappa=1.0, tau=1e-4, seed=11, step=2, tensor_id=5)
    k = _perturbed_argmax(orc, 2, 4, z, 1.0, 1e-4, 11, 2, 5)
    hard = np.argmax(r["y"], axis=1)
    assert (hard == k).all()
    assert (r["y"].max(axis=1) > 1 - 1e-9).mean() > 0.99


def test_large_kappa_no_noise_is_argmax(orc):
    """Section 3.4 (kappa): with logits dominating, sampling is deterministic."""
    w, z, _ = _rand_inputs(4, 32, 4, 8, seed=2)
    r = orc.fwd(4, 8, w, z, kappa=1e5, tau=1.0, flags=orc.NO_NOISE)
    assert (np.argmax(r["y"], 1) == np.argmax(z, 1)).all()
    assert (r["y"].max(1) == 1.0).all()


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_gumbel_max_frequencies(orc, nm):
    """Section 3.4, Eq. 5: P(argmax_i [log p_i + g_i] = j) = p_j.  Every block
    gets the same logits and its own noise; with tau tiny the soft index is the
    Gumbel-max sample, whose frequencies must match softmax(kappa*pi) (chi^2)."""
    from scipy import stats
    n, m = nm
    K = math.comb(m, n)
    rng = np.random.default_rng(77)
    zrow = rng.normal(0, 1.0, size=K).astype(np.float32)
    blocks = 240000 if K == 6 else 140000
    cols = m * 1000
    rows = blocks // 1000
    z = np.tile(zrow, (rows * 1000, 1))
    w = np.ones((rows, cols), dtype=np.float32)
    r = orc.fwd(n, m, w, z, kappa=1.0, tau=1e-3, seed=99, step=0)
    counts = np.bincount(np.argmax(r["y"], 1), minlength=K)
    p = np.exp(zrow.astype(np.float64) - zrow.max())
    p /= p.sum()
    chi2 = ((counts - blocks * p) ** 2 / (blocks * p)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, K - 1)


def test_shift_invariance(orc):
    w, z, _ = _rand_inputs(4, 32, 2, 4, seed=4)
    z = (np.round(z * 1024) / 1024).astype(np.float32)  # z + 0.25 stays exact
    r0 = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, flags=orc.EXACT_LOGITS)
    r1 = orc.fwd(2, 4, w, z + np.float32(0.25), kappa=100.0, tau=4.0, flags=orc.EXACT_LOGITS)
    assert np.allclose(r0["y"], r1["y"], rtol=1e-9, atol=1e-14)


def test_masked_weight_and_bf16(orc):
    import torch
    w, z, _ = _rand_inputs(8, 64, 2, 4, seed=6)
    r = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, seed=1, out_dtype="f32")
    rb = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, seed=1, out_dtype="bf16")
    u = w.astype(np.float64).reshape(-1, 4) * r["m"]
    assert np.array_equal(r["out"].reshape(-1, 4), u.astype(np.float32))
    tb = torch.from_numpy(u.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    # one rounding from fp64 vs torch's rounding of the fp32 value: <= 1 bf16 ulp
    d = np.abs(rb["out"].reshape(-1, 4).astype(np.int64) - tb.astype(np.uint16).astype(np.int64))
    assert d.max() <= 1


def test_bf16_from_double_matches_torch_on_fp32_values(orc):
    """For values that are already fp32, one RNE rounding to bf16 is the same
    as torch's fp32 -> bf16 conversion (round to nearest, ties to even)."""
    import torch
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x00000001, 0x00008000, 0x00018000,
                         0x7F7FFFFF, 0x7F7F8000, 0x80000000, 0xBF808000], dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([orc.bf16_from_double(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# Regulariser (section 3.4, Eq. 8)
# --------------------------------------------------------------------------
def test_regulariser_definition_and_hard_limit(orc):
    w, z, _ = _rand_inputs(4, 64, 2, 4, seed=12)
    r = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, seed=4)
    u = w.astype(np.float64).reshape(-1, 4) * r["m"]
    assert math.isclose(r["reg"], float((u * u).sum()), rel_tol=1e-12)
    # tau -> 0 with no noise: the soft mask is the argmax candidate, so the
    # regulariser is the squared norm of the kept weights
    rh = orc.fwd(2, 4, w, z, kappa=100.0, tau=1e-6, flags=orc.NO_NOISE)
    S = np.array(_golden("candidates_2_4.json")["rows"])
    keep = S[np.argmax(z, 1)]
    kept = (w.astype(np.float64).reshape(-1, 4) ** 2 * keep).sum()
    assert math.isclose(rh["reg"], kept, rel_tol=1e-12)


# --------------------------------------------------------------------------
# Backward to the logits
# --------------------------------------------------------------------------
def _loss(orc, n, m, w, z, G, lam, kappa, tau, flags, seed):
    r = orc.fwd(n, m, w, z, kappa=kappa, tau=tau, seed=seed, flags=flags)
    u = w.astype(np.float64).reshape(-1, m) * r["m"]
    return float((G.astype(np.float64).reshape(-1, m) * u).sum() - lam * (u * u).sum())


@pytest.mark.parametrize("nm,tau,kappa,lam", [((2, 4), 4.0, 100.0, 1e-5), ((2, 4), 0.5, 10.0, 0.3),
                                              ((4, 8), 2.0, 100.0, 1e-5), ((4, 8), 1.0, 3.0, 0.5),
                                              ((1, 4), 1.0, 5.0, 0.1), ((2, 4), 1.0, 1.0, 0.25)])
def test_backward_finite_differences(orc, nm, tau, kappa, lam):
    """Central differences of L = sum G.(W.M~) - lambda*sum (W.M~)^2 through the
    oracle's own forward (noise fixed by the seed, logit step in fp64).  The
    logits sit on a 2^-10 grid so that z +- 2^-20 is exact in fp32."""
    n, m = nm
    rng = np.random.default_rng(21)
    K = math.comb(m, n)
    rows, cols = 2, 2 * m
    w = rng.normal(0, 1.0, size=(rows, cols)).astype(np.float32)
    z = (np.round(rng.normal(0, 0.05, size=(rows * cols // m, K)) * 1024) / 1024).astype(np.float32)
    G = rng.normal(0, 1.0, size=(rows, cols)).astype(np.float32)
    flags = orc.EXACT_LOGITS
    dz = orc.bwd(n, m, w, z, G, kappa=kappa, tau=tau, lam=lam, seed=5, flags=flags)
    h = 2.0 ** -20
    fd = np.zeros_like(dz)
    for b in range(z.shape[0]):
        for i in range(K):
            zp = z.copy(); zp[b, i] += np.float32(h)
            zm = z.copy(); zm[b, i] -= np.float32(h)
            assert zp[b, i] - z[b, i] == np.float32(h) and z[b, i] - zm[b, i] == np.float32(h)
            lp = _loss(orc, n, m, w, zp, G, lam, kappa, tau, flags, 5)
            lm = _loss(orc, n, m, w, zm, G, lam, kappa, tau, flags, 5)
            fd[b, i] = (lp - lm) / (2 * h)
    scale = np.abs(dz).max()
    assert scale > 0
    assert np.abs(dz - fd).max() <= 1e-6 * scale
    # softmax Jacobian rows sum to zero
    assert np.abs(dz.sum(1)).max() <= 1e-12 * scale * K


def test_backward_term_isolation_and_accumulate(orc):
    n, m = 2, 4
    w, z, G = _rand_inputs(4, 32, n, m, seed=31)
    kw = dict(kappa=100.0, tau=4.0, seed=2)
    d_lm = orc.bwd(n, m, w, z, G, lam=0.0, **kw)
    d_reg = orc.bwd(n, m, w, z, np.zeros_like(G), lam=1e-5, **kw)
    d_all = orc.bwd(n, m, w, z, G, lam=1e-5, **kw)
    # linear in the upstream gradient and in lambda (fp64 cancellation in
    # dy_i - sum_k y_k dy_k bounds the agreement relative to the largest entry)
    sc = np.abs(d_all).max()
    assert np.abs(d_all - (d_lm + d_reg)).max() <= 1e-12 * sc
    d_reg2 = orc.bwd(n, m, w, z, np.zeros_like(G), lam=2e-5, **kw)
    assert np.abs(d_reg2 - 2 * d_reg).max() <= 1e-12 * np.abs(d_reg).max()
    assert np.abs(d_reg).max() > 0 and np.abs(d_lm).max() > 0
    prev = np.random.default_rng(1).normal(size=d_all.shape).astype(np.float32)
    d_acc = orc.bwd(n, m, w, z, G, lam=1e-5, dz_prev=prev, **kw)
    assert np.allclose(d_acc, prev.astype(np.float64) + d_all, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# Hard mask, packing, 2:4 compaction (section 3.2 inference flow, Alg. 1 step 3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nm", [(2, 4), (4, 8), (1, 4), (3, 8)])
def test_hard_extract_bruteforce(orc, nm):
    n, m = nm
    rows, cols = 6, 5 * m
    rng = np.random.default_rng(41)
    K = math.comb(m, n)
    z = rng.normal(size=(rows * cols // m, K)).astype(np.float32)
    z[3, :] = 0.5  # all tied: the first candidate wins
    z[4, 1] = z[4, K - 1] = 9.0  # tie between 1 and K-1
    r = orc.hard_extract(n, m, z, rows, cols)
    idx = r["idx"].astype(np.int64)
    assert (idx == np.argmax(z, 1)).all()
    assert idx[3] == 0 and idx[4] == 1
    S = np.array([[1 if (c >> j) & 1 else 0 for j in range(m)]
                  for c in (sum(1 << p for p in t) for t in itertools.combinations(range(m), n))])
    if (n, m) == (2, 4):
        S = np.array(_golden("candidates_2_4.json")["rows"])
    bits = np.unpackbits(r["bits"], bitorder="little")[: rows * cols].reshape(-1, m)
    assert (bits == S[idx]).all()
    assert (bits.sum(1) == n).all()


def test_compaction_roundtrip(orc):
    rows, cols = 5, 36  # 45 blocks: odd count exercises the last half byte
    rng = np.random.default_rng(42)
    w = rng.normal(0, 0.02, size=(rows, cols)).astype(np.float32)
    z = rng.normal(size=(rows * cols // 4, 6)).astype(np.float32)
    for raw in (w, w.view(np.uint32).astype(np.uint32) >> 16):
        raw = raw.astype(np.uint16) if raw.dtype != np.float32 else raw
        r = orc.hard_extract(2, 4, z, rows, cols, w_raw=raw)
        B = rows * cols // 4
        nib = np.empty(B, dtype=np.int64)
        nib[0::2] = r["val_idx"][: (B + 1) // 2] & 0xF
        nib[1::2] = r["val_idx"][: B // 2] >> 4
        p0, p1 = nib & 3, nib >> 2
        assert (p0 < p1).all()
        dense = np.zeros((B, 4), dtype=raw.dtype)
        vals = r["values"].reshape(B, 2)
        dense[np.arange(B), p0] = vals[:, 0]
        dense[np.arange(B), p1] = vals[:, 1]
        S = np.array(_golden("candidates_2_4.json")["rows"])
        want = np.where(S[r["idx"]] == 1, raw.reshape(B, 4), 0)
        assert np.array_equal(dense, want.astype(raw.dtype))
        assert r["val_idx"].size == (B + 1) // 2 and (r["val_idx"][-1] >> 4) == 0


# --------------------------------------------------------------------------
# Mask prior (section 3.4, Eqs. 9-10) and magnitude prior
# --------------------------------------------------------------------------
def test_prior_similarity_2_4(orc):
    g = _golden("prior_similarity_2_4.json")
    S = np.array(_golden("candidates_2_4.json")["rows"])
    z = np.zeros((6, 6), dtype=np.float32)
    z[:, 0] = 1.0  # sigma = sqrt(5)/6 for every block
    sigma = math.sqrt(5.0) / 6.0
    bits = np.packbits(S.reshape(-1), bitorder="little")  # block b's prior = candidate b
    out = orc.prior_init(2, 4, z, 1, 24, alpha=3.0, mode=0, prior_bits=bits)
    sim = (out.astype(np.float64) - z) / (3.0 * sigma)
    for b in range(6):
        dots = S @ S[b]
        assert abs(dots.mean() - g["mean_inner_product"]) < 1e-12
        want = np.array([g["inner_product_to_similarity"][str(d)] for d in dots])
        assert np.allclose(sim[b], want, atol=1e-6)
        assert sorted(want.tolist()) == [-1, 0, 0, 0, 0, 1]
        assert want[b] == 1 and (S[np.argmin(want)] + S[b] == 1).all()


def test_prior_similarity_4_8_multiplicities(orc):
    S = orc.candidate_matrix(4, 8)
    rng = np.random.default_rng(0)
    z = rng.normal(0, 0.01, size=(1, 70)).astype(np.float32)
    prior = S[17]
    out = orc.prior_init(4, 8, z, 1, 8, alpha=1.0, mode=0,
                         prior_bits=np.packbits(prior, bitorder="little"))
    sigma = z.astype(np.float64).std()
    sim = np.round((out.astype(np.float64) - z) / sigma).astype(int)[0]
    assert sorted(np.unique(sim, return_counts=True)[1].tolist()) == [1, 1, 16, 16, 36]
    assert sim.sum() == 0 and sim[17] == 2
    assert (sim == S @ prior - 2).all()


def test_prior_alpha_zero_and_mode1(orc):
    rng = np.random.default_rng(1)
    w = rng.normal(0, 0.02, size=(4, 32)).astype(np.float32)
    z = rng.normal(0, 0.01, size=(32, 6)).astype(np.float32)
    assert np.array_equal(orc.prior_init(2, 4, z, 4, 32, alpha=0.0, w=w), z)
    out = orc.prior_init(2, 4, z, 4, 32, alpha=3.0, mode=1, w=w)
    bits = np.unpackbits(orc.magnitude_mask(2, 4, w), bitorder="little").reshape(-1, 4)
    S = np.array(_golden("candidates_2_4.json")["rows"])
    for b in range(32):
        k0 = [i for i in range(6) if (S[i] == bits[b]).all()][0]
        d = out[b].astype(np.float64) - z[b]
        assert abs(d[k0] - 3.0) < 1e-6 and np.count_nonzero(d) == 1
    # a prior that matches no candidate leaves the block unchanged in mode 1
    bad = np.packbits(np.array([1, 1, 1, 0] * 32), bitorder="little")
    assert np.array_equal(orc.prior_init(2, 4, z, 4, 32, alpha=3.0, mode=1, prior_bits=bad), z)


@pytest.mark.parametrize("nm", [(2, 4), (4, 8), (1, 4)])
def test_magnitude_topn_bruteforce(orc, nm):
    n, m = nm
    rng = np.random.default_rng(5)
    w = rng.normal(0, 1, size=(3, 4 * m)).astype(np.float32)
    w[0, :m] = 0.5
    w[0, 1] = -0.5  # ties with sign differences keep the lower positions
    w[1, :m] = np.float32(-0.0)
    bits = np.unpackbits(orc.magnitude_mask(n, m, w), bitorder="little")[: w.size].reshape(-1, m)
    for b, blk in enumerate(w.reshape(-1, m)):
        a = np.abs(blk.astype(np.float64))
        best = None
        for t in itertools.combinations(range(m), n):
            key = (sum(a[list(t)]), [-p for p in t])
            if best is None or key > best[0]:
                best = (key, t)
        want = np.zeros(m, dtype=np.uint8)
        want[list(best[1])] = 1
        assert (bits[b] == want).all(), (b, blk, bits[b], want)


# --------------------------------------------------------------------------
# Runs: sharding invariance, thread invariance, steps
# --------------------------------------------------------------------------
def test_sharding_invariance(orc):
    w, z, G = _rand_inputs(12, 64, 2, 4, seed=50)
    kw = dict(kappa=100.0, tau=0.5, seed=123, step=4, tensor_id=9)
    full = orc.fwd(2, 4, w, z, **kw)
    dfull = orc.bwd(2, 4, w, z, G, lam=1e-5, **kw)
    bpr = 64 // 4
    for r0, r1 in [(0, 5), (5, 6), (6, 12)]:
        part = orc.fwd(2, 4, w[r0:r1], z[r0 * bpr:r1 * bpr], block_offset=r0 * bpr, **kw)
        assert np.array_equal(part["y"], full["y"][r0 * bpr:r1 * bpr])
        assert np.array_equal(part["out"], full["out"][r0:r1])
        dpart = orc.bwd(2, 4, w[r0:r1], z[r0 * bpr:r1 * bpr], G[r0:r1], lam=1e-5,
                        block_offset=r0 * bpr, **kw)
        assert np.array_equal(dpart, dfull[r0 * bpr:r1 * bpr])


def test_thread_count_invariance(orc):
    w, z, _ = _rand_inputs(64, 256, 2, 4, seed=51)
    old = orc.get_threads()
    try:
        orc.set_threads(1)
        a = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0)
        orc.set_threads(4)
        b = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0)
    finally:
        orc.set_threads(old)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["out"], b["out"])
    assert math.isclose(a["reg"], b["reg"], rel_tol=1e-12)


@pytest.mark.parametrize("n,m,rows,cols", [(2, 4, 37, 72), (4, 8, 13, 56), (2, 4, 1, 4)])
def test_thread_count_invariance_of_the_packing_passes(orc, n, m, rows, cols):
    """The hard extraction and the linear-space draw and gradient split their
    work over threads by block, then pack bits and nibbles by output byte; the
    results must not depend on the thread count (odd block counts, so threads
    meet inside a shared byte)."""
    rng = np.random.default_rng(61)
    B = rows * cols // m
    K = len(orc.candidates(n, m))
    z = rng.standard_normal((B, K)).astype(np.float32)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    pi = rng.standard_normal((B, m)).astype(np.float32)
    old = orc.get_threads()
    res = []
    try:
        for t in (1, 3, 4):
            orc.set_threads(t)
            h = orc.hard_extract(n, m, z, rows, cols, w_raw=w if (n, m) == (2, 4) else None)
            f = orc.maskpro_fwd(n, m, w, pi, seed=5, step=1, tensor_id=2, block_offset=3)
            g = orc.maskpro_grad(n, m, pi, rows, cols, advantage=0.7, seed=5, step=1,
                                 tensor_id=2, block_offset=3)
            res.append((h, f, g))
    finally:
        orc.set_threads(old)
    for h, f, g in res[1:]:
        for k in ("idx", "bits", "values", "val_idx"):
            a, b = res[0][0][k], h[k]
            assert (a is None and b is None) or np.array_equal(a, b), k
        for k in ("order", "bits", "out"):
            assert np.array_equal(res[0][1][k], f[k]), k
        assert np.array_equal(res[0][2], g)


def test_steps_and_tensors_draw_fresh_noise(orc):
    """Section 3.4, Algorithm 1: independent noise per step; the counter also
    separates tensors, so layers do not share draws."""
    w, z, _ = _rand_inputs(2, 32, 2, 4, seed=52)
    ys = [orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, step=s, tensor_id=t)["y"]
          for s, t in [(0, 0), (1, 0), (0, 1)]]
    assert not np.allclose(ys[0], ys[1]) and not np.allclose(ys[0], ys[2])
    again = orc.fwd(2, 4, w, z, kappa=100.0, tau=4.0, step=1, tensor_id=0)["y"]
    assert np.array_equal(again, ys[1])


# --------------------------------------------------------------------------
# AdamW on the logits (section 3.4, Algorithm 1 "update logits"; training
# details: AdamW, lr 5e-4 for LLaMA-2 / Nemotron, weight decay 0.1)
# --------------------------------------------------------------------------
def _adamw_state(n, seed):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1, n).astype(np.float32)
    g = (rng.normal(0, 1e-4, n) * rng.choice([1e-3, 1.0, 30.0], n)).astype(np.float32)
    g[:7] = 0.0
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = (rng.normal(0, 1e-4, n) ** 2).astype(np.float32)
    return z, g, m, v


@pytest.mark.parametrize("t", [1, 2, 7, 100, 2000])
def test_adamw_matches_torch_reference(orc, t):
    """Independent implementation: torch.optim.AdamW in fp64 on the CPU, with
    the oracle's fp32 state injected; the oracle is its fp32 rounding."""
    import torch
    z, g, m, v = _adamw_state(4096, t)
    if t == 1:
        m[:] = 0.0
        v[:] = 0.0
    hp = dict(lr=5e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    zo, mo, vo = orc.adamw(z, g, m, v, t=t, **hp)
    p = torch.nn.Parameter(torch.from_numpy(z.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    if t > 1:
        opt.state[p] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                        "exp_avg": torch.from_numpy(m.astype(np.float64)),
                        "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    p.grad = torch.from_numpy(g.astype(np.float64))
    opt.step()
    st = opt.state[p]
    for got, ref, what in [(zo, p.detach().numpy(), "z"), (mo, st["exp_avg"].numpy(), "m"),
                           (vo, st["exp_avg_sq"].numpy(), "v")]:
        # fp32 rounding of the fp64 result (plus a few fp64 ulps)
        bound = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 0.5 + 1e-15 * np.abs(ref)
        assert (np.abs(got.astype(np.float64) - ref) <= bound + 1e-45).all(), (what, t)


def test_adamw_first_step_closed_form(orc):
    """From zero moments, the first bias-corrected step is g/(|g| + eps) per
    logit: z1 = z0 - lr (g/(|g|+eps) + wd z0)."""
    z, g, _, _ = _adamw_state(2048, 5)
    zero = np.zeros_like(z)
    lr, wd, eps = 5e-4, 0.1, 1e-8
    zo, mo, vo = orc.adamw(z, g, zero, zero, lr=lr, eps=eps, weight_decay=wd, t=1)
    z64, g64 = z.astype(np.float64), g.astype(np.float64)
    ref = z64 - lr * (g64 / (np.abs(g64) + eps) + wd * z64)
    assert np.array_equal(zo, ref.astype(np.float32))
    assert np.array_equal(mo, (0.1 * g64).astype(np.float32))
    assert np.array_equal(vo, (0.001 * g64 * g64).astype(np.float32))


def test_adamw_degenerate_cases(orc):
    z, g, m, v = _adamw_state(1024, 9)
    # lr = 0: the logits do not move, the moments still advance
    zo, mo, vo = orc.adamw(z, g, m, v, lr=0.0, t=3)
    assert np.array_equal(zo, z)
    assert not np.array_equal(mo, m)
    # no gradient, no decay, zero moments: nothing moves
    zero = np.zeros_like(z)
    zo, mo, vo = orc.adamw(z, zero, zero, zero, lr=5e-4, weight_decay=0.0, t=4)
    assert np.array_equal(zo, z) and not mo.any() and not vo.any()
    # decay alone shrinks z by the factor (1 - lr wd)
    zo, _, _ = orc.adamw(z, zero, zero, zero, lr=5e-4, weight_decay=0.1, t=4)
    assert np.array_equal(zo, (z.astype(np.float64) * (1 - 5e-5)).astype(np.float32))


# --------------------------------------------------------------------------
# Training diagnostics (section 3.4 kappa discussion / Figure 5, Figure 6,
# Figure 8, Table 14)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_sample_logits_are_the_soft_index_argument(orc, nm):
    """softmax(a) of the exported perturbed logits is the pinned soft index."""
    n, m = nm
    w, z, _ = _rand_inputs(6, 8 * m, n, m, seed=21)
    kw = dict(kappa=100.0, tau=2.0, seed=5, step=3, tensor_id=2, block_offset=7)
    a = orc.sample_logits(n, m, z, 6, 8 * m, **kw).astype(np.float64)
    y = np.exp(a - a.max(axis=1, keepdims=True))
    y /= y.sum(axis=1, keepdims=True)
    assert np.allclose(y, orc.fwd(n, m, w, z, **kw)["y"], rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_mask_stats_closed_forms(orc, nm):
    n, m = nm
    rows, cols = 32, 16 * m
    w, z, _ = _rand_inputs(rows, cols, n, m, seed=22)
    B, K = z.shape
    h = orc.hard_extract(n, m, z, rows, cols)
    s = orc.mask_stats(n, m, z, rows, cols, kappa=100.0, ref_bits=h["bits"], w=w)
    assert s["blocks"] == B and s["changed"] == 0
    # every block's mask differs from its complement
    s = orc.mask_stats(n, m, z, rows, cols, kappa=100.0, ref_bits=h["bits"] ^ 0xFF)
    assert s["changed"] == B
    # magnitude top-n keeps the largest |w| of each block: never less than the
    # learned mask, and equal when the logits follow the magnitude prior
    s = orc.mask_stats(n, m, z, rows, cols, kappa=100.0, w=w)
    assert s["kept_l1"] <= s["magnitude_l1"] and s["kept_l1"] < s["magnitude_l1"]
    zp = orc.prior_init(n, m, np.zeros_like(z), rows, cols, alpha=1.0, mode=1, w=w)
    s = orc.mask_stats(n, m, zp, rows, cols, kappa=100.0, w=w)
    assert s["kept_l1"] == s["magnitude_l1"]
    # maximum probability: uniform for constant logits, one-hot for large kappa
    s = orc.mask_stats(n, m, np.full_like(z, 0.3), rows, cols, kappa=100.0)
    assert abs(s["max_prob"] - B / K) < 1e-9 * B
    s = orc.mask_stats(n, m, z, rows, cols, kappa=1e6)
    assert abs(s["max_prob"] - B) < 1e-6 * B
    # gradient norm: constant gradient c over B*K logits
    s = orc.mask_stats(n, m, z, rows, cols, kappa=1.0, dz=np.full_like(z, 0.125))
    assert s["grad_sq"] == B * K * 0.125 ** 2


def test_mask_change_between_steps_follows_kappa(orc):
    """Figure 5: with the noise dominating (tiny kappa) the sampled masks of two
    steps are independent draws from a near-uniform distribution and differ in
    a fraction 1 - 1/K of the blocks; with the logits dominating they agree."""
    n, m = 2, 4
    rows, cols = 256, 256
    w, z, _ = _rand_inputs(rows, cols, n, m, seed=23, zstd=0.01)
    B, K = z.shape
    for kappa, expect in [(1e-3, 1 - 1 / K), (1e5, 0.0)]:
        s0 = dict(tau=1.0, seed=4, step=0, tensor_id=0, block_offset=0)
        a0 = orc.sample_logits(n, m, z, rows, cols, kappa=kappa, **s0)
        cands = orc.candidates(n, m)
        bits0 = np.packbits(((cands[np.argmax(a0, axis=1)][:, None] >> np.arange(m)) & 1)
                            .astype(np.uint8).reshape(-1), bitorder="little")
        st = orc.mask_stats(n, m, z, rows, cols, kappa=kappa, ref_bits=bits0,
                            sample=dict(s0, step=1))
        frac = st["changed"] / B
        sd = math.sqrt(expect * (1 - expect) / B) + 1e-12
        assert abs(frac - expect) <= 5 * sd + (0.002 if expect == 0 else 0), (kappa, frac)


# --------------------------------------------------------------------------
# Hard Gumbel-max sample with a straight-through gradient (section 3.4,
# Eq. 5 Gumbel-max; the hard/soft variants of the Gumbel-softmax)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_hard_sample_frequencies(orc, nm):
    """Every block gets the same logits and its own noise: the applied hard
    masks are Gumbel-max draws, whose frequencies match softmax(kappa*pi) at
    any temperature (chi^2)."""
    from scipy import stats
    n, m = nm
    K = math.comb(m, n)
    rng = np.random.default_rng(78)
    zrow = rng.normal(0, 1.0, size=K).astype(np.float32)
    blocks = 120000 if K == 6 else 140000
    rows = blocks // 1000
    z = np.tile(zrow, (rows * 1000, 1))
    w = np.ones((rows, m * 1000), dtype=np.float32)
    r = orc.fwd(n, m, w, z, kappa=1.0, tau=3.0, seed=98, step=5, flags=orc.HARD_SAMPLE,
                out_dtype="f32")
    cands = orc.candidates(n, m)
    got = ((r["out"].reshape(-1, m) != 0) * (1 << np.arange(m))).sum(1)
    index = {int(c): i for i, c in enumerate(cands)}
    counts = np.bincount([index[int(g)] for g in got], minlength=K)
    p = np.exp(zrow.astype(np.float64) - zrow.max())
    p /= p.sum()
    chi2 = ((counts - blocks * p) ** 2 / (blocks * p)).sum()
    assert chi2 < stats.chi2.ppf(1 - 1e-6, K - 1)


@pytest.mark.parametrize("nm", [(2, 4), (4, 8)])
def test_hard_sample_forward_and_straight_through(orc, nm):
    n, m = nm
    w, z, G = _rand_inputs(16, 8 * m, n, m, seed=24)
    kw = dict(kappa=100.0, tau=2.0, seed=3, step=1, tensor_id=5, block_offset=9)
    soft = orc.fwd(n, m, w, z, out_dtype="f32", **kw)
    hard = orc.fwd(n, m, w, z, out_dtype="f32", flags=orc.HARD_SAMPLE, **kw)
    # the soft index is unchanged; the applied mask keeps exactly N weights of a
    # valid candidate, bit for bit, and R is the sum of their squares
    assert np.array_equal(soft["y"], hard["y"])
    ob = hard["out"].reshape(-1, m)
    wb = w.reshape(-1, m)
    kept = ob != 0
    assert (kept.sum(1) == n).all() and np.array_equal(ob[kept], wb[kept])
    cands = set(int(c) for c in orc.candidates(n, m))
    assert all(int(k) in cands for k in (kept * (1 << np.arange(m))).sum(1))
    assert abs(hard["reg"] - float((wb[kept].astype(np.float64) ** 2).sum())) <= 1e-12 * hard["reg"]
    # straight-through: only the regulariser term sees the hard mask
    d_soft = orc.bwd(n, m, w, z, G, lam=0.0, **kw)
    d_hard = orc.bwd(n, m, w, z, G, lam=0.0, flags=orc.HARD_SAMPLE, **kw)
    assert np.array_equal(d_soft, d_hard)
    d_hard = orc.bwd(n, m, w, z, G, lam=0.5, flags=orc.HARD_SAMPLE, **kw)
    assert not np.array_equal(d_hard, orc.bwd(n, m, w, z, G, lam=0.5, **kw))
    assert np.abs(d_hard.sum(axis=1)).max() <= 1e-12 * np.abs(d_hard).max()  # sum_i dz_i = 0


@pytest.mark.parametrize("nm,lam,with_g", [((2, 4), 0.25, True), ((4, 8), 0.25, True),
                                            ((2, 4), 0.5, False), ((4, 8), 0.5, False)])
def test_hard_sample_backward_is_straight_through_autograd(orc, nm, lam, with_g):
    """The hard-sample backward against torch autograd of the straight-through
    estimator written out: the applied mask is M_h + M~ - stopgrad(M~), so
    L = sum G.(W.M) - lambda sum (W.M)^2 takes its value at the hard mask M_h
    and its gradient through the soft mask M~ = softmax(a) S.  The perturbed,
    tempered logits a come from the oracle (they fix the noise) and depend on z
    with slope kappa/tau; M_h is read off the oracle's hard-sample forward.
    A soft mask in the regulariser term, a lost factor 2, a flipped sign of
    lambda or a missing kappa/tau all fail this."""
    import torch
    n, m = nm
    rng = np.random.default_rng(41 + m)
    K = math.comb(m, n)
    rows, cols = 8, 8 * m
    w = rng.normal(0, 1.0, size=(rows, cols)).astype(np.float32)
    z = rng.normal(0, 0.05, size=(rows * cols // m, K)).astype(np.float32)
    G = (rng.normal(0, 1.0, size=(rows, cols)) if with_g else np.zeros((rows, cols))).astype(np.float32)
    kappa, tau = 3.0, 1.5
    kw = dict(kappa=kappa, tau=tau, seed=7, step=2, tensor_id=1, block_offset=3)
    a = orc.sample_logits(n, m, z, rows, cols, **kw).astype(np.float64)
    hard = orc.fwd(n, m, w, z, out_dtype="f32", flags=orc.HARD_SAMPLE, **kw)
    mh = (hard["out"].reshape(-1, m) != 0).astype(np.float64)
    cands = orc.candidates(n, m).astype(np.int64)
    S = torch.tensor((cands[:, None] >> np.arange(m)) & 1, dtype=torch.float64)
    zt = torch.tensor(z.astype(np.float64), requires_grad=True)
    slope = kappa / tau
    at = zt * slope + torch.tensor(a - z.astype(np.float64) * slope)
    ms = torch.softmax(at, dim=1) @ S
    mst = torch.tensor(mh) + ms - ms.detach()
    u = torch.tensor(w.astype(np.float64).reshape(-1, m)) * mst
    L = (torch.tensor(G.astype(np.float64).reshape(-1, m)) * u).sum() - lam * (u * u).sum()
    L.backward()
    ref = zt.grad.numpy()
    d = orc.bwd(n, m, w, z, G, lam=lam, flags=orc.HARD_SAMPLE, **kw)
    scale = np.abs(ref).max()
    assert scale > 0
    assert np.abs(d - ref).max() <= 1e-6 * scale
    # the soft regulariser term gives a different gradient on these inputs
    d_soft = orc.bwd(n, m, w, z, G, lam=lam, **kw)
    assert np.abs(d_soft - ref).max() > 1e-3 * scale
