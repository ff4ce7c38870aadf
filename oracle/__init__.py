"""CPU oracle of the MaskLLM differentiable N:M mask path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the ``sparsity_masks_weights_amd`` package and its HIP library) never imports,
links or calls it, and shares no code with it.

The arithmetic lives in ``maskgs_oracle.c`` (plain C, fp64 apart from the fp32
noise contract described there); this module only builds that file with gcc and
marshals numpy arrays into it.  Every function cites the passage of the MaskLLM
summary page ("MaskLLM: Learnable Semi-Structured Sparsity for Large Language
Models", paper-graph-ui summary of arXiv 2409.17481) that it follows.

``maskpro_oracle.c`` (built into the same library) holds the linear-space
variant MaskPro ("MaskPro: Linear-Space Probabilistic Learning for Strict
(N:M)-Sparsity on LLMs", atlas.scime.ai summary page); its functions are the
``maskpro_*`` ones below and its readings are listed in that file's header.

Parity pins of this oracle live in ``tests/test_oracle_*.py``.  Parity unpinned
(self-consistent definitions the pages do not fix): the choice of Philox word
layout, of the uniform map and of the contract logarithm's coefficients.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maskgs_oracle.c")
_SRC_MP = os.path.join(_HERE, "maskpro_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

NO_NOISE = 1
EXACT_LOGITS = 2
HARD_SAMPLE = 4

_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles).  Returns the .so path."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
           "-fPIC", "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_MP, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    L = ctypes.CDLL(_LIB)
    c = ctypes
    P = c.c_void_p
    L.orc_set_threads.argtypes = [c.c_int]
    L.orc_get_threads.restype = c.c_int
    L.orc_candidates.argtypes = [c.c_int, c.c_int, P, c.c_int]
    L.orc_candidates.restype = c.c_int
    L.orc_philox4x32_10.argtypes = [P, P, P]
    L.orc_philox_word.argtypes = [c.c_uint64, c.c_uint32, c.c_uint32, c.c_uint64]
    L.orc_philox_word.restype = c.c_uint32
    L.orc_philox_words.argtypes = [c.c_uint64, c.c_uint32, c.c_uint32, c.c_uint64, c.c_int64, P]
    L.orc_uniform.argtypes = [c.c_uint32]
    L.orc_uniform.restype = c.c_float
    L.orc_gumbel_coef.argtypes = [P]
    L.orc_gumbel_coef.restype = None
    L.orc_gumbel.argtypes = [c.c_uint32]
    L.orc_gumbel.restype = c.c_float
    L.orc_gumbel_all.argtypes = [P]
    L.orc_bf16_from_double.argtypes = [c.c_double]
    L.orc_bf16_from_double.restype = c.c_uint16
    common = [c.c_int, c.c_int, c.c_int64, c.c_int64, c.c_uint64, c.c_uint32,
              c.c_uint64, c.c_uint32, c.c_float, c.c_float, c.c_uint32]
    L.orc_fwd.argtypes = common + [P, P, P, P, P, P, P]
    L.orc_fwd.restype = c.c_int
    L.orc_bwd.argtypes = common + [P, P, P, c.c_double, P, P]
    L.orc_bwd.restype = c.c_int
    L.orc_hard_extract.argtypes = [c.c_int, c.c_int, c.c_int64, c.c_int64, P, P, c.c_int,
                                   P, P, P, P]
    L.orc_hard_extract.restype = c.c_int
    L.orc_sample_logits.argtypes = common + [P, P]
    L.orc_sample_logits.restype = c.c_int
    L.orc_adamw.argtypes = [c.c_int64, P, P, P, P, c.c_double, c.c_double, c.c_double,
                            c.c_double, c.c_double, c.c_uint32]
    L.orc_adamw.restype = c.c_int
    L.orc_magnitude_mask.argtypes = [c.c_int, c.c_int, c.c_int64, c.c_int64, P, P]
    L.orc_magnitude_mask.restype = c.c_int
    L.orc_prior_init.argtypes = [c.c_int, c.c_int, c.c_int64, c.c_int64, P, P, P,
                                 c.c_float, c.c_int]
    L.orc_prior_init.restype = c.c_int
    mp = [c.c_int, c.c_int, c.c_int64, c.c_int64, c.c_uint64, c.c_uint32, c.c_uint64,
          c.c_uint32, c.c_uint32]
    L.orc_mp_fwd.argtypes = mp + [P, P, P, P, P, P]
    L.orc_mp_fwd.restype = c.c_int
    L.orc_mp_grad.argtypes = mp + [P, P, c.c_double, P, P]
    L.orc_mp_grad.restype = c.c_int
    L.orc_mp_logp.argtypes = [c.c_int, c.c_int, c.c_int64, P, P, P]
    L.orc_mp_logp.restype = c.c_int
    L.orc_mp_init.argtypes = [c.c_int, c.c_int, c.c_int64, c.c_int64, P, P, c.c_float, P]
    L.orc_mp_init.restype = c.c_int
    L.orc_mp_baseline.argtypes = [c.c_int64, P, c.c_double, P, P]
    L.orc_mp_baseline.restype = c.c_int
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def widen_bf16(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the same values as fp32 (exact)."""
    u = np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def set_threads(t: int) -> None:
    lib().orc_set_threads(int(t))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def candidates(n: int, m: int) -> np.ndarray:
    """Candidate masks S as uint8 bitmasks (bit j = keep position j)."""
    buf = np.zeros(128, dtype=np.uint8)
    k = lib().orc_candidates(n, m, _ptr(buf), 128)
    if k < 0:
        raise ValueError(f"invalid N:M {n}:{m}")
    return buf[:k].copy()


def candidate_matrix(n: int, m: int) -> np.ndarray:
    """S as a {0,1} matrix of shape [K, M] (section 3.4, Eq. 7)."""
    c = candidates(n, m)
    return ((c[:, None] >> np.arange(m)[None, :]) & 1).astype(np.int64)


def philox4x32_10(counter, key) -> np.ndarray:
    ctr = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(ctr), _ptr(k), _ptr(out))
    return out


def philox_words(seed: int, step: int, tensor_id: int, n0: int, count: int) -> np.ndarray:
    out = np.zeros(count, dtype=np.uint32)
    lib().orc_philox_words(seed, step, tensor_id, n0, count, _ptr(out))
    return out


def uniform(x: int) -> float:
    return float(lib().orc_uniform(int(x)))


def gumbel_coef() -> np.ndarray:
    """The noise contract's fp32 Taylor coefficients, [side, binade, segment, 4]
    = (2, 24, 32, 4), c0..c3 of -ln(-ln eps) about each segment centre."""
    out = np.zeros((2, 24, 32, 4), dtype=np.float32)
    lib().orc_gumbel_coef(_ptr(out))
    return out


def gumbel(x: int) -> float:
    return float(lib().orc_gumbel(int(x)))


def gumbel_all() -> np.ndarray:
    """g for all 2^23 uniforms, indexed by x >> 9."""
    out = np.zeros(1 << 23, dtype=np.float32)
    lib().orc_gumbel_all(_ptr(out))
    return out


def bf16_from_double(v: float) -> int:
    return int(lib().orc_bf16_from_double(float(v)))


def fwd(n, m, w, z, *, kappa, tau, seed=0, step=0, tensor_id=0, block_offset=0, flags=0,
        out_dtype="bf16"):
    """Forward of the mask path on a [rows, cols] weight.

    Returns dict(y=[B,K] f64, m=[B,M] f64, out=[rows,cols] (uint16 bf16 bits or
    f32), reg=float).  w is fp32 (widen bf16 first), z is fp32 [B, K].
    """
    w = _f32(w)
    rows, cols = w.shape
    B = rows * (cols // m)
    K = len(candidates(n, m))
    z = _f32(z).reshape(B, K)
    y = np.zeros((B, K), dtype=np.float64)
    mk = np.zeros((B, m), dtype=np.float64)
    reg = ctypes.c_double(0.0)
    out16 = np.zeros((rows, cols), dtype=np.uint16) if out_dtype == "bf16" else None
    out32 = np.zeros((rows, cols), dtype=np.float32) if out_dtype == "f32" else None
    rc = lib().orc_fwd(n, m, rows, cols, block_offset, tensor_id, seed, step, kappa, tau, flags,
                       _ptr(w), _ptr(z), _ptr(y), _ptr(mk), _ptr(out16), _ptr(out32),
                       ctypes.addressof(reg))
    if rc != 0:
        raise ValueError("oracle fwd: invalid arguments")
    return dict(y=y, m=mk, out=out16 if out16 is not None else out32, reg=reg.value)


def bwd(n, m, w, z, g_up, *, kappa, tau, lam, seed=0, step=0, tensor_id=0, block_offset=0,
        flags=0, dz_prev=None):
    """Gradient of L_LM - lambda*R with respect to the logits, [B, K] f64."""
    w = _f32(w)
    rows, cols = w.shape
    B = rows * (cols // m)
    K = len(candidates(n, m))
    z = _f32(z).reshape(B, K)
    g_up = _f32(g_up).reshape(rows, cols)
    prev = None if dz_prev is None else _f32(dz_prev).reshape(B, K)
    dz = np.zeros((B, K), dtype=np.float64)
    rc = lib().orc_bwd(n, m, rows, cols, block_offset, tensor_id, seed, step, kappa, tau, flags,
                       _ptr(w), _ptr(z), _ptr(g_up), float(lam), _ptr(prev), _ptr(dz))
    if rc != 0:
        raise ValueError("oracle bwd: invalid arguments")
    return dz


def adamw(z, g, m, v, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, t=1):
    """One AdamW update of the logits z with gradient g (fp32 arrays of one
    shape); returns new (z, m, v) as fp32 arrays, inputs untouched.  The
    update rule and its reading are in maskgs_oracle.c (orc_adamw)."""
    z = _f32(z).copy()
    g = _f32(g).reshape(z.shape)
    m = _f32(m).reshape(z.shape).copy()
    v = _f32(v).reshape(z.shape).copy()
    rc = lib().orc_adamw(z.size, _ptr(z), _ptr(g), _ptr(m), _ptr(v), float(lr), float(beta1),
                         float(beta2), float(eps), float(weight_decay), int(t))
    if rc != 0:
        raise ValueError("oracle adamw: invalid arguments")
    return z, m, v


def sample_logits(n, m, z, rows, cols, *, kappa, tau, seed=0, step=0, tensor_id=0,
                  block_offset=0, flags=0):
    """The perturbed, tempered logits a_i = fp32(fp32(kappa z_i + g_i) fp32(1/tau))
    of every block, fp32 [B, K] (the argument of Eq. 6's softmax)."""
    B = rows * (cols // m)
    K = len(candidates(n, m))
    z = _f32(z).reshape(B, K)
    a = np.zeros((B, K), dtype=np.float32)
    rc = lib().orc_sample_logits(n, m, rows, cols, block_offset, tensor_id, seed, step, kappa,
                                 tau, flags, _ptr(z), _ptr(a))
    if rc != 0:
        raise ValueError("oracle sample_logits: invalid arguments")
    return a


def unpack_masks(bits, nblocks, m):
    """Per-block masks (uint8 bitmasks) from the packed LSB-first stream."""
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    allbits = np.unpackbits(bits, bitorder="little")[: nblocks * m].reshape(nblocks, m)
    return (allbits.astype(np.uint32) << np.arange(m, dtype=np.uint32)).sum(axis=1).astype(np.uint8)


def mask_stats(n, m, z, rows, cols, *, kappa, ref_bits=None, w=None, dz=None, sample=None):
    """Training diagnostics of one tensor, as sums over its blocks (MaskLLM
    summary, section 3.4 kappa discussion / Figure 5, Figure 6, Figure 8,
    Table 14):
      blocks        number of blocks;
      changed       blocks whose hard mask differs from ref_bits (packed);
      max_prob      sum over blocks of max_i softmax(kappa z)_i (fp64);
      kept_l1       sum of |w| at the hard mask's kept positions;
      magnitude_l1  sum of |w| at the magnitude top-n positions;
      grad_sq       sum of dz^2 over all logits (fp64).
    The hard mask is S[first argmax_i z_i], or with sample = dict(tau=..., seed=...,
    step=..., tensor_id=..., block_offset=..., flags=...) the Gumbel-max sample
    S[first argmax_i a_i] of the noise contract.  w: fp32 values [rows, cols]."""
    B = rows * (cols // m)
    cands = candidates(n, m)
    K = len(cands)
    z = _f32(z).reshape(B, K)
    key = z if sample is None else sample_logits(n, m, z, rows, cols, kappa=kappa, **sample)
    hard = cands[np.argmax(key, axis=1)]          # first maximum per block
    out = dict(blocks=B, changed=0, max_prob=0.0, kept_l1=0.0, magnitude_l1=0.0, grad_sq=0.0)
    if ref_bits is not None:
        out["changed"] = int((unpack_masks(ref_bits, B, m) != hard).sum())
    z64 = z.astype(np.float64)
    e = np.exp(float(kappa) * (z64 - z64.max(axis=1, keepdims=True)))
    out["max_prob"] = float((1.0 / e.sum(axis=1)).sum())
    if w is not None:
        aw = np.abs(_f32(w).astype(np.float64)).reshape(B, m)
        pos = np.arange(m, dtype=np.uint32)
        keep = ((hard[:, None].astype(np.uint32) >> pos) & 1).astype(bool)
        out["kept_l1"] = float(aw[keep].sum())
        mag = unpack_masks(magnitude_mask(n, m, w), B, m)
        keep_mag = ((mag[:, None].astype(np.uint32) >> pos) & 1).astype(bool)
        out["magnitude_l1"] = float(aw[keep_mag].sum())
    if dz is not None:
        d = _f32(dz).astype(np.float64)
        out["grad_sq"] = float((d * d).sum())
    return out


def hard_extract(n, m, z, rows, cols, w_raw=None):
    """Argmax index, packed bits and (2:4) compacted values / 2-bit indices.

    w_raw: the weight as stored (uint16 bf16 bits or float32), [rows, cols].
    """
    B = rows * (cols // m)
    K = len(candidates(n, m))
    z = _f32(z).reshape(B, K)
    idx = np.zeros(B, dtype=np.uint8)
    bits = np.zeros((B * m + 7) // 8, dtype=np.uint8)
    values = val_idx = None
    wb = 0
    if w_raw is not None:
        w_raw = np.ascontiguousarray(w_raw)
        wb = w_raw.dtype.itemsize
        values = np.zeros(B * n, dtype=w_raw.dtype)
        val_idx = np.zeros((B + 1) // 2, dtype=np.uint8)
    rc = lib().orc_hard_extract(n, m, rows, cols, _ptr(z), _ptr(w_raw), wb, _ptr(idx),
                                _ptr(bits), _ptr(values), _ptr(val_idx))
    if rc != 0:
        raise ValueError(f"oracle hard_extract: rc={rc}")
    return dict(idx=idx, bits=bits, values=values, val_idx=val_idx)


def magnitude_mask(n, m, w):
    w = _f32(w)
    rows, cols = w.shape
    B = rows * (cols // m)
    bits = np.zeros((B * m + 7) // 8, dtype=np.uint8)
    if lib().orc_magnitude_mask(n, m, rows, cols, _ptr(w), _ptr(bits)) != 0:
        raise ValueError("oracle magnitude_mask: invalid arguments")
    return bits


def prior_init(n, m, z, rows, cols, *, alpha, mode=0, prior_bits=None, w=None):
    """Eq. 9-10 prior seeding; returns a new fp32 [B, K] array."""
    B = rows * (cols // m)
    K = len(candidates(n, m))
    zz = _f32(z).reshape(B, K).copy()
    pb = None if prior_bits is None else np.ascontiguousarray(prior_bits, dtype=np.uint8)
    ww = None if w is None else _f32(w)
    if pb is None and ww is None:
        raise ValueError("prior_init needs prior_bits or w")
    rc = lib().orc_prior_init(n, m, rows, cols, _ptr(zz), _ptr(pb), _ptr(ww), float(alpha),
                              int(mode))
    if rc != 0:
        raise ValueError(f"oracle prior_init: rc={rc}")
    return zz


# --------------------------------------------------------------------------
# MaskPro (linear-space logits, N-way draw without replacement, policy
# gradient); arithmetic and readings in maskpro_oracle.c.
# --------------------------------------------------------------------------
MP_NO_NOISE = 1


def maskpro_fwd(n, m, w, pi, *, seed=0, step=0, tensor_id=0, block_offset=0, flags=0,
                out_dtype="bf16"):
    """Ordered draw and masked weight ("Approach": N-way sampling without
    replacement from one categorical per block of M).

    w: fp32 [rows, cols]; pi: fp32 [B, M].  Returns dict(order=[B, N] uint8
    positions in draw order, bits=packed LSB-first mask, out=[rows, cols]
    masked weight (uint16 bf16 bits or fp32))."""
    w = _f32(w)
    rows, cols = w.shape
    B = rows * (cols // m)
    pi = _f32(pi).reshape(B, m)
    order = np.zeros((B, n), dtype=np.uint8)
    bits = np.zeros((B * m + 7) // 8, dtype=np.uint8)
    out16 = np.zeros((rows, cols), dtype=np.uint16) if out_dtype == "bf16" else None
    out32 = np.zeros((rows, cols), dtype=np.float32) if out_dtype == "f32" else None
    rc = lib().orc_mp_fwd(n, m, rows, cols, block_offset, tensor_id, seed, step, flags,
                          _ptr(w), _ptr(pi), _ptr(order), _ptr(bits), _ptr(out16), _ptr(out32))
    if rc != 0:
        raise ValueError("oracle maskpro_fwd: invalid arguments")
    return dict(order=order, bits=bits, out=out16 if out16 is not None else out32)


def maskpro_logp(n, m, pi, order):
    """log-likelihood of each block's ordered draw, f64 [B]."""
    pi = _f32(pi).reshape(-1, m)
    B = pi.shape[0]
    order = np.ascontiguousarray(order, dtype=np.uint8).reshape(B, n)
    out = np.zeros(B, dtype=np.float64)
    if lib().orc_mp_logp(n, m, B, _ptr(pi), _ptr(order), _ptr(out)) != 0:
        raise ValueError("oracle maskpro_logp: invalid arguments")
    return out


def maskpro_grad(n, m, pi, rows, cols, *, advantage, order=None, seed=0, step=0, tensor_id=0,
                 block_offset=0, flags=0, dpi_prev=None):
    """Policy gradient A * d(log p)/d(pi), f64 [B, M]; the draw is `order`
    ([B, N] positions) or, when None, the draw of maskpro_fwd with the same
    noise arguments.  dpi_prev: accumulate onto it."""
    B = rows * (cols // m)
    pi = _f32(pi).reshape(B, m)
    od = None if order is None else np.ascontiguousarray(order, dtype=np.uint8).reshape(B, n)
    prev = None if dpi_prev is None else _f32(dpi_prev).reshape(B, m)
    out = np.zeros((B, m), dtype=np.float64)
    rc = lib().orc_mp_grad(n, m, rows, cols, block_offset, tensor_id, seed, step, flags,
                           _ptr(pi), _ptr(od), float(advantage), _ptr(prev), _ptr(out))
    if rc != 0:
        raise ValueError("oracle maskpro_grad: invalid arguments")
    return out


def maskpro_init(n, m, rows, cols, *, c, prior_bits=None, w=None):
    """Initial logits: C at the initial mask's kept positions, 0 elsewhere;
    fp32 [B, M].  The mask is prior_bits (packed) or the magnitude top-N of w."""
    B = rows * (cols // m)
    pb = None if prior_bits is None else np.ascontiguousarray(prior_bits, dtype=np.uint8)
    ww = None if w is None else _f32(w)
    if pb is None and ww is None:
        raise ValueError("maskpro_init needs prior_bits or w")
    pi = np.zeros((B, m), dtype=np.float32)
    if lib().orc_mp_init(n, m, rows, cols, _ptr(pb), _ptr(ww), float(c), _ptr(pi)) != 0:
        raise ValueError("oracle maskpro_init: invalid arguments")
    return pi


def maskpro_baseline(residuals, *, mu, b0=0.0):
    """Advantages of a sequence of loss residuals under the moving-average
    baseline; returns (adv [T] f64, baseline after the last step)."""
    r = np.ascontiguousarray(residuals, dtype=np.float64)
    adv = np.zeros(len(r), dtype=np.float64)
    b = ctypes.c_double(float(b0))
    if lib().orc_mp_baseline(len(r), _ptr(r), float(mu), ctypes.addressof(b), _ptr(adv)) != 0:
        raise ValueError("oracle maskpro_baseline: invalid arguments")
    return adv, b.value
