"""libmaskgs: MaskLLM's differentiable N:M mask path on AMD Instinct MI355X.

This package is a thin ctypes binding over the C ABI declared in
``include/maskgs.h`` (the HIP library ``libmaskgs.so`` built next to this file).
Every step of the path runs in the library's kernels; Python only marshals
arguments: it checks tensor device, dtype, shape and contiguity, takes device
pointers and torch's current HIP stream, and maps status codes to exceptions.
There is no CPU fallback: without the built library every call raises.

Entry points carry the C names (``maskgs_fwd`` ...).  Citations refer to the
summary page "MaskLLM: Learnable Semi-Structured Sparsity for Large Language
Models" (paper-graph-ui summary of arXiv 2409.17481); the ``maskpro_*`` entry
points (``include/maskpro.h``) follow the summary page "MaskPro: Linear-Space
Probabilistic Learning for Strict (N:M)-Sparsity on LLMs" (atlas.scime.ai).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmaskgs.so")

MASKGS_OK = 0
MASKGS_E_NULL = 1
MASKGS_E_SHAPE = 2
MASKGS_E_UNSUPPORTED = 3
MASKGS_E_DTYPE = 4
MASKGS_E_ALIGN = 5
MASKGS_E_RANGE = 6
MASKGS_E_HIP = 7
MASKGS_E_CAPACITY = 8
MASKGS_F32 = 0
MASKGS_BF16 = 1
MASKGS_NO_NOISE = 1
MASKGS_HARD_SAMPLE = 2

EXPORTS = ("maskgs_abi_version", "maskgs_status_str", "maskgs_candidates", "maskgs_fwd",
           "maskgs_fwd_hard",
           "maskgs_bwd", "maskgs_bwd_adamw", "maskgs_mask_stats", "maskgs_reg_reduce", "maskgs_hard_extract", "maskgs_prior_init",
           "maskgs_debug_philox", "maskgs_debug_gumbel",
           "maskpro_fwd", "maskpro_bwd", "maskpro_init", "maskpro_baseline")


class MaskgsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class TensorDesc(ctypes.Structure):
    """maskgs_tensor_desc: N:M, weight shape, global block offset, tensor id."""
    _fields_ = [("n", ctypes.c_int32), ("m", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("block_offset", ctypes.c_uint64),
                ("tensor_id", ctypes.c_uint32)]


class SampleParams(ctypes.Structure):
    """maskgs_sample_params: Philox seed and step, kappa, tau, flags."""
    _fields_ = [("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("kappa", ctypes.c_float),
                ("tau", ctypes.c_float), ("flags", ctypes.c_uint32)]


class AdamWParams(ctypes.Structure):
    """maskgs_adamw_params: lr, beta1, beta2, eps, weight decay, update count t."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("t", ctypes.c_uint32)]


class DrawParams(ctypes.Structure):
    """maskpro_draw_params: Philox seed and step, flags."""
    _fields_ = [("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmaskgs.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmaskgs is not built ({path} missing); run "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    c = ctypes
    P = c.c_void_p
    DP = c.POINTER(TensorDesc)
    SP = c.POINTER(SampleParams)
    L.maskgs_abi_version.restype = c.c_int
    L.maskgs_status_str.argtypes = [c.c_int]
    L.maskgs_status_str.restype = c.c_char_p
    L.maskgs_candidates.argtypes = [c.c_int32, c.c_int32, P, c.c_int32, c.POINTER(c.c_int32)]
    L.maskgs_fwd.argtypes = [DP, SP, P, c.c_int, P, P, c.c_int, P, P, P]
    L.maskgs_fwd_hard.argtypes = [DP, SP, P, c.c_int, P, P, c.c_int, P, P, P, P, P, P, P]
    L.maskgs_bwd.argtypes = [DP, SP, P, c.c_int, P, P, P, c.c_int, c.c_float, P, c.c_int32, P]
    L.maskgs_bwd_adamw.argtypes = [DP, SP, P, c.c_int, P, P, P, c.c_int, c.c_float, P, P,
                                   c.POINTER(AdamWParams), P]
    L.maskgs_mask_stats.argtypes = [DP, P, c.c_float, c.POINTER(SampleParams), P, P, c.c_int, P,
                                    P, P]
    L.maskgs_reg_reduce.argtypes = [DP, SP, P, c.c_int, P, P, P, P]
    L.maskgs_hard_extract.argtypes = [DP, P, P, c.c_int, P, P, P, P, P]
    L.maskgs_prior_init.argtypes = [DP, P, P, P, c.c_int, c.c_float, c.c_int32, P]
    L.maskgs_debug_philox.argtypes = [c.c_uint64, c.c_uint32, c.c_uint32, c.c_uint64, c.c_int64,
                                      P, P]
    L.maskgs_debug_gumbel.argtypes = [P, c.c_int64, P, P]
    L.maskpro_fwd.argtypes = [DP, c.POINTER(DrawParams), P, c.c_int, P, P, c.c_int, P, P, P]
    L.maskpro_bwd.argtypes = [DP, c.POINTER(DrawParams), P, P, c.c_float, P, c.c_int32, P]
    L.maskpro_init.argtypes = [DP, P, P, c.c_int, c.c_float, P, P]
    L.maskpro_baseline.argtypes = [c.c_double, c.c_double, c.POINTER(c.c_double),
                                   c.POINTER(c.c_double)]
    for name in EXPORTS:
        if name not in ("maskgs_status_str",):
            getattr(L, name).restype = c.c_int
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != MASKGS_OK:
        msg = load_library().maskgs_status_str(status).decode()
        raise MaskgsError(fn, status, msg)


# --------------------------------------------------------------------------
# Argument marshalling
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MASKGS_F32
    if t.dtype == torch.bfloat16:
        return MASKGS_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t, name, dtype=None, numel=None, device=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def num_candidates(n: int, m: int) -> int:
    return {(2, 4): 6, (4, 8): 70}[(n, m)]


@dataclass
class Tensor:
    """Shape bookkeeping for one masked weight (or a row range of one)."""
    n: int
    m: int
    rows: int
    cols: int
    block_offset: int = 0
    tensor_id: int = 0

    @property
    def k(self) -> int:
        return num_candidates(self.n, self.m)

    @property
    def nblocks(self) -> int:
        return self.rows * (self.cols // self.m)

    def desc(self) -> TensorDesc:
        return TensorDesc(self.n, self.m, self.rows, self.cols, self.block_offset, self.tensor_id)


def sample_params(seed=0, step=0, kappa=100.0, tau=4.0, flags=0) -> SampleParams:
    return SampleParams(seed, step, kappa, tau, flags)


# --------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def maskgs_abi_version() -> int:
    return load_library().maskgs_abi_version()


def maskgs_candidates(n: int, m: int) -> list:
    """Candidate masks S as bitmasks (section 3.2; section 3.4 Eq. 7)."""
    buf = (ctypes.c_uint8 * 128)()
    k = ctypes.c_int32(0)
    _check("maskgs_candidates",
           load_library().maskgs_candidates(n, m, buf, 128, ctypes.byref(k)))
    return list(buf[: k.value])


def maskgs_fwd(t: Tensor, p: SampleParams, w, z, out, y_save=None, reg_accum=None, stream=None):
    """W (.) M~ (section 3.4, Eqs. 5-7); optional soft index and regulariser."""
    dev = w.device
    _check("maskgs_fwd", load_library().maskgs_fwd(
        ctypes.byref(t.desc()), ctypes.byref(p),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), _dtype_code(w),
        _ptr(z, "z", _torch().float32, t.nblocks * t.k, dev),
        _ptr(out, "out", numel=t.rows * t.cols, device=dev), _dtype_code(out),
        _ptr(y_save, "y_save", _torch().float32, t.nblocks * t.k, dev),
        _ptr(reg_accum, "reg_accum", _torch().float64, 1, dev), _stream(stream)))
    return out


def maskgs_fwd_hard(t: Tensor, p: SampleParams, w, z, out, y_save=None, reg_accum=None,
                    idx=None, mask_bits=None, values=None, val_idx=None, stream=None):
    """maskgs_fwd plus the hard mask of the same logits (z read once)."""
    torch = _torch()
    dev = w.device
    B = t.nblocks
    _check("maskgs_fwd_hard", load_library().maskgs_fwd_hard(
        ctypes.byref(t.desc()), ctypes.byref(p),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), _dtype_code(w),
        _ptr(z, "z", torch.float32, B * t.k, dev),
        _ptr(out, "out", numel=t.rows * t.cols, device=dev), _dtype_code(out),
        _ptr(y_save, "y_save", torch.float32, B * t.k, dev),
        _ptr(reg_accum, "reg_accum", torch.float64, 1, dev),
        _ptr(idx, "idx", torch.uint8, B, dev),
        _ptr(mask_bits, "mask_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(values, "values", w.dtype, B * t.n, dev),
        _ptr(val_idx, "val_idx", torch.uint8, (B + 1) // 2, dev), _stream(stream)))
    return out


def maskgs_bwd(t: Tensor, p: SampleParams, w, z, y_saved, dout, lam: float, dz,
               accumulate: bool = False, stream=None):
    """dL/dz for L = L_LM - lambda*R (section 3.4 Eq. 8, softmax backward)."""
    dev = w.device
    f32 = _torch().float32
    _check("maskgs_bwd", load_library().maskgs_bwd(
        ctypes.byref(t.desc()), ctypes.byref(p),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), _dtype_code(w),
        _ptr(z, "z", f32, t.nblocks * t.k, dev),
        _ptr(y_saved, "y_saved", f32, t.nblocks * t.k, dev),
        _ptr(dout, "dout", numel=t.rows * t.cols, device=dev), _dtype_code(dout),
        float(lam), _ptr(dz, "dz", f32, t.nblocks * t.k, dev), int(bool(accumulate)),
        _stream(stream)))
    return dz


def maskgs_bwd_adamw(t: Tensor, p: SampleParams, w, z, y_saved, dout, lam: float, exp_avg,
                     exp_avg_sq, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.1, step_t: int = 1,
                     stream=None):
    """Backward to the logits fused with their AdamW update (section 3.4,
    Algorithm 1): z, exp_avg and exp_avg_sq are updated in place."""
    dev = w.device
    f32 = _torch().float32
    opt = AdamWParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                      int(step_t))
    _check("maskgs_bwd_adamw", load_library().maskgs_bwd_adamw(
        ctypes.byref(t.desc()), ctypes.byref(p),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), _dtype_code(w),
        _ptr(z, "z", f32, t.nblocks * t.k, dev),
        _ptr(y_saved, "y_saved", f32, t.nblocks * t.k, dev),
        _ptr(dout, "dout", numel=t.rows * t.cols, device=dev), _dtype_code(dout),
        float(lam), _ptr(exp_avg, "exp_avg", f32, t.nblocks * t.k, dev),
        _ptr(exp_avg_sq, "exp_avg_sq", f32, t.nblocks * t.k, dev), ctypes.byref(opt),
        _stream(stream)))
    return z


STATS_FIELDS = ("blocks", "changed", "max_prob", "kept_l1", "magnitude_l1", "grad_sq")


def new_stats(device):
    """A zeroed device maskgs_stats (48 bytes) for maskgs_mask_stats."""
    return _torch().zeros(6, dtype=_torch().int64, device=device)


def read_stats(stats) -> dict:
    """The maskgs_stats fields of a device buffer from new_stats()."""
    host = stats.detach().cpu()
    f = host[2:].view(_torch().float64)
    return dict(blocks=int(host[0]), changed=int(host[1]), max_prob=float(f[0]),
                kept_l1=float(f[1]), magnitude_l1=float(f[2]), grad_sq=float(f[3]))


def maskgs_mask_stats(t: Tensor, z, kappa: float, stats, sample: SampleParams = None,
                      ref_bits=None, w=None, dz=None, stream=None):
    """Adds one tensor's training diagnostics (mask change, maximum probability,
    kept-weight norm vs magnitude, gradient norm; section 3.4 Figure 5, Figures
    6 and 8, Table 14) to `stats` (from new_stats)."""
    torch = _torch()
    dev = z.device
    B = t.nblocks
    w_dt = _dtype_code(w) if w is not None else MASKGS_BF16
    _check("maskgs_mask_stats", load_library().maskgs_mask_stats(
        ctypes.byref(t.desc()), _ptr(z, "z", torch.float32, B * t.k, dev), float(kappa),
        None if sample is None else ctypes.byref(sample),
        _ptr(ref_bits, "ref_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), w_dt,
        _ptr(dz, "dz", torch.float32, B * t.k, dev),
        _ptr(stats, "stats", torch.int64, 6, dev), _stream(stream)))
    return stats


def maskgs_reg_reduce(t: Tensor, p: SampleParams, w, z, y_saved, reg_accum, stream=None):
    """Adds R = sum ||W (.) M~||^2 (Eq. 8) to reg_accum (float64, 1 element)."""
    dev = w.device
    f32 = _torch().float32
    _check("maskgs_reg_reduce", load_library().maskgs_reg_reduce(
        ctypes.byref(t.desc()), ctypes.byref(p),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), _dtype_code(w),
        _ptr(z, "z", f32, t.nblocks * t.k, dev),
        _ptr(y_saved, "y_saved", f32, t.nblocks * t.k, dev),
        _ptr(reg_accum, "reg_accum", _torch().float64, 1, dev), _stream(stream)))
    return reg_accum


def maskgs_hard_extract(t: Tensor, z, w=None, idx=None, mask_bits=None, values=None,
                        val_idx=None, stream=None):
    """argmax(z) per block, packed mask bits, 2:4 values and 2-bit indices."""
    torch = _torch()
    dev = z.device
    B = t.nblocks
    w_dt = _dtype_code(w) if w is not None else MASKGS_BF16
    _check("maskgs_hard_extract", load_library().maskgs_hard_extract(
        ctypes.byref(t.desc()), _ptr(z, "z", torch.float32, B * t.k, dev),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), w_dt,
        _ptr(idx, "idx", torch.uint8, B, dev),
        _ptr(mask_bits, "mask_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(values, "values", None if w is None else w.dtype, B * t.n, dev),
        _ptr(val_idx, "val_idx", torch.uint8, (B + 1) // 2, dev), _stream(stream)))


def maskgs_prior_init(t: Tensor, z, alpha: float, mode: int = 0, prior_bits=None, w=None,
                      stream=None):
    """Eq. 9-10 prior seeding of z in place (prior bits or magnitude top-N of w)."""
    torch = _torch()
    dev = z.device
    B = t.nblocks
    w_dt = _dtype_code(w) if w is not None else MASKGS_BF16
    _check("maskgs_prior_init", load_library().maskgs_prior_init(
        ctypes.byref(t.desc()), _ptr(z, "z", torch.float32, B * t.k, dev),
        _ptr(prior_bits, "prior_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), w_dt, float(alpha), int(mode),
        _stream(stream)))
    return z


def maskgs_debug_philox(seed: int, step: int, tensor_id: int, n0: int, words, stream=None):
    torch = _torch()
    _check("maskgs_debug_philox", load_library().maskgs_debug_philox(
        seed, step, tensor_id, n0, words.numel(), _ptr(words, "words", torch.int32),
        _stream(stream)))
    return words


def maskgs_debug_gumbel(words, g, stream=None):
    torch = _torch()
    _check("maskgs_debug_gumbel", load_library().maskgs_debug_gumbel(
        _ptr(words, "words", torch.int32), words.numel(),
        _ptr(g, "g", torch.float32, words.numel()), _stream(stream)))
    return g


# --------------------------------------------------------------------------
# autograd pairing of maskgs_fwd / maskgs_bwd
# --------------------------------------------------------------------------
def _masked_weight_function():
    torch = _torch()

    class MaskedWeight(torch.autograd.Function):
        """W (.) M~ as a differentiable function of the logits z (MaskLLM
        summary, section 3.4, Eqs. 5-8): the forward is maskgs_fwd, the
        backward maskgs_bwd.  W is frozen (no gradient).  The backward adds the
        regulariser term of -lambda * R to dz itself, so R is returned as a
        non-differentiable side output (for logging) and must not also enter
        the loss."""

        @staticmethod
        def forward(ctx, z, w, t, p, lam, save_y, out_dtype):
            out = torch.empty(w.shape, dtype=out_dtype, device=w.device)
            y = torch.empty_like(z) if save_y else None
            reg = torch.zeros(1, dtype=torch.float64, device=w.device)
            maskgs_fwd(t, p, w, z, out, y, reg)
            ctx.save_for_backward(w, None if save_y else z, y)
            ctx.t = t
            ctx.p = SampleParams(p.seed, p.step, p.kappa, p.tau, p.flags)
            ctx.lam = float(lam)
            ctx.mark_non_differentiable(reg)
            return out, reg

        @staticmethod
        def backward(ctx, dout, _dreg):
            w, z, y = ctx.saved_tensors
            dz = torch.empty_like(y if y is not None else z)
            maskgs_bwd(ctx.t, ctx.p, w, z, y, dout.contiguous(), ctx.lam, dz)
            return dz, None, None, None, None, None, None

    return MaskedWeight


_MaskedWeight = None


def masked_weight(z, w, t: Tensor, p: SampleParams, lam: float = 0.0, save_y: bool = True,
                  out_dtype=None):
    """(W (.) M~, R) with autograd to z; see _masked_weight_function.

    save_y keeps the soft index for the backward; under MASKGS_HARD_SAMPLE the
    backward must recompute it from z (it needs the sample's argmax, which a
    saved fp32 soft index does not determine), so the soft index is then never
    saved, whatever save_y says."""
    global _MaskedWeight
    torch = _torch()
    if _MaskedWeight is None:
        _MaskedWeight = _masked_weight_function()
    if p.flags & MASKGS_HARD_SAMPLE:
        save_y = False
    return _MaskedWeight.apply(z, w, t, p, lam, save_y,
                               torch.bfloat16 if out_dtype is None else out_dtype)


# --------------------------------------------------------------------------
# Linear-space mask learner (include/maskpro.h; MaskPro summary page,
# "Approach" and "Limitations")
# --------------------------------------------------------------------------
def draw_params(seed=0, step=0, flags=0) -> DrawParams:
    return DrawParams(seed, step, flags)


def _order_dtypes(m):
    torch = _torch()
    if m == 4:
        return torch.uint8
    return tuple(d for d in (torch.int16, getattr(torch, "uint16", None)) if d is not None)


def maskpro_fwd(t: Tensor, p: DrawParams, pi, w=None, out=None, mask_bits=None, order=None,
                stream=None):
    """Ordered draw of N of M positions per block (Gumbel-top-k on pi + g) and
    the hard-masked weights; pi fp32 [B, M]; order: uint8 [B] (2:4) or
    int16/uint16 [B] (4:8)."""
    torch = _torch()
    dev = pi.device
    B = t.nblocks
    w_dt = _dtype_code(w) if w is not None else MASKGS_BF16
    o_dt = _dtype_code(out) if out is not None else MASKGS_BF16
    _check("maskpro_fwd", load_library().maskpro_fwd(
        ctypes.byref(t.desc()), ctypes.byref(p), _ptr(w, "w", numel=t.rows * t.cols, device=dev),
        w_dt, _ptr(pi, "pi", torch.float32, B * t.m, dev),
        _ptr(out, "out", numel=t.rows * t.cols, device=dev), o_dt,
        _ptr(mask_bits, "mask_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(order, "order", _order_dtypes(t.m), B, dev), _stream(stream)))
    return out


def maskpro_bwd(t: Tensor, p: DrawParams, pi, advantage: float, dpi, order=None,
                accumulate=False, stream=None):
    """Policy gradient advantage * dlogp(draw)/dpi into dpi fp32 [B, M]; the draw
    is `order` (maskpro_fwd's) or drawn again from pi and p."""
    torch = _torch()
    dev = pi.device
    B = t.nblocks
    _check("maskpro_bwd", load_library().maskpro_bwd(
        ctypes.byref(t.desc()), ctypes.byref(p), _ptr(pi, "pi", torch.float32, B * t.m, dev),
        _ptr(order, "order", _order_dtypes(t.m), B, dev), float(advantage),
        _ptr(dpi, "dpi", torch.float32, B * t.m, dev), 1 if accumulate else 0, _stream(stream)))
    return dpi


def maskpro_init(t: Tensor, pi, c: float, prior_bits=None, w=None, stream=None):
    """Initial logits: c at the initial mask's kept positions, 0 elsewhere."""
    torch = _torch()
    dev = pi.device
    B = t.nblocks
    w_dt = _dtype_code(w) if w is not None else MASKGS_BF16
    _check("maskpro_init", load_library().maskpro_init(
        ctypes.byref(t.desc()),
        _ptr(prior_bits, "prior_bits", torch.uint8, (B * t.m + 7) // 8, dev),
        _ptr(w, "w", numel=t.rows * t.cols, device=dev), w_dt, float(c),
        _ptr(pi, "pi", torch.float32, B * t.m, dev), _stream(stream)))
    return pi


class Baseline:
    """Moving-average baseline of the loss residual (host scalars, computed by
    the library's maskpro_baseline)."""

    def __init__(self, mu: float, value: float = 0.0):
        self.mu = float(mu)
        self.value = float(value)

    def step(self, residual: float) -> float:
        return maskpro_baseline(self, residual)


def maskpro_baseline(state: Baseline, residual: float) -> float:
    """Returns the advantage residual - baseline, then moves the baseline."""
    b = ctypes.c_double(state.value)
    adv = ctypes.c_double(0.0)
    _check("maskpro_baseline", load_library().maskpro_baseline(
        float(residual), state.mu, ctypes.byref(b), ctypes.byref(adv)))
    state.value = b.value
    return adv.value
