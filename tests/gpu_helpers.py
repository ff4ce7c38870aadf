"""Helpers of the GPU parity tests: tolerance checks and oracle marshalling."""
import numpy as np

RTOL = 1e-5
ATOL = 1e-6


def to_np(t):
    """A torch tensor as numpy (bf16 as its uint16 bit pattern)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a):
    """uint16 bf16 bits -> fp32 values; fp32 passes through."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def assert_close(got, ref, what, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    diff = np.abs(got - ref)
    bad = diff > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside |d| <= {atol} + {rtol}|ref|; "
            f"first at {tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}; "
            f"max |d| {diff.max():.3g}")


def _ordered(u16):
    u = u16.astype(np.int64)
    return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)


def assert_bf16_ulp(got_u16, ref_u16, what, max_ulp=1):
    d = np.abs(_ordered(got_u16) - _ordered(ref_u16))
    if (d > max_ulp).any():
        i = np.argwhere(d > max_ulp)[0]
        raise AssertionError(f"{what}: {int((d > max_ulp).sum())} values beyond {max_ulp} bf16 "
                             f"ulp; first at {tuple(i)}: {got_u16[tuple(i)]:#06x} vs "
                             f"{ref_u16[tuple(i)]:#06x}")


def assert_out(got, ref, what):
    """Masked weight: bf16 within one ulp, fp32 within the fp32 tolerance."""
    if got.dtype == np.uint16:
        assert_bf16_ulp(got, ref, what)
    else:
        assert_close(got, ref, what)


def sample_rows(rows):
    """Every 61st row plus the first and the last."""
    return sorted(set(range(0, rows, 61)) | {rows - 1})


def check_rows(orc, n, m, spec, p, w, z, G, lam, y, out, dz, what):
    """The oracle on sampled rows of one tensor against the GPU's whole-tensor
    outputs: the soft index y (skipped when None: not saved), the masked
    weight and the logit gradient.  A row range is a tensor with a block
    offset, so the oracle draws the noise of the whole tensor."""
    import torch
    bpr = spec.cols // m
    rows = sample_rows(spec.rows)
    K = z.shape[1]
    sel = torch.tensor(rows, device=w.device)
    bsel = (sel[:, None] * bpr + torch.arange(bpr, device=w.device)[None, :]).reshape(-1)
    wn = to_np(w.index_select(0, sel))
    zn = to_np(z.index_select(0, bsel)).reshape(len(rows), bpr, K)
    Gn = to_np(G.index_select(0, sel))
    yg = None if y is None else to_np(y.index_select(0, bsel)).reshape(len(rows), bpr, K)
    og = to_np(out.index_select(0, sel))
    dg = to_np(dz.index_select(0, bsel)).reshape(len(rows), bpr, K)
    for i, r in enumerate(rows):
        kw = dict(kappa=p.kappa, tau=p.tau, seed=p.seed, step=p.step,
                  tensor_id=spec.tensor_id, block_offset=r * bpr)
        f = orc.fwd(n, m, widen(wn[i:i + 1]), zn[i], **kw)
        if yg is not None:
            assert_close(yg[i], f["y"], f"{what} row {r} y")
        assert_out(og[i:i + 1], f["out"], f"{what} row {r} out")
        d = orc.bwd(n, m, widen(wn[i:i + 1]), zn[i], widen(Gn[i:i + 1]), lam=lam, **kw)
        assert_close(dg[i], d, f"{what} row {r} dz")
