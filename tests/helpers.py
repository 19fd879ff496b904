"""Shared helpers for the GPU parity tests: error metrics and tolerances.

Tolerances (the stated bar for this operation):
  float32 inputs:                max|err| / max|ref| <= 1e-4
  bfloat16 inputs, fp32 accum:   max|err| / max|ref| <= 2e-2  and  sum|err| / sum|ref| <= 2e-3
  key selection and ring slots:  bit-exact
The mean relative error is taken as sum|err| / sum|ref| over all compared elements (an
element-wise mean of |err|/|ref| is dominated by outputs near zero).
"""
import numpy as np
import torch

TOL_F32_MAX = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_SUM = 2e-3


def errors(got, ref):
    got = np.asarray(got.detach().cpu().to(torch.float64) if isinstance(got, torch.Tensor)
                     else got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - ref)
    max_rel = err.max() / max(np.abs(ref).max(), 1e-300)
    sum_rel = err.sum() / max(np.abs(ref).sum(), 1e-300)
    return float(max_rel), float(sum_rel)


def assert_parity(got, ref, in_dtype: str, label: str = ""):
    max_rel, sum_rel = errors(got, ref)
    if in_dtype == "f32":
        assert max_rel <= TOL_F32_MAX, "%s max_rel %.3e" % (label, max_rel)
    else:
        assert max_rel <= TOL_BF16_MAX, "%s max_rel %.3e" % (label, max_rel)
        assert sum_rel <= TOL_BF16_SUM, "%s sum_rel %.3e" % (label, sum_rel)
    return max_rel, sum_rel


def errors_blocked(got, ref, block: int = 4096):
    """errors() over a [B, N, ...] pair in blocks of rows along N, so that outputs of a
    whole long sequence are compared without float64 copies of the whole tensor. Returns
    (max|err| / max|ref|, sum|err| / sum|ref|) over every element."""
    ref = np.asarray(ref)
    assert tuple(got.shape) == ref.shape, (tuple(got.shape), ref.shape)
    emax = rmax = esum = rsum = 0.0
    for a in range(0, ref.shape[1], block):
        g = got[:, a:a + block].detach().to("cpu", torch.float64).numpy()
        r = ref[:, a:a + block].astype(np.float64, copy=False)
        assert np.all(np.isfinite(g)), "non-finite output in rows %d.." % a
        e = np.abs(g - r)
        emax = max(emax, float(e.max()))
        rmax = max(rmax, float(np.abs(r).max()))
        esum += float(e.sum())
        rsum += float(np.abs(r).sum())
    return emax / max(rmax, 1e-300), esum / max(rsum, 1e-300)


def misaligned(t):
    """The same values at a data pointer 4 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    off = 4 // t.element_size()
    out = flat[off:off + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 != 0
    return out
