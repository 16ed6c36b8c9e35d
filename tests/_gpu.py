"""Helpers for the GPU parity tests (imported by tests only)."""
import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def f16_close(got, ref, rtol=2.0 ** -9, atol_frac=2.0 ** -10):
    """|g - r| <= rtol |r| + atol_frac * max|r| elementwise (fp16 outputs of
    fp32-accumulated kernels vs the fp64 oracle rounded once)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite output"
    scale = np.max(np.abs(r)) if r.size else 0.0
    err = np.abs(g - r)
    lim = rtol * np.abs(r) + atol_frac * scale + 1e-7
    bad = err > lim
    assert not bad.any(), (f"{bad.sum()} of {bad.size} elements off; worst {err.max():.3e} "
                           f"at {np.unravel_index(np.argmax(err - lim), err.shape)}; max|ref| {scale:.3e}")
