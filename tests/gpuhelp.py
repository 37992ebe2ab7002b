"""Helpers for the GPU parity tests (imported by tests marked gpu only)."""
from __future__ import annotations

import numpy as np

TOL = 1e-4  # relative tolerance of fp32 row outputs against the fp64 reference


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def nan_f32(*shape):
    torch = torch_cuda()
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def sentinel_i32(*shape, value=-2**31):
    torch = torch_cuda()
    return torch.full(shape, value, dtype=torch.int32, device="cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def check_rows(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray, what: str, tol: float = TOL):
    """The parity bar for fp32 rows: no NaN left (every output written);
    normwise |y - y_ref| <= tol * S on every row; and elementwise
    |y - y_ref| <= tol * |y_ref| on every row with |y_ref| >= 0.1 * S."""
    y = np.asarray(y_gpu, np.float64).ravel()
    y_ref = np.asarray(y_ref, np.float64).ravel()
    S = np.asarray(S, np.float64).ravel()
    assert y.shape == y_ref.shape == S.shape, what
    assert not np.isnan(y).any(), "%s: %d outputs left unwritten (NaN sentinel)" % (
        what, int(np.isnan(y).sum()))
    err = np.abs(y - y_ref)
    bad = err > tol * S
    assert not bad.any(), "%s: %d rows beyond %g*S, worst %g*S at %d" % (
        what, int(bad.sum()), tol, float((err / np.maximum(S, 1e-300)).max()),
        int((err / np.maximum(S, 1e-300)).argmax()))
    well = np.abs(y_ref) >= 0.1 * S
    bad = well & (err > tol * np.abs(y_ref))
    assert not bad.any(), "%s: %d well-conditioned rows beyond %g relative" % (
        what, int(bad.sum()), tol)
    return float((err / np.maximum(S, 1e-300)).max())


def quantize_gpu(zq, x: np.ndarray, with_sx: bool = True):
    """Quantize on the GPU; returns device tensors (qx, dx, sx)."""
    torch = torch_cuda()
    x2 = np.atleast_2d(x).astype(np.float32)
    t, k = x2.shape
    xd = dev(x2)
    qx = torch.full((t, k), 0x55, dtype=torch.int8, device="cuda")
    dx = nan_f32(t, k // 32)
    sx = sentinel_i32(t, k // 32) if with_sx else None
    zq.zq_quantize_act(xd, t, k, k, qx, dx, sx)
    return qx, dx, sx
