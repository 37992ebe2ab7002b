"""GPU parity of the RMS normalization fused with the activation
quantization and with the DMMV.

Chained like the SwiGLU stage: the GPU's fp32 xn is checked against the
oracle's fp64 normalization within XN_TOL (derived from the fp32 steps:
the sum of squares over at most ~80 sequential fused multiply-adds plus a
tree of depth <= 10, one division, one addition, a root, a reciprocal and
two products: |relative error| <= ~45 * 2^-24 < 3e-6); its quantization
must be bit-exact against the oracle's quantization of that same xn; the
DMMV rows are checked against the oracle's rows on those codes."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8
XN_TOL = 4e-6


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def norm_weight(k, seed):
    rng = np.random.default_rng(seed)
    return (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)


def check_xn(xn_gpu, x, w, eps, what):
    ref = oracle.rms_norm(x, w, eps)
    xn = np.asarray(xn_gpu, np.float64)
    assert not np.isnan(xn).any(), what
    err = np.abs(xn - ref)
    bad = err > XN_TOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements beyond %g relative, worst %g" % (
        what, int(bad.sum()), XN_TOL, float((err / np.maximum(np.abs(ref), 1e-300)).max()))


def check_codes(xn_gpu, qx, dx, sx, what):
    rq, rd, rs = oracle.quantize_act(np.asarray(xn_gpu, np.float32))
    assert np.array_equal(qx, rq), what
    assert np.array_equal(dx.view(np.uint32), rd.view(np.uint32)), what
    if sx is not None:
        assert np.array_equal(sx, rs), what


@pytest.mark.parametrize("n_tok,k,eps", [(1, 32, 1e-6), (1, 2048, 1e-6), (3, 4096, 0.25),
                                         (7, 5120, 1e-6), (2, 16384, 1e-5), (512, 5120, 1e-6),
                                         (5, 96, 0.0)])
def test_rms_norm_quantize(zq, n_tok, k, eps):
    torch = torch_cuda()
    x = inputs.gen_activation(n_tok, k, 500 + k + n_tok).reshape(n_tok, k)
    w = norm_weight(k, 501 + k)
    qx = torch.full((n_tok, k), 0x55, dtype=torch.int8, device="cuda")
    dx, sx, xn = nan_f32(n_tok, k // 32), sentinel_i32(n_tok, k // 32), nan_f32(n_tok, k)
    zq.zq_rms_norm_quantize(dev(x), dev(w), eps, n_tok, k, k, qx, dx, sx, xn)
    xn_h = host(xn)
    check_xn(xn_h, x, w, eps, "rms_norm %d x %d" % (n_tok, k))
    check_codes(xn_h, host(qx), host(dx), host(sx), "rms_norm codes %d x %d" % (n_tok, k))
    # without the optional outputs: the same codes and scales
    qx2 = torch.full((n_tok, k), 0x55, dtype=torch.int8, device="cuda")
    dx2 = nan_f32(n_tok, k // 32)
    zq.zq_rms_norm_quantize(dev(x), dev(w), eps, n_tok, k, k, qx2, dx2)
    assert np.array_equal(host(qx2), host(qx))
    assert np.array_equal(host(dx2).view(np.uint32), host(dx).view(np.uint32))


def test_rms_norm_quantize_stride_and_closed_form(zq):
    """A row stride beyond k; a constant token normalizes to sign * w
    (eps = 0), so its codes are those of w."""
    torch = torch_cuda()
    k, stride = 256, 320
    x = np.zeros((2, stride), np.float32)
    x[0, :k] = -0.75
    x[1, :k] = inputs.gen_activation(1, k, 7)
    x[:, k:] = np.nan                    # never read
    w = norm_weight(k, 8)
    qx = torch.zeros((2, k), dtype=torch.int8, device="cuda")
    dx, xn = nan_f32(2, k // 32), nan_f32(2, k)
    zq.zq_rms_norm_quantize(dev(x), dev(w), 0.0, 2, k, stride, qx, dx, None, xn)
    xn_h = host(xn)
    assert np.array_equal(xn_h[0], -w)
    check_xn(xn_h[1], x[1, :k], w, 0.0, "strided token")
    check_codes(xn_h, host(qx), host(dx), None, "strided codes")


@pytest.mark.parametrize("wt,rows,k", [(Q8_0, 64, 2048), (Q4_0, 4096, 4096), (Q4_0, 1000, 5120),
                                       (Q8_0, 300, 16384), (Q4_0, 33, 32)])
def test_rms_norm_dmmv_f32(zq, wt, rows, k):
    torch = torch_cuda()
    w = inputs.gen_weights(wt, rows, k, 600 + rows + k)
    x = inputs.gen_activation(1, k, 601 + k)
    nw = norm_weight(k, 602)
    eps = 1e-6
    y = nan_f32(rows)
    qx = torch.full((k,), 0x55, dtype=torch.int8, device="cuda")
    dx, sx, xn = nan_f32(k // 32), sentinel_i32(k // 32), nan_f32(k)
    zq.zq_rms_norm_dmmv_f32(wt, dev(w), rows, k, dev(x), dev(nw), eps, y, 0, qx, dx, sx, xn)
    xn_h = host(xn)
    check_xn(xn_h, x, nw, eps, "fused norm %d x %d" % (rows, k))
    check_codes(xn_h, host(qx), host(dx), host(sx), "fused codes")
    y_ref, S = oracle.dmmv(wt, w, rows, k, host(qx), host(dx))
    check_rows(host(y), y_ref, S, "norm dmmv %d x %d" % (rows, k))
    # accumulate, and without the optional outputs: the same bits
    y2 = dev(np.ones(rows, np.float32))
    zq.zq_rms_norm_dmmv_f32(wt, dev(w), rows, k, dev(x), dev(nw), eps, y2, 1)
    assert np.array_equal((host(y) + 1.0).view(np.uint32), host(y2).view(np.uint32))


def test_rms_norm_lmhead_argmax(zq):
    """The LM-head step with the final norm: same rows as the plain fused
    norm DMMV, bit for bit, and the argmax of those rows."""
    torch = torch_cuda()
    rows, k = 248320, 2048
    w = dev(inputs.gen_weights(Q4_0, rows, k, 3100))
    x = inputs.gen_activation(1, k, 3101)
    nw = norm_weight(k, 3102)
    eps = 1e-6
    ws_bytes = zq.zq_dmmv_f32_argmax_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y, idx = nan_f32(rows), sentinel_i32(1)
    zq.zq_rms_norm_dmmv_f32_argmax(Q4_0, w, rows, k, dev(x), dev(nw), eps, y, idx, ws, ws_bytes)
    y_plain, xn = nan_f32(rows), nan_f32(k)
    qx = torch.empty(k, dtype=torch.int8, device="cuda")
    dx = nan_f32(k // 32)
    zq.zq_rms_norm_dmmv_f32(Q4_0, w, rows, k, dev(x), dev(nw), eps, y_plain, 0, qx, dx, None, xn)
    yh = host(y)
    assert np.array_equal(yh.view(np.uint32), host(y_plain).view(np.uint32))
    assert int(host(idx)[0]) == int(np.argmax(yh))
    check_xn(host(xn), x, nw, eps, "lm head norm")
    check_codes(host(xn), host(qx), host(dx), None, "lm head codes")
    rng = np.random.default_rng(9)
    sel = np.unique(np.concatenate([[0, rows - 1, int(np.argmax(yh))],
                                    rng.integers(0, rows, 500)])).astype(np.int64)
    y_ref, S = oracle.dmmv(Q4_0, host(w), rows, k, host(qx), host(dx), rows_eval=sel)
    check_rows(yh[sel], y_ref, S, "lm head rows")
