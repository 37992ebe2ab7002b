"""GPU parity of the batched prefill GEMM (int8 matrix cores + per-block fp32
rescale) against the oracle: per-block integer sums bit-exact, entries within
1e-4, GEMM with one token equal to the DMMV."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4, Q8 = 4, 8


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def gemm(zq, wtype, wd, n, k, qx, dx, m, y=None, flags=0):
    y = nan_f32(m, n) if y is None else y
    zq.zq_gemm_prefill(wtype, wd, n, k, qx, dx, None, m, y, flags)
    return y


@pytest.mark.parametrize("wtype", [Q4, Q8])
@pytest.mark.parametrize("m,n,k", [(1, 64, 32), (64, 64, 128), (70, 100, 96), (130, 65, 5 * 32),
                                   (3, 200, 512), (128, 192, 2048)])
def test_gemm_small_full(zq, wtype, m, n, k):
    seed = m * 1000 + n + k + wtype
    w = inputs.gen_weights(wtype, n, k, seed)
    x = inputs.gen_activation(m, k, seed + 1).reshape(m, k)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    wd = dev(w)
    isums = sentinel_i32(m, n, k // 32)
    zq.zq_gemm_isums(wtype, wd, n, k, qx, None, m, 0, m, 0, n, isums)
    isums_h = host(isums)
    mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y_ref, S = oracle.gemm_entries(wtype, w, n, k, rq, rd, m, mi.ravel(), ni.ravel())
    for t in range(m):  # per-token isums against the oracle's DMMV sums
        _, _, ref_is = oracle.dmmv(wtype, w, n, k, rq[t], rd[t], want_isums=True)
        assert np.array_equal(isums_h[t], ref_is), t
    y = gemm(zq, wtype, wd, n, k, qx, dx, m)
    check_rows(host(y).ravel(), y_ref, S, "gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("wtype", [Q4, Q8])
def test_gemm_one_token_equals_dmmv(zq, wtype):
    n, k = 5120, 5120
    w = inputs.gen_weights(wtype, n, k, 41)
    x = inputs.gen_activation(1, k, 42)
    qx, dx, sx = quantize_gpu(zq, x)
    wd = dev(w)
    gi = sentinel_i32(1, n, k // 32)
    zq.zq_gemm_isums(wtype, wd, n, k, qx, None, 1, 0, 1, 0, n, gi)
    di = sentinel_i32(n, k // 32)
    zq.zq_dmmv_isums(wtype, wd, n, k, qx, sx, di)
    assert np.array_equal(host(gi)[0], host(di))
    yg = host(gemm(zq, wtype, wd, n, k, qx, dx, 1))[0]
    yd = nan_f32(n)
    if wtype == Q4:
        zq.zq_dmmv_q4_0(wd, n, k, qx, dx, sx, yd)
    else:
        zq.zq_dmmv_q8_0(wd, n, k, qx, dx, yd)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.dmmv(wtype, w, n, k, rq, rd)
    check_rows(yg, y_ref, S, "gemm m=1")
    check_rows(host(yd), y_ref, S, "dmmv k=5120")


def test_gemm_accumulate(zq):
    m, n, k = 64, 128, 256
    w = inputs.gen_weights(Q4, n, k, 51)
    x = inputs.gen_activation(m, k, 52).reshape(m, k)
    qx, dx, _ = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    prev = np.random.default_rng(53).standard_normal((m, n)).astype(np.float32)
    y = dev(prev.copy())
    gemm(zq, Q4, dev(w), n, k, qx, dx, m, y=y, flags=1)
    mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y_ref, S = oracle.gemm_entries(Q4, w, n, k, rq, rd, m, mi.ravel(), ni.ravel())
    y_ref = y_ref + prev.ravel().astype(np.float64)
    S = S + np.abs(prev.ravel().astype(np.float64))
    check_rows(host(y).ravel(), y_ref, S, "gemm accumulate")


@pytest.mark.parametrize("s", [0, 1])
def test_workload_prefill_full_sampled(zq, s):
    """M=512, N=5120, K=5120 in the launch configuration the bench times:
    the whole output is produced; sampled entries (all tiles' corners plus
    random ones) against the oracle, and one sub-range of isums exactly."""
    cfg = inputs.WORKLOADS[5]
    m, n, k = cfg["m"], cfg["n"], cfg["k"]
    w = inputs.gen_weights(Q4, n, k, inputs.seed_for(5, s))
    x = inputs.gen_activation(m, k, inputs.seed_for(5, s) + 1)
    qx, dx, _ = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    assert np.array_equal(host(qx), rq)
    wd = dev(w)
    y = host(gemm(zq, Q4, wd, n, k, qx, dx, m))
    assert not np.isnan(y).any()
    rng = np.random.default_rng(s)
    corners_m = np.concatenate([np.arange(0, m, 64), np.arange(63, m, 64)])
    corners_n = np.concatenate([np.arange(0, n, 64), np.arange(63, n, 64)])
    mi = np.concatenate([np.repeat(corners_m, 8), rng.integers(0, m, 1500)])
    ni = np.concatenate([rng.choice(corners_n, corners_m.size * 8), rng.integers(0, n, 1500)])
    y_ref, S = oracle.gemm_entries(Q4, w, n, k, rq, rd, m, mi, ni)
    check_rows(y[mi, ni], y_ref, S, "prefill sampled")
    m0, m1, n0, n1 = 448, 512, 5056, 5120
    isums = sentinel_i32(m1 - m0, n1 - n0, k // 32)
    zq.zq_gemm_isums(Q4, wd, n, k, qx, None, m, m0, m1, n0, n1, isums)
    ih = host(isums)
    for t in range(0, m1 - m0, 7):
        _, _, ref_is = oracle.dmmv(Q4, w, n, k, rq[m0 + t], rd[m0 + t],
                                   rows_eval=np.arange(n0, n1), want_isums=True)
        assert np.array_equal(ih[t], ref_is), t
