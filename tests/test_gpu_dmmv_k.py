"""GPU parity of the Q4_K DMMV (GGML K-quant super-blocks) against the
oracle: per-sub-block integer sums bit-exact, rows within the bar of the
sub-block error scale S = sum_b |dx_b| (|d sc isum| + |dmin m s_b|)."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_K = 12


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def run(zq, w, rows, k, qx, dx, sx, y=None, flags=0):
    y = nan_f32(rows) if y is None else y
    zq.zq_dmmv_q4_k(dev(w), rows, k, qx, dx, sx, y, flags)
    return y


# k = 256 .. 16384 take one pass of the lane layouts (64-element units:
# 4, 8, 32, 64, 80 = 16 x 5, 256 = 64 x 4); 20480 takes two passes.
@pytest.mark.parametrize("rows,k", [(1, 256), (7, 512), (33, 2048), (300, 4096), (130, 5120),
                                    (9, 16384), (5, 20480), (4099, 1024)])
def test_q4k_isums_and_rows(zq, rows, k):
    seed = 600 + rows + k
    w = inputs.gen_weights_k(Q4_K, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S, is_ref = oracle.k_dmmv(Q4_K, w, rows, k, rq, rd, want_isums=True)
    isums = sentinel_i32(rows, k // 32)
    zq.zq_dmmv_isums(Q4_K, dev(w), rows, k, qx, sx, isums)
    assert np.array_equal(host(isums), is_ref)
    check_rows(host(run(zq, w, rows, k, qx, dx, sx)), y_ref, S, "q4_k %d x %d" % (rows, k))
    # without block sums the kernel sums the codes itself: same rows, same bits
    y2 = host(run(zq, w, rows, k, qx, dx, None))
    assert np.array_equal(y2.view(np.uint32), host(run(zq, w, rows, k, qx, dx, sx)).view(np.uint32))


def test_q4k_accumulate_and_determinism(zq):
    rows, k = 2048, 4096
    w = inputs.gen_weights_k(Q4_K, rows, k, 71)
    x = inputs.gen_activation(1, k, 72)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    prev = np.random.default_rng(3).standard_normal(rows).astype(np.float32)
    y = dev(prev)
    run(zq, w, rows, k, qx, dx, sx, y=y, flags=1)
    y_ref, S = oracle.k_dmmv(Q4_K, w, rows, k, rq, rd, y_prev=prev)
    check_rows(host(y), y_ref, S, "q4_k accumulate")
    a = host(run(zq, w, rows, k, qx, dx, sx))
    b = host(run(zq, w, rows, k, qx, dx, sx))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_q4k_closed_form(zq):
    """Unit scales, min 2 at dmin 0.5, every code 3: each weight is 3 - 1 = 2,
    so every row is 2 * sum_b dx_b * s_b."""
    rows, k = 70, 1024
    sb = np.zeros(144, np.uint8)
    sb[0:2] = np.frombuffer(np.float16(1.0).astype("<f2").tobytes(), np.uint8)
    sb[2:4] = np.frombuffer(np.float16(0.5).astype("<f2").tobytes(), np.uint8)
    sb[4:8] = 1                     # sub-blocks 0-3: scale 1
    sb[8:12] = 2                    # sub-blocks 0-3: min 2
    sb[12:16] = 1 | (2 << 4)        # sub-blocks 4-7: scale 1, min 2 (top bits 0)
    sb[16:] = 0x33                  # every code 3
    w = np.tile(sb, rows * (k // 256))
    x = inputs.gen_activation(1, k, 73)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, rs = oracle.quantize_act(x)
    expect = 2.0 * sum(float(rd[b]) * int(rs[b]) for b in range(k // 32))
    y = host(run(zq, w, rows, k, qx, dx, sx))
    y_ref, S = oracle.k_dmmv(Q4_K, w, rows, k, rq, rd)
    assert np.all(np.abs(y_ref - expect) <= 1e-12 * S)
    check_rows(y, y_ref, S, "q4_k closed form")
    assert np.all(y == y[0])


def test_q4k_empty_rows(zq):
    y = nan_f32(4)
    w = inputs.gen_weights_k(Q4_K, 1, 256, 1)
    qx, dx, sx = quantize_gpu(zq, inputs.gen_activation(1, 256, 2))
    assert zq.zq_dmmv_q4_k(dev(w), 0, 256, qx, dx, sx, y, 0) == 0
    assert np.isnan(host(y)).all()


def test_q4k_full_size(zq):
    """4096 x 4096 and the 5120 x 5120 prefill weight shape, every row."""
    for rows, k in ((4096, 4096), (5120, 5120)):
        w = inputs.gen_weights_k(Q4_K, rows, k, 7000 + k)
        x = inputs.gen_activation(1, k, 7001 + k)
        qx, dx, sx = quantize_gpu(zq, x)
        rq, rd, _ = oracle.quantize_act(x)
        y_ref, S = oracle.k_dmmv(Q4_K, w, rows, k, rq, rd)
        check_rows(host(run(zq, w, rows, k, qx, dx, sx)), y_ref, S, "q4_k %d x %d" % (rows, k))
