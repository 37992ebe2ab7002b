"""GPU parity of the K-quant DMMV (GGML Q4_K / Q5_K / Q6_K super-blocks)
against the oracle: per-32-block integer sums bit-exact, rows within the bar
of the error scale S (Q4_K / Q5_K: sum_b |dx_b| (|d sc isum| + |dmin m s_b|);
Q6_K: sum_b |dx_b d isum_b|)."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_K, Q5_K, Q6_K = 12, 13, 14
KTYPES = (Q4_K, Q5_K, Q6_K)
NAME = {Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k"}


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def run(zq, wt, w, rows, k, qx, dx, sx, y=None, flags=0):
    y = nan_f32(rows) if y is None else y
    wd = w if not isinstance(w, np.ndarray) else dev(w)
    if wt == Q4_K:
        rc = zq.zq_dmmv_q4_k(wd, rows, k, qx, dx, sx, y, flags)
    elif wt == Q5_K:
        rc = zq.zq_dmmv_q5_k(wd, rows, k, qx, dx, sx, y, flags)
    else:
        rc = zq.zq_dmmv_q6_k(wd, rows, k, qx, dx, y, flags)
    assert rc == 0
    return y


def f16_bytes(v):
    return np.frombuffer(np.float16(v).astype("<f2").tobytes(), np.uint8)


# k = 256 .. 16384 take one pass of the lane layouts (64-element units:
# 4, 8, 32, 64, 80 = 16 x 5, 256 = 64 x 4); 20480 takes two passes.
SHAPES = [(1, 256), (7, 512), (33, 2048), (300, 4096), (130, 5120), (9, 16384), (5, 20480),
          (4099, 1024)]


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_k_isums_and_rows(zq, wt, rows, k):
    seed = 600 + 7 * wt + rows + k
    w = inputs.gen_weights_k(wt, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S, is_ref = oracle.k_dmmv(wt, w, rows, k, rq, rd, want_isums=True)
    isums = sentinel_i32(rows, k // 32)
    assert zq.zq_dmmv_isums(wt, dev(w), rows, k, qx, sx, isums) == 0
    assert np.array_equal(host(isums), is_ref)
    wd = dev(w)
    y = host(run(zq, wt, wd, rows, k, qx, dx, sx))
    check_rows(y, y_ref, S, "%s %d x %d" % (NAME[wt], rows, k))
    if wt != Q6_K:
        # without block sums the kernel sums the codes itself: same bits
        y2 = host(run(zq, wt, wd, rows, k, qx, dx, None))
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
def test_k_accumulate_and_determinism(zq, wt):
    rows, k = 2048, 4096
    w = inputs.gen_weights_k(wt, rows, k, 71 + wt)
    x = inputs.gen_activation(1, k, 72 + wt)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    prev = np.random.default_rng(3).standard_normal(rows).astype(np.float32)
    wd = dev(w)
    y = dev(prev)
    run(zq, wt, wd, rows, k, qx, dx, sx, y=y, flags=1)
    y_ref, S = oracle.k_dmmv(wt, w, rows, k, rq, rd, y_prev=prev)
    check_rows(host(y), y_ref, S, "%s accumulate" % NAME[wt])
    a = host(run(zq, wt, wd, rows, k, qx, dx, sx))
    b = host(run(zq, wt, wd, rows, k, qx, dx, sx))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def closed_form_superblock(wt):
    """A super-block whose every weight is the same number c:
    Q4_K: d 1, dmin 0.5, scale 1, min 2, code 3 -> 3 - 1 = 2;
    Q5_K: as Q4_K with every fifth bit set -> code 19 -> 19 - 1 = 18;
    Q6_K: d 0.5, scale -3, code 5 | 2 << 4 = 37 -> 0.5 * -3 * 5 = -7.5."""
    if wt in (Q4_K, Q5_K):
        sb = np.zeros(inputs.K_BLOCK_BYTES[wt], np.uint8)
        sb[0:2] = f16_bytes(1.0)
        sb[2:4] = f16_bytes(0.5)
        sb[4:8] = 1                     # sub-blocks 0-3: scale 1
        sb[8:12] = 2                    # sub-blocks 0-3: min 2
        sb[12:16] = 1 | (2 << 4)        # sub-blocks 4-7: scale 1, min 2 (top bits 0)
        if wt == Q4_K:
            sb[16:] = 0x33
            return sb, 2.0
        sb[16:48] = 0xFF                # every fifth bit
        sb[48:] = 0x33
        return sb, 18.0
    sb = np.zeros(210, np.uint8)
    sb[0:128] = 0x55                    # low 4 bits 5 in both nibbles
    sb[128:192] = 0xAA                  # top 2 bits 2 for every quarter
    sb[192:208] = np.uint8(0xFD)        # int8 scale -3
    sb[208:210] = f16_bytes(0.5)
    return sb, -7.5


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
def test_k_closed_form(zq, wt):
    """Every weight equals c, so every row is c * sum_b dx_b * s_b."""
    rows, k = 70, 1024
    sb, c = closed_form_superblock(wt)
    w = np.tile(sb, rows * (k // 256))
    x = inputs.gen_activation(1, k, 73)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, rs = oracle.quantize_act(x)
    expect = c * sum(float(rd[b]) * int(rs[b]) for b in range(k // 32))
    y = host(run(zq, wt, w, rows, k, qx, dx, sx))
    y_ref, S = oracle.k_dmmv(wt, w, rows, k, rq, rd)
    assert np.all(np.abs(y_ref - expect) <= 1e-12 * S)
    check_rows(y, y_ref, S, "%s closed form" % NAME[wt])
    assert np.all(y == y[0])


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
def test_k_empty_rows(zq, wt):
    y = nan_f32(4)
    w = inputs.gen_weights_k(wt, 1, 256, 1)
    qx, dx, sx = quantize_gpu(zq, inputs.gen_activation(1, 256, 2))
    run(zq, wt, w, 0, 256, qx, dx, sx, y=y)
    assert np.isnan(host(y)).all()


def test_q6k_last_superblock_of_buffer(zq):
    """Q6_K super-blocks are 2-byte aligned.  With an odd count the last one
    starts 4-byte aligned, the case whose dword windows end closest to the
    super-block's end, and here it ends the tensor."""
    torch = torch_cuda()
    rows, k = 3, 256                   # 3 super-blocks of 210 bytes: 630 bytes
    w = inputs.gen_weights_k(Q6_K, rows, k, 91)
    wd = torch.empty(w.size, dtype=torch.uint8, device="cuda")
    wd.copy_(torch.from_numpy(w))
    x = inputs.gen_activation(1, k, 92)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.k_dmmv(Q6_K, w, rows, k, rq, rd)
    check_rows(host(run(zq, Q6_K, wd, rows, k, qx, dx, None)), y_ref, S, "q6_k tail")


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
def test_k_full_size(zq, wt):
    """4096 x 4096 and the 5120 x 5120 prefill weight shape, every row."""
    for rows, k in ((4096, 4096), (5120, 5120)):
        w = inputs.gen_weights_k(wt, rows, k, 7000 + k + wt)
        x = inputs.gen_activation(1, k, 7001 + k)
        qx, dx, sx = quantize_gpu(zq, x)
        rq, rd, _ = oracle.quantize_act(x)
        y_ref, S = oracle.k_dmmv(wt, w, rows, k, rq, rd)
        check_rows(host(run(zq, wt, w, rows, k, qx, dx, sx)), y_ref, S,
                   "%s %d x %d" % (NAME[wt], rows, k))


def test_q6k_lmhead_sampled(zq):
    """The pages' LM-head format at its shape, 248 320 x 2048 Q6_K: every
    output written, sampled rows (first, last, and across the grid) checked
    against the oracle, and the isums of the last eight rows bit-exact."""
    rows, k = 248320, 2048
    w = inputs.gen_weights_k(Q6_K, rows, k, 7100)
    x = inputs.gen_activation(1, k, 7101)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    wd = dev(w)
    y = host(run(zq, Q6_K, wd, rows, k, qx, dx, None))
    assert not np.isnan(y).any()
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 4000)])).astype(np.int64)
    y_ref, S = oracle.k_dmmv(Q6_K, w, rows, k, rq, rd, rows_eval=idx)
    check_rows(y[idx], y_ref, S, "q6_k lm head sampled")
    tail = w[(rows - 8) * 8 * 210:]
    isums = sentinel_i32(8, k // 32)
    assert zq.zq_dmmv_isums(Q6_K, dev(tail), 8, k, qx, None, isums) == 0
    _, _, is_ref = oracle.k_dmmv(Q6_K, tail, 8, k, rq, rd, want_isums=True)
    assert np.array_equal(host(isums), is_ref)
