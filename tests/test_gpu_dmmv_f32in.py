"""GPU parity of the fp32-input forms of the K-quant and multi-token DMMV:
zq_dmmv_k_f32 (the activation quantized inside the product's launch) and
zq_dmmv_tokens_f32 (the quantizer's launch, then the product).

For each: the quantized activation they store is bit-exact against
oracle.quantize_act; the rows equal, bit for bit, those of the two-launch
path (zq_quantize_act, then zq_dmmv_q4_k / q5_k / q6_k or zq_dmmv_tokens),
whose kernels use the same lane layout and summation order; and the rows
are within the bar of the oracle's (oracle.k_dmmv / oracle.dmmv on the
oracle's codes)."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8
Q4_K, Q5_K, Q6_K = 12, 13, 14
KTYPES = (Q4_K, Q5_K, Q6_K)
NAME = {Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k", Q4_0: "q4_0", Q8_0: "q8_0"}


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def two_launch_k(zq, wt, wd, rows, k, x):
    qx, dx, sx = quantize_gpu(zq, x)
    y = nan_f32(rows)
    if wt == Q4_K:
        rc = zq.zq_dmmv_q4_k(wd, rows, k, qx, dx, sx, y)
    elif wt == Q5_K:
        rc = zq.zq_dmmv_q5_k(wd, rows, k, qx, dx, sx, y)
    else:
        rc = zq.zq_dmmv_q6_k(wd, rows, k, qx, dx, y)
    assert rc == 0
    return host(y)


def check_codes(qx, dx, sx, x, what):
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(qx).reshape(rq.shape), rq), what + " codes"
    assert np.array_equal(host(dx).reshape(rd.shape).view(np.uint32),
                          np.asarray(rd, np.float32).view(np.uint32)), what + " scales"
    assert np.array_equal(host(sx).reshape(rs.shape), rs), what + " sums"


# one pass of every lane layout (k = 256 .. 16384), ragged and single rows,
# the decode shape and both workgroup sizes (2048 x 2048 takes 4 waves per
# workgroup, 4096 x 4096 and 8193 x 4096 take 8, the latter with a ragged
# last row group)
K_SHAPES = [(1, 256), (7, 512), (33, 2048), (300, 4096), (130, 5120), (9, 16384), (4099, 1024),
            (4096, 4096), (2048, 2048), (8193, 4096)]


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
@pytest.mark.parametrize("rows,k", K_SHAPES)
def test_k_f32(zq, wt, rows, k):
    torch = torch_cuda()
    seed = 6100 + 7 * wt + rows + k
    w = inputs.gen_weights_k(wt, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    wd = dev(w)
    qx = torch.zeros(k, dtype=torch.int8, device="cuda")
    dx = nan_f32(k // 32)
    sx = sentinel_i32(k // 32)
    y = nan_f32(rows)
    assert zq.zq_dmmv_k_f32(wt, wd, rows, k, dev(x), y, 0, qx, dx, sx) == 0
    torch.cuda.synchronize()
    what = "%s %d x %d" % (NAME[wt], rows, k)
    check_codes(qx, dx, sx, x, what)
    yh = host(y)
    assert np.array_equal(yh.view(np.uint32), two_launch_k(zq, wt, wd, rows, k, x).view(np.uint32)), \
        what + " against the two-launch path"
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.k_dmmv(wt, w, rows, k, rq, rd)
    check_rows(yh, y_ref, S, what)


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
@pytest.mark.parametrize("rows", [248320, 200003])
def test_k_f32_walking_groups(zq, wt, rows):
    """Row counts past the capped grid (the LM head's 248 320 and a ragged
    200 003 at k = 2048), where every wave walks several row groups with the
    next group's units requested before the current one's arithmetic: every
    row bit-identical to the two-launch path, sampled rows (both ends and
    across the grid) against the oracle."""
    torch = torch_cuda()
    k = 2048
    seed = 6300 + wt + rows
    w = inputs.gen_weights_k(wt, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    wd = dev(w)
    y = nan_f32(rows)
    assert zq.zq_dmmv_k_f32(wt, wd, rows, k, dev(x), y, 0) == 0
    torch.cuda.synchronize()
    yh = host(y)
    what = "%s %d x %d" % (NAME[wt], rows, k)
    assert np.array_equal(yh.view(np.uint32), two_launch_k(zq, wt, wd, rows, k, x).view(np.uint32)), \
        what + " against the two-launch path"
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 1500)])).astype(np.int64)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.k_dmmv(wt, w, rows, k, rq, rd, rows_eval=idx)
    check_rows(yh[idx], y_ref, S, what + " sampled")


@pytest.mark.parametrize("wt", KTYPES, ids=lambda t: NAME[t])
def test_k_f32_accumulate_without_outputs(zq, wt):
    torch = torch_cuda()
    rows, k = 1000, 2048
    w = inputs.gen_weights_k(wt, rows, k, 6200 + wt)
    x = inputs.gen_activation(1, k, 6201 + wt)
    prev = np.random.default_rng(6202).standard_normal(rows).astype(np.float32)
    wd = dev(w)
    y = dev(prev)
    assert zq.zq_dmmv_k_f32(wt, wd, rows, k, dev(x), y, 1) == 0
    torch.cuda.synchronize()
    plain = two_launch_k(zq, wt, wd, rows, k, x)
    assert np.array_equal(host(y).view(np.uint32), (prev + plain).view(np.uint32))


def two_launch_tok(zq, wt, wd, rows, k, x, n_tok):
    qx, dx, sx = quantize_gpu(zq, x.reshape(n_tok, k))
    y = nan_f32(n_tok, rows)
    assert zq.zq_dmmv_tokens(wt, wd, rows, k, qx, dx, sx, n_tok, y) == 0
    return host(y)


# The tile form (5..8 tokens, 64..128 blocks, < 65 536 rows, >= 8 M weights;
# a ragged last row tile at 2100 and 4100 rows) and the vector form (3
# tokens, short matrices).
TOK_SHAPES = [
    (Q4_0, 4096, 4096, 8), (Q4_0, 4096, 4096, 5), (Q8_0, 2048, 4096, 8), (Q4_0, 2100, 4096, 6),
    (Q8_0, 4100, 2048, 7), (Q4_0, 4096, 4096, 3), (Q8_0, 300, 1024, 8), (Q4_0, 33, 512, 2),
]


@pytest.mark.parametrize("wt,rows,k,n_tok", TOK_SHAPES)
def test_tokens_f32(zq, wt, rows, k, n_tok):
    torch = torch_cuda()
    seed = 6300 + rows + k + n_tok + wt
    w = inputs.gen_weights(wt, rows, k, seed)
    x = inputs.gen_activation(n_tok, k, seed + 1).reshape(n_tok, k)
    wd = dev(w)
    qx = torch.zeros((n_tok, k), dtype=torch.int8, device="cuda")
    dx = nan_f32(n_tok, k // 32)
    sx = sentinel_i32(n_tok, k // 32)
    y = nan_f32(n_tok, rows)
    assert zq.zq_dmmv_tokens_f32(wt, wd, rows, k, dev(x), n_tok, qx, dx, sx, y) == 0
    torch.cuda.synchronize()
    what = "%s %d x %d, %d tokens" % (NAME[wt], rows, k, n_tok)
    check_codes(qx, dx, sx, x, what)
    yh = host(y)
    assert np.array_equal(yh.view(np.uint32),
                          two_launch_tok(zq, wt, wd, rows, k, x, n_tok).view(np.uint32)), \
        what + " against the two-launch path"
    rq, rd, _ = oracle.quantize_act(x)
    # every row of every token for the small shapes; a sample of rows (both
    # ends and a seeded spread) for the large ones
    if rows * k <= (1 << 21):
        rows_eval = None
    else:
        rng = np.random.default_rng(seed)
        rows_eval = np.unique(np.concatenate([np.arange(16), np.arange(rows - 16, rows),
                                              rng.integers(0, rows, 96)]))
    for t in range(n_tok):
        if rows_eval is None:
            y_ref, S = oracle.dmmv(wt, w, rows, k, rq[t], rd[t])
            check_rows(yh[t], y_ref, S, what + " token %d" % t)
        else:
            y_ref, S = oracle.dmmv(wt, w, rows, k, rq[t], rd[t], rows_eval=rows_eval)
            check_rows(yh[t][rows_eval], y_ref, S, what + " token %d (sampled rows)" % t)


def test_tokens_f32_accumulate(zq):
    torch = torch_cuda()
    wt, rows, k, n_tok = Q4_0, 4096, 4096, 8
    w = inputs.gen_weights(wt, rows, k, 6400)
    x = inputs.gen_activation(n_tok, k, 6401).reshape(n_tok, k)
    prev = np.random.default_rng(6402).standard_normal((n_tok, rows)).astype(np.float32)
    wd = dev(w)
    qx = torch.zeros((n_tok, k), dtype=torch.int8, device="cuda")
    dx = nan_f32(n_tok, k // 32)
    sx = sentinel_i32(n_tok, k // 32)
    y = dev(prev)
    assert zq.zq_dmmv_tokens_f32(wt, wd, rows, k, dev(x), n_tok, qx, dx, sx, y, 1) == 0
    torch.cuda.synchronize()
    plain = two_launch_tok(zq, wt, wd, rows, k, x, n_tok)
    assert np.array_equal(host(y).view(np.uint32), (prev + plain).view(np.uint32))
