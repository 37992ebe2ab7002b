"""GPU parity of the multi-token DMMV (2..8 tokens in one weight pass)
against the oracle's single-token rows, token by token."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def run_tok(zq, wt, w, rows, k, qx, dx, sx, n_tok, y=None, flags=0):
    y = nan_f32(n_tok, rows) if y is None else y
    wd = dev(w) if isinstance(w, np.ndarray) else w
    assert zq.zq_dmmv_tokens(wt, wd, rows, k, qx, dx, sx, n_tok, y, flags) == 0
    return y


def oracle_rows(wt, w, rows, k, x, rows_eval=None, y_prev=None):
    """Per token: the oracle's quantization and fp64 rows."""
    rq, rd, _ = oracle.quantize_act(x)
    out = []
    for t in range(x.shape[0]):
        yp = None if y_prev is None else y_prev[t]
        out.append(oracle.dmmv(wt, w, rows, k, rq[t], rd[t], rows_eval=rows_eval, y_prev=yp))
    return out


# k spans one pass of every (LPR, BPL) layout and several passes; rows are
# ragged against the row groups.
@pytest.mark.parametrize("wt", [Q4_0, Q8_0])
@pytest.mark.parametrize("n_tok", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("rows,k", [(1, 32), (37, 64), (130, 512), (300, 2048), (65, 4096),
                                    (9, 5120), (5, 16384), (4099, 1024)])
def test_tokens_rows(zq, wt, n_tok, rows, k):
    seed = 900 + 31 * n_tok + rows + k + wt
    w = inputs.gen_weights(wt, rows, k, seed)
    x = inputs.gen_activation(n_tok, k, seed + 1).reshape(n_tok, k)
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, wt, w, rows, k, qx, dx, sx, n_tok))
    for t, (y_ref, S) in enumerate(oracle_rows(wt, w, rows, k, x)):
        check_rows(y[t], y_ref, S, "wt %d tokens %d, token %d, %d x %d" % (wt, n_tok, t, rows, k))
    if wt == Q4_0:
        # without block sums the kernel sums the codes itself: same bits
        y2 = host(run_tok(zq, wt, w, rows, k, qx, dx, None, n_tok))
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("wt", [Q4_0, Q8_0])
def test_tokens_accumulate_and_determinism(zq, wt):
    rows, k, n_tok = 2048, 2048, 6
    w = inputs.gen_weights(wt, rows, k, 95 + wt)
    x = inputs.gen_activation(n_tok, k, 96)
    qx, dx, sx = quantize_gpu(zq, x)
    prev = np.random.default_rng(4).standard_normal((n_tok, rows)).astype(np.float32)
    y = dev(prev)
    wd = dev(w)
    run_tok(zq, wt, wd, rows, k, qx, dx, sx, n_tok, y=y, flags=1)
    yh = host(y)
    for t, (y_ref, S) in enumerate(oracle_rows(wt, w, rows, k, x, y_prev=prev)):
        check_rows(yh[t], y_ref, S, "accumulate token %d" % t)
    a = host(run_tok(zq, wt, wd, rows, k, qx, dx, sx, n_tok))
    b = host(run_tok(zq, wt, wd, rows, k, qx, dx, sx, n_tok))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tokens_identical_tokens_equal_single(zq):
    """n copies of one token give n identical rows, each within the bar of
    the single-token DMMV's oracle (P11-style invariance over tokens)."""
    rows, k = 1000, 2048
    w = inputs.gen_weights(Q4_0, rows, k, 97)
    x1 = inputs.gen_activation(1, k, 98)
    x = np.tile(x1, (8, 1))
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, Q4_0, w, rows, k, qx, dx, sx, 8))
    assert all(np.array_equal(y[0].view(np.uint32), y[t].view(np.uint32)) for t in range(8))
    rq, rd, _ = oracle.quantize_act(x1)
    y_ref, S = oracle.dmmv(Q4_0, w, rows, k, rq, rd)
    check_rows(y[0], y_ref, S, "identical tokens")


def test_tokens_empty(zq):
    w = inputs.gen_weights(Q4_0, 4, 64, 1)
    x = inputs.gen_activation(2, 64, 2)
    qx, dx, sx = quantize_gpu(zq, x)
    y = nan_f32(2, 4)
    assert zq.zq_dmmv_tokens(Q4_0, dev(w), 0, 64, qx, dx, sx, 2, y, 0) == 0
    assert np.isnan(host(y)).all()


@pytest.mark.parametrize("n_tok", [2, 4, 8])
def test_tokens_full_size(zq, n_tok):
    """4096 x 4096 Q4_0, every row of every token."""
    rows, k = 4096, 4096
    w = inputs.gen_weights(Q4_0, rows, k, 2000 + n_tok)
    x = inputs.gen_activation(n_tok, k, 2001)
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, Q4_0, w, rows, k, qx, dx, sx, n_tok))
    for t, (y_ref, S) in enumerate(oracle_rows(Q4_0, w, rows, k, x)):
        check_rows(y[t], y_ref, S, "4096 x 4096, %d tokens, token %d" % (n_tok, t))


def test_tokens_lmhead_sampled(zq):
    """The LM-head shape 248 320 x 2048 with 8 tokens: every output written,
    sampled rows of every token against the oracle."""
    rows, k, n_tok = 248320, 2048, 8
    w = inputs.gen_weights(Q4_0, rows, k, 3000)
    x = inputs.gen_activation(n_tok, k, 3001)
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, Q4_0, w, rows, k, qx, dx, sx, n_tok))
    assert not np.isnan(y).any()
    rng = np.random.default_rng(6)
    idx = np.unique(np.concatenate([np.arange(32), np.arange(rows - 32, rows),
                                    rng.integers(0, rows, 1000)])).astype(np.int64)
    for t, (y_ref, S) in enumerate(oracle_rows(Q4_0, w, rows, k, x, rows_eval=idx)):
        check_rows(y[t][idx], y_ref, S, "lm head 8 tokens, token %d" % t)


# Tall matrices with 3+ tokens take the matrix-core form (rows >= 65536,
# its LDS within 64 KB): rows ragged against the 128-row workgroups, k from
# one block (less than one 8-block chunk) to 4096 (at 8 tokens the vector
# form again), block counts that end a chunk part-way and split a pair of
# blocks (9 and 65), 2 tokens the vector form; every row's first and last
# outputs and sampled ones against the oracle.
@pytest.mark.parametrize("wt", [Q4_0, Q8_0])
@pytest.mark.parametrize("n_tok", [2, 3, 5, 8])
@pytest.mark.parametrize("rows,k", [(65536 + 37, 32), (65536 + 1, 288), (70001, 2048),
                                    (66000, 2080), (65600, 4096)])
def test_tokens_tall_matrix_cores(zq, wt, n_tok, rows, k):
    seed = 7000 + 31 * n_tok + k + wt
    if wt == Q8_0 and k == 4096:
        # 285 MB of Q8_0: the matrix is built on the device by repeating a
        # seeded base of BASE_ROWS rows (a period that no row tile, wave or
        # workgroup size divides, so a row mapped to the wrong tile still
        # reads different bytes); the oracle evaluates the base rows
        base = inputs.gen_weights(wt, BASE_ROWS, k, seed)
        w = tile_rows_on_device(base, BASE_ROWS, rows)
        w_ref, ref_rows = base, BASE_ROWS
    else:
        w = inputs.gen_weights(wt, rows, k, seed)
        w_ref, ref_rows = w, rows
    x = inputs.gen_activation(n_tok, k, seed + 1).reshape(n_tok, k)
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, wt, w, rows, k, qx, dx, sx, n_tok))
    assert not np.isnan(y).any()
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 512)])).astype(np.int64)
    for t, (y_ref, S) in enumerate(oracle_rows(wt, w_ref, ref_rows, k, x,
                                               rows_eval=idx % ref_rows)):
        check_rows(y[t][idx], y_ref, S, "tall %d x %d, %d tokens, token %d" % (rows, k, n_tok, t))


BASE_ROWS = 4099


def tile_rows_on_device(base: np.ndarray, base_rows: int, rows: int):
    """A rows-row weight matrix on the device whose row r is row r % base_rows
    of `base` (rows are whole blocks, so rows concatenate as bytes)."""
    rb = base.size // base_rows
    reps = -(-rows // base_rows)
    return dev(base).repeat(reps)[:rows * rb].contiguous()


# Shorter matrices with 5..8 tokens, 64..128 blocks per row and at least
# 8 M weights take the tile form: rows ragged against the 16-row tiles, a
# last chunk that ends part-way (65 blocks) and splits a block pair.
@pytest.mark.parametrize("wt", [Q4_0, Q8_0])
@pytest.mark.parametrize("n_tok", [5, 8])
@pytest.mark.parametrize("rows,k", [(4100, 2048), (4033, 2080), (4096, 4096)])
def test_tokens_tile_form(zq, wt, n_tok, rows, k):
    seed = 7500 + 31 * n_tok + k + wt
    w = inputs.gen_weights(wt, rows, k, seed)
    x = inputs.gen_activation(n_tok, k, seed + 1).reshape(n_tok, k)
    qx, dx, sx = quantize_gpu(zq, x)
    y = host(run_tok(zq, wt, w, rows, k, qx, dx, sx, n_tok))
    for t, (y_ref, S) in enumerate(oracle_rows(wt, w, rows, k, x)):
        check_rows(y[t], y_ref, S, "tile %d x %d, %d tokens, token %d" % (rows, k, n_tok, t))
    prev = np.random.default_rng(seed).standard_normal((n_tok, rows)).astype(np.float32)
    y2 = dev(prev)
    run_tok(zq, wt, w, rows, k, qx, dx, sx, n_tok, y=y2, flags=1)
    yh = host(y2)
    idx = np.arange(0, rows, 7)
    for t, (y_ref, S) in enumerate(oracle_rows(wt, w, rows, k, x, rows_eval=idx, y_prev=prev)):
        check_rows(yh[t][idx], y_ref, S, "tile accumulate, token %d" % t)


def test_tokens_tall_accumulate(zq):
    rows, k, n_tok = 65536 + 5, 2048, 4
    w = inputs.gen_weights(Q4_0, rows, k, 7100)
    x = inputs.gen_activation(n_tok, k, 7101)
    qx, dx, sx = quantize_gpu(zq, x)
    prev = np.random.default_rng(7102).standard_normal((n_tok, rows)).astype(np.float32)
    y = dev(prev)
    run_tok(zq, Q4_0, w, rows, k, qx, dx, sx, n_tok, y=y, flags=1)
    yh = host(y)
    idx = np.unique(np.concatenate([np.arange(16), np.arange(rows - 16, rows),
                                    np.random.default_rng(3).integers(0, rows, 256)])).astype(np.int64)
    for t, (y_ref, S) in enumerate(oracle_rows(Q4_0, w, rows, k, x, rows_eval=idx, y_prev=prev)):
        check_rows(yh[t][idx], y_ref, S, "tall accumulate, token %d" % t)
