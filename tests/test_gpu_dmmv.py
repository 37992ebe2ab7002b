"""GPU parity of the activation quantizer, the Q4_0/Q8_0 DMMV and argmax
against the CPU oracle, through the C ABI.

Bar: bit-exact qx / dx / sx and per-block int32 sums; fp32 rows within 1e-4 of
the fp64 reference (normwise against S, elementwise on well-conditioned rows);
argmax exact on the GPU's own logits.
"""
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
    assert _zq.zq_device_check(0) == 0, "not a gfx950 device"
    return _zq


# --------------------------------------------------------------- quantize --

def special_activation(k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(k).astype(np.float32)
    nb = k // 32
    if nb >= 1:
        x[0:32] = 0.0                                    # zero block -> d = 0
    if nb >= 2:                                          # half-way cases
        u = 2.0 ** -5
        blk = np.zeros(32)
        blk[0] = 127 * u
        blk[1:7] = np.array([2.5, -2.5, 0.5, -0.5, 1.5, -1.5]) * u
        x[32:64] = blk
    if nb >= 3:
        x[64:96] = np.float32(3.3)                       # constant block
    if nb >= 4:
        x[96:128] *= np.float32(1e-30)                   # tiny magnitudes
    if nb >= 5:
        x[128:160] *= np.float32(1e30)                   # huge magnitudes
    return x


@pytest.mark.parametrize("t,k", [(1, 32), (1, 2048), (1, 4096), (3, 96), (7, 5120), (512, 5120),
                                 (1, 512)])
def test_quantize_bitexact(zq, t, k):
    x = inputs.gen_activation(t, k, 7000 + t + k).reshape(t, k)
    x[0] = special_activation(k, 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(host(dx).view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(host(sx), rs)


def test_quantize_halfway_after_rounding(zq):
    """fp32 products that round to exactly c + 1/2: the GPU must round the
    product before deciding, as the oracle does (no fused multiply-add)."""
    from cases import halfway_after_rounding
    for seed in (1, 2, 3):
        x, hits = halfway_after_rounding(seed)
        qx, dx, sx = quantize_gpu(zq, x)
        rq, rd, rs = oracle.quantize_act(x)
        q = host(qx)[0]
        assert all(int(rq[i]) == want for i, want in hits)
        assert np.array_equal(q, rq), int((q != rq).sum())
        assert np.array_equal(host(dx)[0], rd) and np.array_equal(host(sx)[0], rs)


def test_quantize_strided_rows_and_null_sums(zq):
    torch = torch_cuda()
    t, k, stride = 5, 256, 260
    x = np.random.default_rng(3).standard_normal((t, stride)).astype(np.float32)
    qx = torch.zeros((t, k), dtype=torch.int8, device="cuda")
    dx = nan_f32(t, k // 32)
    zq.zq_quantize_act(dev(x), t, k, stride, qx, dx, None)
    rq, rd, _ = oracle.quantize_act(x[:, :k])
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(host(dx), rd)


# ------------------------------------------------------------------ dmmv ---

SHAPES = [(1, 32), (7, 64), (64, 2048), (130, 96), (33, 512), (257, 4096), (70, 5120),
          (19, 32 * 200), (5, 32 * 9), (1000, 32 * 3)]


def run_dmmv(zq, wtype, w_np, rows, k, qx, dx, sx, y=None, flags=0):
    y = nan_f32(rows) if y is None else y
    wd = dev(w_np)
    if wtype == Q4:
        zq.zq_dmmv_q4_0(wd, rows, k, qx, dx, sx, y, flags)
    else:
        zq.zq_dmmv_q8_0(wd, rows, k, qx, dx, y, flags)
    return y


@pytest.mark.parametrize("wtype", [Q4, Q8])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_dmmv_isums_and_rows(zq, wtype, rows, k):
    seed = 100 * rows + k + wtype
    w = inputs.gen_weights(wtype, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(qx)[0], rq)
    y_ref, S, isums_ref = oracle.dmmv(wtype, w, rows, k, rq, rd, want_isums=True)
    isums = sentinel_i32(rows, k // 32)
    zq.zq_dmmv_isums(wtype, dev(w), rows, k, qx, sx, isums)
    assert np.array_equal(host(isums), isums_ref)
    y = run_dmmv(zq, wtype, w, rows, k, qx, dx, sx)
    check_rows(host(y), y_ref, S, "dmmv wtype=%d %dx%d" % (wtype, rows, k))
    if wtype == Q4:  # the kernel's own block sums when sx is not given
        isums2 = sentinel_i32(rows, k // 32)
        zq.zq_dmmv_isums(wtype, dev(w), rows, k, qx, None, isums2)
        assert np.array_equal(host(isums2), isums_ref)
        y2 = run_dmmv(zq, wtype, w, rows, k, qx, dx, None)
        assert np.array_equal(host(y2), host(y))


@pytest.mark.parametrize("wtype", [Q4, Q8])
@pytest.mark.parametrize("rows,k", SHAPES + [(4096, 4096), (5000, 2048), (20000, 512)])
def test_dmmv_f32_fused(zq, wtype, rows, k):
    """Quantize + DMMV in one launch: the quantized activation it writes out is
    bit-exact with the oracle, the rows are within tolerance."""
    torch = torch_cuda()
    seed = 300 * rows + k + wtype
    w = inputs.gen_weights(wtype, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    if k >= 64:
        x[:64] = special_activation(64, 2)
    y = nan_f32(rows)
    qxo = torch.full((k,), 0x55, dtype=torch.int8, device="cuda")
    dxo = nan_f32(k // 32)
    sxo = sentinel_i32(k // 32)
    wd = dev(w)
    zq.zq_dmmv_f32(wtype, wd, rows, k, dev(x), y, 0, qxo, dxo, sxo)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(qxo), rq)
    assert np.array_equal(host(dxo).view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(host(sxo), rs)
    y_ref, S = oracle.dmmv(wtype, w, rows, k, rq, rd)
    check_rows(host(y), y_ref, S, "fused wtype=%d %dx%d" % (wtype, rows, k))
    # accumulate, and no quantized-activation output
    y2 = y.clone()
    zq.zq_dmmv_f32(wtype, wd, rows, k, dev(x), y2, 1)
    assert np.allclose(host(y2), 2 * host(y), rtol=1e-6, atol=0)


@pytest.mark.parametrize("wtype", [Q4, Q8])
def test_dmmv_accumulate(zq, wtype):
    rows, k = 300, 2048
    w = inputs.gen_weights(wtype, rows, k, 31)
    x = inputs.gen_activation(1, k, 32)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    prev = np.random.default_rng(33).standard_normal(rows).astype(np.float32)
    y = dev(prev.copy())
    run_dmmv(zq, wtype, w, rows, k, qx, dx, sx, y=y, flags=1)
    y_ref, S = oracle.dmmv(wtype, w, rows, k, rq, rd, y_prev=prev)
    check_rows(host(y), y_ref, S, "accumulate")


@pytest.mark.parametrize("wtype", [Q4, Q8])
def test_dmmv_all_ones_exact(zq, wtype):
    """Every row must come back as exactly 2032.0 (= K * 127/128)."""
    rows, k = 200, 2048
    if wtype == Q8:
        blk = np.frombuffer(np.array([1.0], "<f2").tobytes() + bytes([1] * 32), np.uint8)
    else:
        blk = np.frombuffer(np.array([1.0], "<f2").tobytes() + bytes([0x99] * 16), np.uint8)
    w = np.tile(blk, rows * (k // 32))
    x = np.full(k, 127 / 128, np.float32)
    qx, dx, sx = quantize_gpu(zq, x)
    y = run_dmmv(zq, wtype, w, rows, k, qx, dx, sx)
    assert (host(y) == 2032.0).all()


@pytest.mark.parametrize("wtype", [Q4, Q8])
def test_dmmv_single_nonzero_block(zq, wtype):
    """All scales zero except (r*, b*) = 2^-3 with a lossless activation:
    exactly one non-zero row with the exact value 2^-3 * 2^-6 * isum."""
    rows, k = 130, 32 * 66
    nb = k // 32
    bb = inputs.BLOCK_BYTES[wtype]
    rng = np.random.default_rng(5)
    kint = rng.integers(-127, 128, size=k)
    kint[::32] = 127
    x = (kint * 2.0 ** -6).astype(np.float32)
    qx, dx, sx = quantize_gpu(zq, x)
    base = inputs.gen_weights(wtype, rows, k, 77).reshape(rows * nb, bb)
    base[:, 0:2] = 0
    for rstar, bstar in [(0, 0), (rows - 1, nb - 1), (63, 31), (64, 32), (65, 64), (128, 65)]:
        w = base.copy()
        w[rstar * nb + bstar, 0:2] = np.frombuffer(np.array([0.125], "<f2").tobytes(), np.uint8)
        y = host(run_dmmv(zq, wtype, w.reshape(-1), rows, k, qx, dx, sx))
        blk = w[rstar * nb + bstar]
        vals = (blk[2:].view(np.int8).astype(np.int64) if wtype == Q8 else
                np.concatenate([blk[2:] & 15, blk[2:] >> 4]).astype(np.int64) - 8)
        want = np.zeros(rows)
        want[rstar] = 0.125 * 2.0 ** -6 * int(np.dot(vals, kint[bstar * 32:(bstar + 1) * 32]))
        assert np.array_equal(y.astype(np.float64), want), (rstar, bstar)


def test_dmmv_every_fp16_scale(zq):
    """Scales run through every finite fp16 bit pattern (subnormals included):
    the GPU must decode each exactly (integer sums unaffected; rows within
    tolerance of the fp64 reference)."""
    rows, k = 1024, 2048
    nb = k // 32
    w = inputs.gen_weights(Q4, rows, k, 55).reshape(rows * nb, 18)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(pats.view(np.float16))
    pats = np.where(finite, pats, 0).astype("<u2")
    w[:, 0:2] = pats.view(np.uint8).reshape(-1, 2)
    w = w.reshape(-1)
    x = inputs.gen_activation(1, k, 56)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.dmmv(Q4, w, rows, k, rq, rd)
    y = run_dmmv(zq, Q4, w, rows, k, qx, dx, sx)
    check_rows(host(y), y_ref, S, "every fp16 scale")


@pytest.mark.parametrize("wtype", [Q4, Q8])
def test_dmmv_deterministic(zq, wtype):
    rows, k = 4096, 4096
    w = inputs.gen_weights(wtype, rows, k, 9)
    x = inputs.gen_activation(1, k, 10)
    qx, dx, sx = quantize_gpu(zq, x)
    y1 = host(run_dmmv(zq, wtype, w, rows, k, qx, dx, sx))
    y2 = host(run_dmmv(zq, wtype, w, rows, k, qx, dx, sx))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_dmmv_empty_rows(zq):
    torch = torch_cuda()
    qx, dx, sx = quantize_gpu(zq, inputs.gen_activation(1, 64, 1))
    y = nan_f32(1)
    zq.zq_dmmv_q4_0(dev(np.zeros(64, np.uint8)), 0, 64, qx, dx, sx, y)
    torch.cuda.synchronize()
    assert np.isnan(host(y)).all()  # nothing written


# -------------------------------------------------------------- argmax -----

def gpu_argmax(zq, y_np):
    torch = torch_cuda()
    n = y_np.size
    yd = dev(y_np.astype(np.float32))
    ws_bytes = zq.zq_argmax_workspace_bytes(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = sentinel_i32(1)
    zq.zq_argmax_f32(yd, n, out, ws, ws_bytes)
    return int(host(out)[0])


def test_argmax_cases(zq):
    y = np.zeros(100, np.float32)
    y[5] = y[7] = 3.0
    assert gpu_argmax(zq, y) == 5
    assert gpu_argmax(zq, -np.arange(1, 130, dtype=np.float32)) == 0
    assert gpu_argmax(zq, np.arange(67, dtype=np.float32)) == 66
    assert gpu_argmax(zq, np.full(1, -7.0, np.float32)) == 0
    for n in (63, 64, 65, 1023, 1025, 248320, 1 << 20):
        y = np.random.default_rng(n).standard_normal(n).astype(np.float32)
        assert gpu_argmax(zq, y) == oracle.argmax_f32(y), n
    y = np.zeros(248320, np.float32)
    y[[1000, 200000, 248319]] = 1.0  # ties across partial blocks -> lowest
    assert gpu_argmax(zq, y) == 1000


# ---------------------------------------------- workloads at full size -----

@pytest.mark.parametrize("wl", [1, 2])
@pytest.mark.parametrize("s", [0, 1, 2])
def test_workload_dmmv_full(zq, wl, s):
    cfg = inputs.WORKLOADS[wl]
    wt, rows, k = cfg["wtype"], cfg["rows"], cfg["k"]
    w = inputs.gen_weights(wt, rows, k, inputs.seed_for(wl, s))
    x = inputs.gen_activation(1, k, inputs.seed_for(wl, s) + 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(qx)[0], rq) and np.array_equal(host(dx)[0], rd)
    assert np.array_equal(host(sx)[0], rs)
    y_ref, S, isums_ref = oracle.dmmv(wt, w, rows, k, rq, rd, want_isums=True)
    isums = sentinel_i32(rows, k // 32)
    zq.zq_dmmv_isums(wt, dev(w), rows, k, qx, sx, isums)
    assert np.array_equal(host(isums), isums_ref)
    y = run_dmmv(zq, wt, w, rows, k, qx, dx, sx)
    check_rows(host(y), y_ref, S, cfg["name"])
    yf = nan_f32(rows)
    zq.zq_dmmv_f32(wt, dev(w), rows, k, dev(x), yf)
    check_rows(host(yf), y_ref, S, cfg["name"] + " fused")


def test_workload_lmhead_full_and_argmax(zq):
    """248320 x 2048 Q4_0 logits, every row against the oracle, then argmax."""
    torch = torch_cuda()
    cfg = inputs.WORKLOADS[3]
    wt, rows, k = cfg["wtype"], cfg["rows"], cfg["k"]
    w = inputs.gen_weights(wt, rows, k, inputs.seed_for(3))
    x = inputs.gen_activation(1, k, inputs.seed_for(3) + 1)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    assert np.array_equal(host(qx)[0], rq)
    y = run_dmmv(zq, wt, w, rows, k, qx, dx, sx)
    y_ref, S = oracle.dmmv(wt, w, rows, k, rq, rd)
    y_h = host(y)
    check_rows(y_h, y_ref, S, cfg["name"])
    ws_bytes = zq.zq_argmax_workspace_bytes(rows)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = sentinel_i32(1)
    zq.zq_argmax_f32(y, rows, out, ws, ws_bytes)
    idx = int(host(out)[0])
    # exact on the GPU's own logits
    assert idx == oracle.argmax_f32(y_h)
    # against the oracle's logits: equal unless its top two are within the
    # fp32 error bound of each other
    order = np.argsort(-y_ref, kind="stable")
    i1, i2 = int(order[0]), int(order[1])
    if y_ref[i1] - y_ref[i2] >= 1e-4 * (S[i1] + S[i2]):
        assert idx == i1
    else:
        assert y_ref[i1] - y_ref[idx] <= 1e-4 * (S[i1] + S[idx])


# ------------------------------------------- LM head in two launches -------

def lmhead_gpu(zq, wt, w_dev, rows, k, x_np):
    """zq_dmmv_f32_argmax on one activation: (y, idx) on the host."""
    torch = torch_cuda()
    ws_bytes = zq.zq_dmmv_f32_argmax_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = nan_f32(rows)
    out = sentinel_i32(1)
    zq.zq_dmmv_f32_argmax(wt, w_dev, rows, k, dev(x_np.astype(np.float32).ravel()), y, out, ws,
                          ws_bytes)
    return host(y), int(host(out)[0])


def fused_rows(zq, wt, w_dev, rows, k, x_np):
    y = nan_f32(rows)
    zq.zq_dmmv_f32(wt, w_dev, rows, k, dev(x_np.astype(np.float32).ravel()), y)
    return host(y)


@pytest.mark.parametrize("wtype", [Q4, Q8])
@pytest.mark.parametrize("rows,k", [(1, 32), (7, 96), (1000, 2048), (4097, 2080), (300, 8192),
                                    (70000, 256), (5000, 16384)])
def test_lmhead_fused_small(zq, wtype, rows, k):
    """y equals zq_dmmv_f32's rows bit for bit (the same kernel, whose
    workgroups here walk several row groups) and the oracle's within the
    bar; the index is the exact argmax of those logits."""
    seed = 77 + rows + k + wtype
    w = inputs.gen_weights(wtype, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    wd = dev(w)
    y, idx = lmhead_gpu(zq, wtype, wd, rows, k, x)
    y_f = fused_rows(zq, wtype, wd, rows, k, x)
    assert np.array_equal(y.view(np.uint32), y_f.view(np.uint32))
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.dmmv(wtype, w, rows, k, rq, rd)
    check_rows(y, y_ref, S, "lmhead %d x %d" % (rows, k))
    assert idx == oracle.argmax_f32(y)


# Every branch of the fused DMMV's launch table: two blocks per lane past
# 8192 rows (4 row steps), four and five blocks per lane at mid size (2 row
# steps), and past 16384 rows two blocks (4 waves of 4 row steps) and eight
# (4 waves of 2).  The rows against the oracle; the argmax form's rows equal
# the plain form's bit for bit and its index is their exact argmax.
@pytest.mark.parametrize("wtype", [Q4, Q8])
@pytest.mark.parametrize("rows,k", [(10001, 4096), (3000, 8192), (5000, 5120), (20000, 4096),
                                    (17000, 8192)])
def test_dmmv_f32_launch_table(zq, wtype, rows, k):
    seed = 91 + rows + k + wtype
    w = inputs.gen_weights(wtype, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    wd = dev(w)
    y_f = fused_rows(zq, wtype, wd, rows, k, x)
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.dmmv(wtype, w, rows, k, rq, rd)
    check_rows(y_f, y_ref, S, "launch table %d x %d" % (rows, k))
    y, idx = lmhead_gpu(zq, wtype, wd, rows, k, x)
    assert np.array_equal(y.view(np.uint32), y_f.view(np.uint32))
    assert idx == oracle.argmax_f32(y)


def test_lmhead_fused_ties_and_ends(zq):
    """Equal logits resolve to the lowest row, across workgroups too; the
    maximum at the first and at the last row is found."""
    rows, k = 9000, 64
    base = inputs.gen_weights(Q4, 1, k, 5).ravel()  # one 36-byte row
    x = inputs.gen_activation(1, k, 6)
    rq, rd, _ = oracle.quantize_act(x)
    # every row identical -> all logits equal -> row 0
    w = np.tile(base, rows)
    y, idx = lmhead_gpu(zq, Q4, dev(w), rows, k, x)
    assert np.all(y == y[0]) and idx == 0
    # rows with all-zero scales give 0; one row copies base with a positive
    # logit: place it (and a tie) at chosen rows
    y1, _ = oracle.dmmv(Q4, base, 1, k, rq, rd)
    sign = 1.0 if y1[0] > 0 else -1.0
    zero_row = base.copy().reshape(2, 18)
    zero_row[:, 0:2] = 0                           # fp16 scale 0 in both blocks
    neg = base.copy().reshape(2, 18)
    if sign < 0:                                   # flip to a positive logit: negate scales
        for b in range(2):
            d = np.frombuffer(neg[b, 0:2].tobytes(), np.float16)[0]
            neg[b, 0:2] = np.frombuffer(np.float16(-d).tobytes(), np.uint8)
    pos = neg.ravel()
    for rows_at in ([0], [rows - 1], [4500, 8999], [123, 124, 8000]):
        w = np.tile(zero_row.ravel(), rows)
        for r in rows_at:
            w[r * 36:(r + 1) * 36] = pos
        y, idx = lmhead_gpu(zq, Q4, dev(w), rows, k, x)
        assert y[rows_at[0]] > 0
        assert idx == min(rows_at), rows_at


@pytest.mark.parametrize("wl", [3, 13])
def test_workload_lmhead_two_launch_full(zq, wl):
    """248320 x 2048 Q4_0 and Q8_0 through zq_dmmv_f32_argmax: the same
    logits as zq_dmmv_f32, bit for bit, the oracle's within the bar, and the
    exact argmax of them."""
    cfg = inputs.WORKLOADS[wl]
    wt, rows, k = cfg["wtype"], cfg["rows"], cfg["k"]
    w = inputs.gen_weights(wt, rows, k, inputs.seed_for(wl))
    x = inputs.gen_activation(1, k, inputs.seed_for(wl) + 1)
    wd = dev(w)
    y, idx = lmhead_gpu(zq, wt, wd, rows, k, x)
    y_f = fused_rows(zq, wt, wd, rows, k, x)
    assert np.array_equal(y.view(np.uint32), y_f.view(np.uint32))
    rq, rd, _ = oracle.quantize_act(x)
    y_ref, S = oracle.dmmv(wt, w, rows, k, rq, rd)
    check_rows(y, y_ref, S, cfg["name"] + " two-launch")
    assert idx == oracle.argmax_f32(y)
    # out_idx = NULL: the logits alone, identical
    torch = torch_cuda()
    ws_bytes = zq.zq_dmmv_f32_argmax_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y2 = nan_f32(rows)
    zq.zq_dmmv_f32_argmax(wt, wd, rows, k, dev(x.ravel()), y2, None, ws, ws_bytes)
    assert np.array_equal(host(y2).view(np.uint32), y.view(np.uint32))
