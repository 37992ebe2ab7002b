"""GPU parity of the F16 / F32 weight DMMV (zq_dmmv_float) against the
oracle's fp64 rows over the same fp32 activation, at the row bar: rows of
one, several and ragged chunk passes, ragged against the row groups, the
accumulate flag, and the LM-head shape on sampled rows."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, torch_cuda

pytestmark = pytest.mark.gpu

F16, F32 = 16, 32


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


# k from one 16-byte chunk to 16384, with chunk counts that end a pass of
# 64 lanes part-way (4104 F16 = 513 chunks, 1000 F32 = 250 chunks); rows
# ragged against the 1-, 2- and 4-row groups and the 4- and 8-wave
# workgroups (70001 x 2048 takes the 4-row LM-head launch).
@pytest.mark.parametrize("wt", [F16, F32])
@pytest.mark.parametrize("rows,k", [(1, 8), (37, 64), (130, 512), (300, 2048), (4096, 4096),
                                    (65, 4104), (7, 1000), (5, 16384), (4099, 1024),
                                    (70001, 2048)])
def test_float_rows(zq, wt, rows, k):
    seed = 8000 + rows + k + wt
    w = inputs.gen_weights_float(wt, rows, k, seed)
    x = inputs.gen_activation(1, k, seed + 1)
    y = nan_f32(rows)
    assert zq.zq_dmmv_float(wt, dev(w), rows, k, dev(x), y) == 0
    y_ref, S = oracle.float_dmmv(wt, w, rows, k, x)
    check_rows(host(y), y_ref, S, "float %d: %d x %d" % (wt, rows, k))


@pytest.mark.parametrize("wt", [F16, F32])
def test_float_accumulate_and_determinism(zq, wt):
    rows, k = 1031, 2048
    w = inputs.gen_weights_float(wt, rows, k, 8100 + wt)
    x = inputs.gen_activation(1, k, 8101)
    prev = np.random.default_rng(8102).standard_normal(rows).astype(np.float32)
    wd, xd = dev(w), dev(x)
    y = dev(prev)
    zq.zq_dmmv_float(wt, wd, rows, k, xd, y, 1)
    y_ref, S = oracle.float_dmmv(wt, w, rows, k, x, y_prev=prev)
    check_rows(host(y), y_ref, S, "float accumulate")
    a, b = nan_f32(rows), nan_f32(rows)
    zq.zq_dmmv_float(wt, wd, rows, k, xd, a)
    zq.zq_dmmv_float(wt, wd, rows, k, xd, b)
    assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))


def test_float_lmhead_sampled(zq):
    """The F16 LM head, 248 320 x 2048 (1 GB), built on the device from a
    seeded base of 4099 rows (a period no row group or workgroup divides);
    every row written, sampled rows against the oracle's base rows."""
    torch = torch_cuda()
    rows, k, base_rows = 248320, 2048, 4099
    base = inputs.gen_weights_float(F16, base_rows, k, 8200)
    reps = -(-rows // base_rows)
    wd = dev(base).repeat(reps)[:rows * k * 2].contiguous()
    x = inputs.gen_activation(1, k, 8201)
    y = nan_f32(rows)
    zq.zq_dmmv_float(F16, wd, rows, k, dev(x), y)
    yh = host(y)
    assert not np.isnan(yh).any()
    rng = np.random.default_rng(8202)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 2000)])).astype(np.int64)
    y_ref, S = oracle.float_dmmv(F16, base, base_rows, k, x, rows_eval=idx % base_rows)
    check_rows(yh[idx], y_ref, S, "F16 LM head")
    del wd
    torch.cuda.empty_cache()
