"""The allocation-free LM-head step against the workspace form it mirrors:
two calls in a row on one GPU (the second over a smaller matrix, so it
reads fewer partials than the first left in the shared array), each giving
the rows and the index of zq_dmmv_f32_argmax bit for bit; the index is also
the oracle's argmax of those rows."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import dev, host, nan_f32, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8


def test_noalloc_matches_workspace_form():
    torch = torch_cuda()
    from block_quant_matrix_amd import zq
    assert zq.zq_device_check(0) == 0
    ws_bytes = zq.zq_dmmv_f32_argmax_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for wt, rows, k, seed in [(Q4_0, 248320, 2048, 9100), (Q8_0, 3001, 1024, 9101)]:
        w = dev(inputs.gen_weights(wt, rows, k, seed))
        x = dev(inputs.gen_activation(1, k, seed + 1))
        y_ref, i_ref = nan_f32(rows), sentinel_i32(1)
        assert zq.zq_dmmv_f32_argmax(wt, w, rows, k, x, y_ref, i_ref, ws, ws_bytes) == 0
        y, i = nan_f32(rows), sentinel_i32(1)
        assert zq.zq_dmmv_f32_argmax_noalloc(wt, w, rows, k, x, y, i) == 0
        torch.cuda.synchronize()
        yh = host(y)
        assert not np.isnan(yh).any()
        assert np.array_equal(yh.view(np.uint32), host(y_ref).view(np.uint32)), (wt, rows, k)
        idx = int(host(i)[0])
        assert idx == int(host(i_ref)[0]) == oracle.argmax_f32(yh), (wt, rows, k)
    # argument errors are reported before anything runs
    with pytest.raises(zq.ZQError):
        zq.zq_dmmv_f32_argmax_noalloc(Q4_0, w, 0, 1024, x, y, i)
    with pytest.raises(zq.ZQError):
        zq.zq_dmmv_f32_argmax_noalloc(Q4_0, w, 16, 32768, x, y, i)
