"""GPU parity of zq_moe_ffn_norm_route: one layer's MoE block from the
un-normalized state, the RMS norm and Q8_0 router included (the fused norm +
router DMMV launch, then the routed block's two).

Checked against the oracle stage by stage on the GPU's own intermediates,
as the decode chain's test does: xn against the fp64 RMS norm (4e-6); the
logits against the oracle's router rows on xn's codes (row bar); ids exactly
and weights within 1e-6 against the oracle router on those logits (and bit
for bit against zq_moe_gate_up_route run on the published xn and logits,
whose codes feed the next check); y = x + the oracle's weighted down rows on
those codes (row bar, the state in the error scale), and against the
unchained oracle block at the end-to-end MoE bar."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8
EPS = 1e-6
XN_TOL = 4e-6
MOE_E2E_TOL = 1e-3


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


# the pages' widths, with and without a shared expert, Q8_0 experts, another
# width, more experts
CASES = [
    (Q4_0, 2048, 128, 8, 512, True),
    (Q4_0, 2048, 64, 4, 256, False),
    (Q8_0, 2048, 100, 6, 1024, True),
    (Q4_0, 1024, 64, 6, 512, True),
    (Q4_0, 2048, 256, 8, 512, True),
]


@pytest.mark.parametrize("wt,d_model,n_routed,top_k,d_ff,shared", CASES)
def test_norm_route_block(zq, wt, d_model, n_routed, top_k, d_ff, shared):
    torch = torch_cuda()
    seed = 7100 + d_model + n_routed + d_ff + wt
    rng = np.random.default_rng(seed)
    n_exp = n_routed + (1 if shared else 0)
    n_sel = top_k + (1 if shared else 0)
    router = inputs.gen_weights(Q8_0, n_routed, d_model, seed + 1)
    gu, gs, dn, ds = inputs.moe_banks(seed + 2, n_exp, d_model, d_ff, wt)
    nw = (1 + 0.1 * rng.standard_normal(d_model)).astype(np.float32)
    g = np.float32(rng.standard_normal()) if shared else None
    x = inputs.gen_activation(1, d_model, seed + 3)
    gu_d, dn_d, r_d, nw_d = dev(gu), dev(dn), dev(router), dev(nw)
    g_d = None if g is None else dev(np.array([g], np.float32))
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    xn, logits = nan_f32(d_model), nan_f32(n_routed)
    ids, wts = sentinel_i32(n_sel), nan_f32(n_sel)
    xy = dev(x)  # y is x itself: the residual add
    assert zq.zq_moe_ffn_norm_route(wt, gu_d, gs, dn_d, ds, n_exp, d_model, d_ff, r_d, nw_d, EPS,
                                    xy, n_routed, top_k, g_d, xn, logits, ids, wts, ws, ws_bytes,
                                    xy, 1) == 0
    torch.cuda.synchronize()
    what = "wt %d d_model %d, %d experts top %d, d_ff %d" % (wt, d_model, n_routed, top_k, d_ff)
    xn_h, lg_h, ids_h, wts_h, y_h = host(xn), host(logits), host(ids), host(wts), host(xy)
    ref = oracle.rms_norm(x, nw, EPS)
    assert (np.abs(xn_h - ref) <= XN_TOL * np.abs(ref)).all(), what + " xn"
    rq, rd, _ = oracle.quantize_act(xn_h)
    lr, lS = oracle.dmmv(Q8_0, router, n_routed, d_model, rq, rd)
    check_rows(lg_h, lr, lS, what + " router logits")
    rids, rw = oracle.moe_route(lg_h, top_k, g)
    assert np.array_equal(ids_h, rids), what + " expert ids"
    assert np.allclose(wts_h, rw, rtol=1e-6, atol=0), what + " expert weights"
    # the gate/up stage on the published xn and logits
    ids2, wts2 = sentinel_i32(n_sel), nan_f32(n_sel)
    qh = torch.zeros((n_sel, d_ff), dtype=torch.int8, device="cuda")
    dh, sh = nan_f32(n_sel, d_ff // 32), sentinel_i32(n_sel, d_ff // 32)
    assert zq.zq_moe_gate_up_route(wt, gu_d, gs, n_exp, d_model, d_ff, logits, n_routed, top_k,
                                   g_d, xn, ids2, wts2, qh, dh, sh) == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(ids2), ids_h)
    assert np.array_equal(host(wts2).view(np.uint32), wts_h.view(np.uint32))
    xb = x.astype(np.float64)
    y_ref, S = oracle.moe_down_weighted(wt, dn, ds, d_model, d_ff, ids_h, wts_h.astype(np.float64),
                                        host(qh), host(dh))
    check_rows(y_h, xb + y_ref, S + np.abs(xb), what + " state after the block")
    y_u, S_u = oracle.moe_ffn(wt, gu, gs, dn, ds, d_model, d_ff, ids_h, wts_h, xn_h)
    check_rows(y_h, xb + y_u, S_u + np.abs(xb), what + " unchained block", tol=MOE_E2E_TOL)
