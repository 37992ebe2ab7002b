"""The per-token decode chain (norm + router DMMV, routed MoE block with the
residual add, final norm + LM head + argmax) against the oracle, layer by
layer, at the widths of the pages' model: d_model 2048, 128 routed experts
of 512 (top 8) plus a shared expert.

Each layer is checked on the GPU's own state before it (chained, as the
single stages are), so that a near-tie in one layer cannot compound:
  - xn against the oracle's fp64 RMS norm of the GPU's state (4e-6, the fp32
    bound of the norm's steps);
  - router logits against the oracle's rows on the codes of that xn;
  - ids exactly and weights within 1e-6 against the oracle router on the
    GPU's logits;
  - the gate/up stage (run once more on the same inputs, which gives the
    block's own codes bit for bit): rows within the row bar, h within 1e-6
    of SwiGLU of those rows, its codes bit-exact;
  - the new state against state + the oracle's weighted down rows on those
    codes, at the row bar with the previous state in the error scale (the
    accumulate reading); and against the unchained oracle block on xn at
    the looser end-to-end MoE bar.
Then the LM head on the final state, its argmax, and a graph replay of the
whole token that must give the eager run's bits.  Finally the oracle runs
the whole chain on its own state and the final argmax must agree unless
the oracle's top two logits are a near tie."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8
D_MODEL, N_ROUTED, TOP_K, D_FF, VOCAB, LAYERS = 2048, 128, 8, 512, 8192, 3
EPS = 1e-6
XN_TOL = 4e-6        # fp32 RMS norm against the fp64 oracle
MOE_E2E_TOL = 1e-3   # unchained MoE block (an exp ulp may flip one code)
E2E_CHAIN_TOL = 1e-2  # the whole chain unchained, normwise only


def check_xn(xn_gpu, x, w, what):
    ref = oracle.rms_norm(x, w, EPS)
    xn = np.asarray(xn_gpu, np.float64)
    assert not np.isnan(xn).any(), what
    err = np.abs(xn - ref)
    assert (err <= XN_TOL * np.abs(ref)).all(), "%s: worst %g relative" % (
        what, float((err / np.maximum(np.abs(ref), 1e-300)).max()))


@pytest.fixture(scope="module")
def setup():
    torch = torch_cuda()
    from block_quant_matrix_amd import zq
    from block_quant_matrix_amd.chain import DecodeChain
    assert zq.zq_device_check(0) == 0
    rng = np.random.default_rng(81)
    H = dict(router=[], banks=[], gates=[], norms=[])
    router_d, banks_d, gates_d, norms_d = [], [], [], []
    for layer in range(LAYERS):
        r = inputs.gen_weights(Q8_0, N_ROUTED, D_MODEL, 82 + layer)
        gu, gs, dn, ds = inputs.moe_banks(90 + layer, N_ROUTED + 1, D_MODEL, D_FF)
        g = np.float32(rng.standard_normal())
        nw = (1 + 0.1 * rng.standard_normal(D_MODEL)).astype(np.float32)
        H["router"].append(r)
        H["banks"].append((gu, gs, dn, ds))
        H["gates"].append(g)
        H["norms"].append(nw)
        router_d.append(dev(r))
        banks_d.append((dev(gu), gs, dev(dn), ds, N_ROUTED + 1))
        gates_d.append(dev(np.array([g], np.float32)))
        norms_d.append(dev(nw))
    H["lm"] = inputs.gen_weights(Q4_0, VOCAB, D_MODEL, 99)
    H["final"] = (1 + 0.1 * rng.standard_normal(D_MODEL)).astype(np.float32)
    c = DecodeChain(torch, router_d, banks_d, dev(H["lm"]), norms_d, dev(H["final"]),
                    d_model=D_MODEL, n_routed=N_ROUTED, top_k=TOP_K, d_ff=D_FF, vocab=VOCAB,
                    shared_gate=gates_d, eps=EPS)
    return torch, zq, c, H


def check_layer(torch, zq, c, H, layer, x_before):
    """The checks of one layer on the GPU's state before it; returns the
    GPU's ids."""
    xn, logits = host(c.xn).copy(), host(c.logits).copy()
    ids, wts, x_after = host(c.ids).copy(), host(c.wts).copy(), host(c.x).copy()
    what = "layer %d" % layer
    check_xn(xn, x_before, H["norms"][layer], what + " norm")
    rq, rd, _ = oracle.quantize_act(xn)
    lr, lS = oracle.dmmv(Q8_0, H["router"][layer], N_ROUTED, D_MODEL, rq, rd)
    check_rows(logits, lr, lS, what + " router logits")
    rids, rw = oracle.moe_route(logits, TOP_K, H["gates"][layer])
    assert np.array_equal(ids, rids), what + " expert ids"
    assert np.allclose(wts, rw, rtol=1e-6, atol=0), what + " expert weights"

    # the gate/up stage alone on the same inputs
    gu_d, gs, dn_d, ds, ne = c.moe_banks[layer]
    gu_h, _, dn_h, _ = H["banks"][layer]
    n_sel = ids.size
    ids2, wts2 = sentinel_i32(n_sel), nan_f32(n_sel)
    qh = torch.zeros((n_sel, D_FF), dtype=torch.int8, device="cuda")
    dh, sh = nan_f32(n_sel, D_FF // 32), sentinel_i32(n_sel, D_FF // 32)
    h, gu = nan_f32(n_sel, D_FF), nan_f32(n_sel, 2 * D_FF)
    zq.zq_moe_gate_up_route(Q4_0, gu_d, gs, ne, D_MODEL, D_FF, c.logits, N_ROUTED, TOP_K,
                            c.shared_gate[layer], c.xn, ids2, wts2, qh, dh, sh, h, gu)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids2), ids)
    assert np.array_equal(host(wts2).view(np.uint32), wts.view(np.uint32))
    gu_g = host(gu)
    gu_ref, gu_S = oracle.moe_gate_up(Q4_0, gu_h, gs, D_MODEL, D_FF, ids, rq, rd)
    check_rows(gu_g, gu_ref, gu_S, what + " gate/up rows")
    h_g = host(h)
    assert np.allclose(h_g, oracle.swiglu(gu_g, D_FF), rtol=1e-6, atol=0), what + " swiglu"
    rqh, rdh, rsh = oracle.quantize_act(h_g)
    qh_g, dh_g = host(qh), host(dh)
    assert np.array_equal(qh_g, rqh) and np.array_equal(dh_g.view(np.uint32), rdh.view(np.uint32))
    assert np.array_equal(host(sh), rsh)

    # down + weighted sum + residual add, on those codes
    xb = x_before.astype(np.float64)
    y_ref, S = oracle.moe_down_weighted(Q4_0, dn_h, ds, D_MODEL, D_FF, ids,
                                        wts.astype(np.float64), qh_g, dh_g)
    check_rows(x_after, xb + y_ref, S + np.abs(xb), what + " state after the MoE block")
    # the unchained block from xn
    y_u, S_u = oracle.moe_ffn(Q4_0, gu_h, gs, dn_h, ds, D_MODEL, D_FF, ids, wts, xn)
    check_rows(x_after, xb + y_u, S_u + np.abs(xb), what + " unchained block", tol=MOE_E2E_TOL)
    return ids


def test_chain_layers_and_lm_head_against_oracle(setup):
    torch, zq, c, H = setup
    x0 = inputs.gen_activation(1, D_MODEL, 83)
    c.x.copy_(dev(x0))
    torch.cuda.synchronize()
    gpu_ids = []
    for layer in range(LAYERS):
        x_before = host(c.x).copy()
        c.step_layer(layer)
        torch.cuda.synchronize()
        gpu_ids.append(check_layer(torch, zq, c, H, layer, x_before))

    # LM head on the final state: the same rows, bit for bit, as the plain
    # fused norm DMMV, which also publishes its xn and codes
    x_final = host(c.x).copy()
    c.y_lm.fill_(float("nan"))
    c.idx.fill_(-1)
    c.lm_head()
    y_plain, xn = nan_f32(VOCAB), nan_f32(D_MODEL)
    qx = torch.zeros(D_MODEL, dtype=torch.int8, device="cuda")
    dx = nan_f32(D_MODEL // 32)
    zq.zq_rms_norm_dmmv_f32(Q4_0, c.lm_w, VOCAB, D_MODEL, c.x, c.final_norm_w, EPS, y_plain, 0,
                            qx, dx, None, xn)
    torch.cuda.synchronize()
    y_lm, idx = host(c.y_lm).copy(), int(host(c.idx)[0])
    assert np.array_equal(y_lm.view(np.uint32), host(y_plain).view(np.uint32))
    check_xn(host(xn), x_final, H["final"], "final norm")
    rq, rd, _ = oracle.quantize_act(host(xn))
    assert np.array_equal(host(qx), rq) and np.array_equal(host(dx).view(np.uint32),
                                                           rd.view(np.uint32))
    y_ref, S = oracle.dmmv(Q4_0, H["lm"], VOCAB, D_MODEL, rq, rd)
    check_rows(y_lm, y_ref, S, "LM-head logits")
    assert idx == oracle.argmax_f32(y_lm)
    top2 = np.argsort(-y_ref, kind="stable")[:2]
    if y_ref[top2[0]] - y_ref[top2[1]] >= 1e-4 * (S[top2[0]] + S[top2[1]]):
        assert idx == int(top2[0])

    # the whole token replayed as a graph gives the eager run's bits
    c.capture()
    c.x.copy_(dev(x0))
    c.y_lm.fill_(float("nan"))
    c.idx.fill_(-1)
    c.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(c.x).view(np.uint32), x_final.view(np.uint32))
    assert np.array_equal(host(c.y_lm).view(np.uint32), y_lm.view(np.uint32))
    assert int(host(c.idx)[0]) == idx

    # the oracle's own chain from x0: same experts every layer and the same
    # token, unless its logits hold a near tie where the choice is made
    x = x0.astype(np.float32)
    for layer in range(LAYERS):
        xn_o = oracle.rms_norm(x, H["norms"][layer], EPS).astype(np.float32)
        q, d, _ = oracle.quantize_act(xn_o)
        lg, lS = oracle.dmmv(Q8_0, H["router"][layer], N_ROUTED, D_MODEL, q, d)
        rids, rw = oracle.moe_route(lg.astype(np.float32), TOP_K, H["gates"][layer])
        if not np.array_equal(rids, gpu_ids[layer]):
            srt = np.sort(lg)[::-1]
            gap = srt[TOP_K - 1] - srt[TOP_K]
            assert gap < 1e-4 * float(lS.max()), "layer %d experts differ without a near tie" % layer
            return
        gu_h, gs, dn_h, ds = H["banks"][layer]
        y, _ = oracle.moe_ffn(Q4_0, gu_h, gs, dn_h, ds, D_MODEL, D_FF, rids, rw, xn_o)
        x = (x.astype(np.float64) + y).astype(np.float32)
    xn_o = oracle.rms_norm(x, H["final"], EPS).astype(np.float32)
    q, d, _ = oracle.quantize_act(xn_o)
    yo, So = oracle.dmmv(Q4_0, H["lm"], VOCAB, D_MODEL, q, d)
    # unchained over three layers an activation code may flip anywhere along
    # the way, so only a normwise bar ten times the end-to-end MoE one
    err = np.abs(y_lm.astype(np.float64) - yo) / So
    print("decode chain end to end: max |logit - oracle| = %.3g * S" % float(err.max()))
    assert float(err.max()) <= E2E_CHAIN_TOL, "oracle chain end to end: %g * S" % float(err.max())
    t2 = np.argsort(-yo, kind="stable")[:2]
    if yo[t2[0]] - yo[t2[1]] >= E2E_CHAIN_TOL * (So[t2[0]] + So[t2[1]]):
        assert idx == int(t2[0])
