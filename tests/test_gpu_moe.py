"""GPU parity of the MoE path: router, expert gather DMMV, swiglu +
re-quantization, weighted down DMMV, and the one-token composite.

Stages are chained: each stage is compared against the oracle evaluated on
the GPU's own output of the previous stage, so the integer parts stay
bit-exact even where exp() may differ by an ulp between CPU and GPU.
"""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4 = 4
WL = inputs.WORKLOADS[4]
E_ROUTED, TOP_K, D_MODEL, D_FF = WL["n_routed"], WL["top_k"], WL["d_model"], WL["d_ff"]
N_EXPERTS = E_ROUTED + 1  # + the shared expert


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


@pytest.fixture(scope="module")
def banks():
    gu, gs, down, ds = inputs.moe_banks(inputs.seed_for(4), N_EXPERTS, D_MODEL, D_FF)
    return dict(gu=gu, gs=gs, down=down, ds=ds, gu_d=dev(gu), down_d=dev(down))


def gpu_route(zq, logits, g, top_k=TOP_K):
    torch = torch_cuda()
    n = logits.size
    m = top_k + (1 if g is not None else 0)
    ids = sentinel_i32(m)
    wts = nan_f32(m)
    gd = None if g is None else dev(np.array([g], np.float32))
    zq.zq_moe_route(dev(logits), n, top_k, gd, ids, wts)
    torch.cuda.synchronize()
    return host(ids), host(wts)


def test_route_against_oracle(zq):
    for s in range(12):
        logits, g = inputs.gen_router(E_ROUTED, inputs.seed_for(4, s))
        if s == 5:
            logits[[3, 9, 70]] = logits.max() + 1.0  # a tie at the top
        ids, wts = gpu_route(zq, logits, g)
        rids, rw = oracle.moe_route(logits, TOP_K, g)
        assert np.array_equal(ids, rids)
        assert np.allclose(wts.astype(np.float64), rw, rtol=1e-6, atol=0)
    ids, wts = gpu_route(zq, np.zeros(E_ROUTED, np.float32), None)
    assert list(ids) == list(range(TOP_K)) and (wts == 0.125).all()
    # larger routers up to the documented limit
    logits = np.random.default_rng(1).standard_normal(1024).astype(np.float32)
    ids, wts = gpu_route(zq, logits, np.float32(0.25), top_k=64)
    rids, rw = oracle.moe_route(logits, 64, np.float32(0.25))
    assert np.array_equal(ids, rids) and np.allclose(wts, rw, rtol=1e-6, atol=0)


def run_chain(zq, banks, seed):
    """Route -> fused gate/up (+ swiglu + re-quantize) -> weighted down, each
    stage checked against the oracle on the GPU's previous output."""
    torch = torch_cuda()
    logits, g = inputs.gen_router(E_ROUTED, seed)
    x = inputs.gen_activation(1, D_MODEL, seed + 7)
    ids, wts = gpu_route(zq, logits, g)
    rids, rw = oracle.moe_route(logits, TOP_K, g)
    assert np.array_equal(ids, rids)
    n_sel = ids.size
    ids_d, wts_d = dev(ids), dev(wts)
    rq, rd, _ = oracle.quantize_act(x)

    qh = torch.zeros((n_sel, D_FF), dtype=torch.int8, device="cuda")
    dh = nan_f32(n_sel, D_FF // 32)
    sh = sentinel_i32(n_sel, D_FF // 32)
    h = nan_f32(n_sel, D_FF)
    gu = nan_f32(n_sel, 2 * D_FF)
    status = sentinel_i32(1, value=0)
    zq.zq_moe_gate_up(Q4, banks["gu_d"], banks["gs"], N_EXPERTS, D_MODEL, D_FF, ids_d, n_sel,
                      dev(x), qh, dh, sh, h, gu, status)
    gu_h = host(gu)
    gu_ref, gu_S = oracle.moe_gate_up(Q4, banks["gu"], banks["gs"], D_MODEL, D_FF, ids, rq, rd)
    check_rows(gu_h, gu_ref, gu_S, "moe fused gate/up rows")
    h_h = host(h)
    h_ref = oracle.swiglu(gu_h, D_FF)  # on the GPU's own gate/up rows
    assert np.allclose(h_h, h_ref, rtol=1e-6, atol=0)
    rqh, rdh, rsh = oracle.quantize_act(h_h)  # same fp32 h -> bit-exact codes
    assert np.array_equal(host(qh), rqh)
    assert np.array_equal(host(dh).view(np.uint32), rdh.view(np.uint32))
    assert np.array_equal(host(sh), rsh)

    y = nan_f32(D_MODEL)
    zq.zq_dmmv_moe(Q4, banks["down_d"], N_EXPERTS, banks["ds"], D_MODEL, D_FF, ids_d, wts_d, n_sel,
                   qh, dh, sh, D_FF, 1, y, 0, status)
    y_h = host(y)
    y_ref, S = oracle.moe_down_weighted(Q4, banks["down"], banks["ds"], D_MODEL, D_FF, ids,
                                       wts.astype(np.float64), rqh, rdh)
    check_rows(y_h, y_ref, S, "moe weighted down")
    assert int(host(status)[0]) == 0
    return dict(x=x, ids=ids, wts=wts, ids_d=ids_d, wts_d=wts_d, y=y_h, rw=rw)


def test_moe_gather_and_swiglu_kernels(zq, banks):
    """The standalone expert gather DMMV and swiglu + quantize kernels."""
    torch = torch_cuda()
    logits, g = inputs.gen_router(E_ROUTED, 4321)
    ids, _ = oracle.moe_route(logits, TOP_K, g)
    n_sel = ids.size
    x = inputs.gen_activation(1, D_MODEL, 4322)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    gu = nan_f32(n_sel, 2 * D_FF)
    zq.zq_dmmv_moe(Q4, banks["gu_d"], N_EXPERTS, banks["gs"], 2 * D_FF, D_MODEL, dev(ids), None,
                   n_sel, qx, dx, sx, 0, 0, gu)
    gu_h = host(gu)
    gu_ref, gu_S = oracle.moe_gate_up(Q4, banks["gu"], banks["gs"], D_MODEL, D_FF, ids, rq, rd)
    check_rows(gu_h, gu_ref, gu_S, "moe gather")
    qh = torch.zeros((n_sel, D_FF), dtype=torch.int8, device="cuda")
    dh = nan_f32(n_sel, D_FF // 32)
    sh = sentinel_i32(n_sel, D_FF // 32)
    h = nan_f32(n_sel, D_FF)
    zq.zq_swiglu_quantize(gu, n_sel, D_FF, qh, dh, sh, h)
    h_h = host(h)
    assert np.allclose(h_h, oracle.swiglu(gu_h, D_FF), rtol=1e-6, atol=0)
    rqh, rdh, rsh = oracle.quantize_act(h_h)
    assert np.array_equal(host(qh), rqh) and np.array_equal(host(dh), rdh)
    assert np.array_equal(host(sh), rsh)


@pytest.mark.parametrize("s", [0, 1, 2])
def test_moe_chain_and_composite(zq, banks, s):
    torch = torch_cuda()
    c = run_chain(zq, banks, inputs.seed_for(4, s))
    n_sel = c["ids"].size
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(D_MODEL, D_FF, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = nan_f32(D_MODEL)
    zq.zq_moe_ffn(Q4, banks["gu_d"], banks["gs"], banks["down_d"], banks["ds"], N_EXPERTS, D_MODEL,
                  D_FF, c["ids_d"], c["wts_d"], n_sel, dev(c["x"]), ws, ws_bytes, y)
    # the composite runs the same kernels in the same order: identical bits
    assert np.array_equal(host(y).view(np.uint32), c["y"].view(np.uint32))
    # unchained end to end against the oracle with its own routing weights
    y_e2e, S = oracle.moe_ffn(Q4, banks["gu"], banks["gs"], banks["down"], banks["ds"], D_MODEL,
                              D_FF, c["ids"], c["rw"], c["x"])
    check_rows(host(y), y_e2e, S, "moe end to end", tol=1e-3)
    # accumulate: y += again
    prev = host(y).copy()
    zq.zq_moe_ffn(Q4, banks["gu_d"], banks["gs"], banks["down_d"], banks["ds"], N_EXPERTS, D_MODEL,
                  D_FF, c["ids_d"], c["wts_d"], n_sel, dev(c["x"]), ws, ws_bytes, y, 1)
    assert np.allclose(host(y), 2 * prev, rtol=1e-6, atol=0)


@pytest.mark.parametrize("d_model,d_ff,n_sel", [(5120, 64, 3), (256, 96, 17), (64, 32, 1)])
def test_moe_ffn_other_shapes(zq, d_model, d_ff, n_sel):
    """A model wider than the fused gate/up kernel takes (the separate
    quantize / gather / swiglu path), more than 16 selected experts (two
    chunks of down windows), and the smallest shapes."""
    torch = torch_cuda()
    E = n_sel + 2
    gu, gs, down, ds = inputs.moe_banks(777 + d_model, E, d_model, d_ff)
    ids = np.random.default_rng(d_ff).permutation(E)[:n_sel].astype(np.int32)
    wts = np.random.default_rng(d_ff + 1).uniform(0.1, 1.0, n_sel).astype(np.float32)
    x = inputs.gen_activation(1, d_model, 778)
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = nan_f32(d_model)
    zq.zq_moe_ffn(Q4, dev(gu), gs, dev(down), ds, E, d_model, d_ff, dev(ids), dev(wts), n_sel,
                  dev(x), ws, ws_bytes, y)
    y_ref, S = oracle.moe_ffn(Q4, gu, gs, down, ds, d_model, d_ff, ids, wts.astype(np.float64), x)
    check_rows(host(y), y_ref, S, "moe %dx%d n_sel=%d" % (d_model, d_ff, n_sel), tol=1e-3)


def test_moe_bad_expert_id_is_skipped_and_reported(zq, banks):
    qx, dx, sx = quantize_gpu(zq, inputs.gen_activation(1, D_FF, 3))
    qh = qx.repeat(3, 1).contiguous()
    dh = dx.repeat(3, 1).contiguous()
    sh = sx.repeat(3, 1).contiguous()
    ids = np.array([5, 999, 7], np.int32)
    wts = np.array([0.5, 0.25, 0.25], np.float32)
    status = sentinel_i32(1, value=0)
    y = nan_f32(D_MODEL)
    zq.zq_dmmv_moe(Q4, banks["down_d"], N_EXPERTS, banks["ds"], D_MODEL, D_FF, dev(ids), dev(wts), 3,
                   qh, dh, sh, D_FF, 1, y, 0, status)
    assert int(host(status)[0]) == -4  # ZQ_ERANGE
    rq, rd, _ = oracle.quantize_act(inputs.gen_activation(1, D_FF, 3))
    y_ref, S = oracle.moe_down_weighted(Q4, banks["down"], banks["ds"], D_MODEL, D_FF, [5, 7],
                                        [0.5, 0.25], np.stack([rq, rq]), np.stack([rd, rd]))
    check_rows(host(y), y_ref, S, "bad id skipped")
    # gather: the bad slot's output block is left untouched
    gu = nan_f32(3, D_MODEL)
    status2 = sentinel_i32(1, value=0)
    zq.zq_dmmv_moe(Q4, banks["down_d"], N_EXPERTS, banks["ds"], D_MODEL, D_FF, dev(ids), None, 3,
                   qh, dh, sh, D_FF, 0, gu, 0, status2)
    g = host(gu)
    assert np.isnan(g[1]).all() and not np.isnan(g[0]).any() and not np.isnan(g[2]).any()
    assert int(host(status2)[0]) == -4


def test_moe_no_selected_expert(zq, banks):
    torch = torch_cuda()
    y = nan_f32(D_MODEL)
    ids = sentinel_i32(1, value=0)
    wts = nan_f32(1)
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(D_MODEL, D_FF, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    zq.zq_moe_ffn(Q4, banks["gu_d"], banks["gs"], banks["down_d"], banks["ds"], N_EXPERTS, D_MODEL,
                  D_FF, ids, wts, 0, dev(np.zeros(D_MODEL, np.float32)), ws, ws_bytes, y)
    assert (host(y) == 0).all()


# ------------------------------------------------ router folded in ---------

def routed_ffn(zq, gu_d, gs, down_d, ds, n_experts, d_model, d_ff, logits, top_k, g, x, y=None,
               flags=0):
    torch = torch_cuda()
    n_routed = logits.size
    n_sel = top_k + (1 if g is not None else 0)
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ids = sentinel_i32(n_sel)
    wts = nan_f32(n_sel)
    y = nan_f32(d_model) if y is None else y
    gd = None if g is None else dev(np.array([g], np.float32))
    zq.zq_moe_ffn_route(Q4, gu_d, gs, down_d, ds, n_experts, d_model, d_ff, dev(logits), n_routed,
                        top_k, gd, dev(x), ids, wts, ws, ws_bytes, y, flags)
    return host(ids), host(wts), y


def unfused_ffn(zq, gu_d, gs, down_d, ds, n_experts, d_model, d_ff, logits, top_k, g, x):
    torch = torch_cuda()
    ids, wts = gpu_route(zq, logits, g, top_k=top_k)
    n_sel = ids.size
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = nan_f32(d_model)
    zq.zq_moe_ffn(Q4, gu_d, gs, down_d, ds, n_experts, d_model, d_ff, dev(ids), dev(wts), n_sel,
                  dev(x), ws, ws_bytes, y)
    return ids, wts, host(y)


@pytest.mark.parametrize("s", [0, 1, 2, 3])
def test_moe_ffn_route_equals_route_then_ffn(zq, banks, s):
    """Two launches give the router's ids and weights and the composite's
    rows, bit for bit; seed 3 puts a three-way tie at the top."""
    logits, g = inputs.gen_router(E_ROUTED, inputs.seed_for(4, 10 + s))
    if s == 3:
        logits[[3, 9, 70]] = logits.max() + 1.0
    x = inputs.gen_activation(1, D_MODEL, inputs.seed_for(4, 10 + s) + 7)
    args = (banks["gu_d"], banks["gs"], banks["down_d"], banks["ds"], N_EXPERTS, D_MODEL, D_FF,
            logits, TOP_K, g, x)
    ids, wts, y = routed_ffn(zq, *args)
    rids, rwts, ry = unfused_ffn(zq, *args)
    assert np.array_equal(ids, rids)
    assert np.array_equal(wts.view(np.uint32), rwts.view(np.uint32))
    assert np.array_equal(host(y).view(np.uint32), ry.view(np.uint32))
    oids, _ = oracle.moe_route(logits, TOP_K, g)
    assert np.array_equal(ids, oids)
    # accumulate
    prev = host(y).copy()
    routed_ffn(zq, *args, y=y, flags=1)
    assert np.allclose(host(y), 2 * prev, rtol=1e-6, atol=0)


@pytest.mark.parametrize("d_model,d_ff,n_routed,top_k,shared", [
    (64, 32, 200, 17, True),      # 18 selected: two chunks of down windows
    (256, 96, 1024, 64, False),   # the router's limits, no shared expert
    (5120, 64, 40, 3, True),      # wider than the fused gate/up: router launch + unfused path
])
def test_moe_ffn_route_other_shapes(zq, d_model, d_ff, n_routed, top_k, shared):
    E = n_routed + (1 if shared else 0)
    gu, gs, down, ds = inputs.moe_banks(4242 + d_model + top_k, E, d_model, d_ff)
    rng = np.random.default_rng(n_routed + top_k)
    logits = rng.standard_normal(n_routed).astype(np.float32)
    g = np.float32(rng.standard_normal()) if shared else None
    x = inputs.gen_activation(1, d_model, 4243 + d_ff)
    args = (dev(gu), gs, dev(down), ds, E, d_model, d_ff, logits, top_k, g, x)
    ids, wts, y = routed_ffn(zq, *args)
    rids, rwts, ry = unfused_ffn(zq, *args)
    assert np.array_equal(ids, rids)
    assert np.array_equal(wts.view(np.uint32), rwts.view(np.uint32))
    assert np.array_equal(host(y).view(np.uint32), ry.view(np.uint32))
    oids, ow = oracle.moe_route(logits, top_k, g)
    assert np.array_equal(ids, oids)
    y_ref, S = oracle.moe_ffn(Q4, gu, gs, down, ds, d_model, d_ff, ids, ow, x)
    check_rows(host(y), y_ref, S, "routed moe %dx%d" % (d_model, d_ff), tol=1e-3)


def test_moe_gate_up_route_stage(zq, banks):
    """The routed gate/up stage equals route + zq_moe_gate_up, output by
    output and bit for bit (ids, weights, gate||up rows, h, codes, scales,
    sums)."""
    torch = torch_cuda()
    for s in range(3):
        logits, g = inputs.gen_router(E_ROUTED, inputs.seed_for(4, 20 + s))
        x = inputs.gen_activation(1, D_MODEL, inputs.seed_for(4, 20 + s) + 7)
        n_sel = TOP_K + 1
        outs = []
        for routed in (True, False):
            qh = torch.zeros((n_sel, D_FF), dtype=torch.int8, device="cuda")
            dh = nan_f32(n_sel, D_FF // 32)
            sh = sentinel_i32(n_sel, D_FF // 32)
            h = nan_f32(n_sel, D_FF)
            gu = nan_f32(n_sel, 2 * D_FF)
            if routed:
                ids = sentinel_i32(n_sel)
                wts = nan_f32(n_sel)
                zq.zq_moe_gate_up_route(Q4, banks["gu_d"], banks["gs"], N_EXPERTS, D_MODEL, D_FF,
                                        dev(logits), E_ROUTED, TOP_K, dev(np.array([g], np.float32)),
                                        dev(x), ids, wts, qh, dh, sh, h, gu)
                ids, wts = host(ids), host(wts)
            else:
                ids, wts = gpu_route(zq, logits, g)
                zq.zq_moe_gate_up(Q4, banks["gu_d"], banks["gs"], N_EXPERTS, D_MODEL, D_FF,
                                  dev(ids), n_sel, dev(x), qh, dh, sh, h, gu)
            outs.append([ids, wts.view(np.uint32)] +
                        [host(t).view(np.uint8) for t in (qh, dh, sh, h, gu)])
        for a, b in zip(*outs):
            assert np.array_equal(a, b)


def test_router_nan_logits_fill_every_slot(zq, banks):
    """NaN logits rank below every number (ties by id), so every slot gets a
    distinct expert in range, both in the router launch and inside the
    routed gate/up pass: the selection the oracle makes when every NaN is
    replaced by a number below all the others (the oracle takes finite
    logits only)."""
    logits, g = inputs.gen_router(E_ROUTED, inputs.seed_for(4, 40))
    logits[[0, 5, int(np.argmax(logits)), 77]] = np.nan
    low = np.float32(np.nanmin(logits) - 1000.0)
    clean = np.where(np.isnan(logits), low, logits).astype(np.float32)
    rids, _ = oracle.moe_route(clean, TOP_K, g)
    ids, _ = gpu_route(zq, logits, g)
    assert np.array_equal(ids, rids)
    x = inputs.gen_activation(1, D_MODEL, 41)
    ids2, wts2, y = routed_ffn(zq, banks["gu_d"], banks["gs"], banks["down_d"], banks["ds"],
                               N_EXPERTS, D_MODEL, D_FF, logits, TOP_K, g, x)
    assert np.array_equal(ids2, rids)
    assert np.isfinite(host(y)).all()
    # all logits NaN: still TOP_K distinct experts (ids 0..TOP_K-1) and the
    # shared one; the weights are then undefined
    ids3, _ = gpu_route(zq, np.full(E_ROUTED, np.nan, np.float32), g)
    assert list(ids3) == list(range(TOP_K)) + [E_ROUTED]
