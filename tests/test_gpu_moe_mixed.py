"""GPU parity of the expert-indexed K-quant DMMV and of the MoE block with
experts in the pages' own formats (routed gate/up Q4_K, down Q5_K, shared
expert Q8_0), against the oracle."""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, quantize_gpu, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 4, 8, 12, 13, 14
NAME = {Q4_0: "q4_0", Q8_0: "q8_0", Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k"}


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


def gen_bank(wt, n_experts, rows, k, seed):
    if wt in (Q4_K, Q5_K, Q6_K):
        w = inputs.gen_weights_k(wt, n_experts * rows, k, seed)
        return w, rows * (k // 256) * inputs.K_BLOCK_BYTES[wt]
    w = inputs.gen_weights(wt, n_experts * rows, k, seed)
    return w, rows * (k // 32) * inputs.BLOCK_BYTES[wt]


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K], ids=lambda t: NAME[t])
def test_dmmv_moe_kquant_gather_and_weighted(zq, wt):
    E, rows, k = 6, 96, 512
    bank, stride = gen_bank(wt, E, rows, k, 810 + wt)
    bank_d = dev(bank)
    ids_h = np.array([3, 0, 5, 3], np.int32)
    n = ids_h.size
    wts_h = np.array([0.5, -1.25, 0.125, 2.0], np.float32)
    # gather over one broadcast activation
    x = inputs.gen_activation(1, k, 811)
    qx, dx, sx = quantize_gpu(zq, x)
    rq, rd, _ = oracle.quantize_act(x)
    y = nan_f32(n, rows)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(ids_h), None, n, qx, dx, sx, 0,
                   zq.ZQ_MOE_GATHER, y)
    yh = host(y)
    for s, e in enumerate(ids_h):
        y_ref, S = oracle.expert_rows_any(wt, bank, stride, rows, k, int(e), rq, rd)
        check_rows(yh[s], y_ref, S, "%s gather slot %d" % (NAME[wt], s))
    # weighted sum over per-slot activations
    xs = inputs.gen_activation(n, k, 812)
    qxs, dxs, sxs = quantize_gpu(zq, xs)
    rqs, rds, _ = oracle.quantize_act(xs)
    y2 = nan_f32(rows)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(ids_h), dev(wts_h), n, qxs, dxs, sxs, k,
                   zq.ZQ_MOE_WEIGHTED_SUM, y2)
    y_ref = np.zeros(rows)
    S = np.zeros(rows)
    for s, e in enumerate(ids_h):
        ye, Se = oracle.expert_rows_any(wt, bank, stride, rows, k, int(e), rqs[s], rds[s])
        y_ref += float(wts_h[s]) * ye
        S += abs(float(wts_h[s])) * Se
    check_rows(host(y2), y_ref, S, "%s weighted" % NAME[wt])
    # an id out of range is skipped and reported
    status = sentinel_i32(1, value=0)
    bad = dev(np.array([3, 9, 0], np.int32))
    y3 = nan_f32(3, rows)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, bad, None, 3, qx, dx, sx, 0, zq.ZQ_MOE_GATHER,
                   y3, 0, status)
    y3h = host(y3)
    assert int(host(status)[0]) == zq.ZQ_ERANGE
    assert np.isnan(y3h[1]).all() and not np.isnan(y3h[0]).any() and not np.isnan(y3h[2]).any()


def gen_bank_padded(wt, n_experts, rows, k, seed):
    """Experts at a stride rounded up to 16 bytes (the K-quant bank
    alignment), padding filled with 0xFF bytes that no kernel may read."""
    w, m = gen_bank(wt, n_experts, rows, k, seed)
    stride = (m + 15) // 16 * 16
    out = np.full(n_experts * stride, 0xFF, np.uint8)
    for e in range(n_experts):
        out[e * stride:e * stride + m] = w.reshape(-1)[e * m:(e + 1) * m]
    return out, stride


def weighted_ref(wt, bank, stride, rows, k, ids, wts, rqs, rds, n_experts):
    y_ref, S = np.zeros(rows), np.zeros(rows)
    for s, e in enumerate(ids):
        if not 0 <= e < n_experts:
            continue
        ye, Se = oracle.expert_rows_any(wt, bank, stride, rows, k, int(e), rqs[s], rds[s])
        y_ref += float(wts[s]) * ye
        S += abs(float(wts[s])) * Se
    return y_ref, S


# K-quants: k = 256 .. 2048 take the slots-in-lanes kernel (16 .. 2 slots
# per round; 17 and 5 slots need a second and third round); 768 the
# per-slot loop.  Q4_0 / Q8_0: k = 256, 512 (4 lanes per slot, 2 and 4
# blocks per lane; 17 slots take two rounds), 768 and 1024 (8 lanes per
# slot, 3 and 4 blocks) take the slots-in-lanes kernel, 2048 the staged
# kernel.  rows: ragged against 1, 2 and 4 row steps per wave.
@pytest.mark.parametrize("wt", [Q4_0, Q8_0, Q4_K, Q5_K, Q6_K], ids=lambda t: NAME[t])
@pytest.mark.parametrize("rows,k,n_sel", [(4097, 256, 17), (2051, 512, 9), (333, 1024, 8),
                                          (130, 2048, 5), (77, 768, 3)])
def test_dmmv_moe_weighted_layouts(zq, wt, rows, k, n_sel):
    E = 7
    bank, stride = gen_bank_padded(wt, E, rows, k, 820 + wt + k)
    bank_d = dev(bank)
    rng = np.random.default_rng(821 + n_sel)
    ids_h = rng.integers(0, E, n_sel).astype(np.int32)
    wts_h = rng.standard_normal(n_sel).astype(np.float32)
    xs = inputs.gen_activation(n_sel, k, 822 + k)
    qxs, dxs, sxs = quantize_gpu(zq, xs)
    rqs, rds, _ = oracle.quantize_act(xs)
    y = nan_f32(rows)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(ids_h), dev(wts_h), n_sel, qxs, dxs, sxs, k,
                   zq.ZQ_MOE_WEIGHTED_SUM, y)
    y_ref, S = weighted_ref(wt, bank, stride, rows, k, ids_h, wts_h, rqs, rds, E)
    check_rows(host(y), y_ref, S, "%s weighted %d x %d, %d slots" % (NAME[wt], rows, k, n_sel))
    # accumulate onto y; an out-of-range id in the middle is skipped and reported
    prev = np.random.default_rng(5).standard_normal(rows).astype(np.float32)
    y2 = dev(prev)
    bad = ids_h.copy()
    bad[n_sel // 2] = E + 3
    status = sentinel_i32(1, value=0)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(bad), dev(wts_h), n_sel, qxs, dxs, sxs, k,
                   zq.ZQ_MOE_WEIGHTED_SUM, y2, zq.ZQ_ACCUMULATE, status)
    assert int(host(status)[0]) == zq.ZQ_ERANGE
    y_ref2, S2 = weighted_ref(wt, bank, stride, rows, k, bad, wts_h, rqs, rds, E)
    check_rows(host(y2), prev.astype(np.float64) + y_ref2, S2 + np.abs(prev),
               "%s weighted accumulate, bad id" % NAME[wt])
    if wt == Q4_0:
        # without block sums the kernel sums the codes itself: the same bits
        y4 = nan_f32(rows)
        zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(ids_h), dev(wts_h), n_sel, qxs, dxs,
                       None, k, zq.ZQ_MOE_WEIGHTED_SUM, y4)
        assert np.array_equal(host(y4).view(np.uint32), host(y).view(np.uint32))
    # no selected expert: zeros
    y3 = nan_f32(rows)
    zq.zq_dmmv_moe(wt, bank_d, E, stride, rows, k, dev(ids_h), dev(wts_h), 0, qxs, dxs, sxs, k,
                   zq.ZQ_MOE_WEIGHTED_SUM, y3)
    assert (host(y3) == 0).all()


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K], ids=lambda t: NAME[t])
@pytest.mark.parametrize("d_model,d_ff", [(1024, 256), (2048, 512), (4096, 96)])
def test_moe_gate_up_kquant(zq, wt, d_model, d_ff):
    """The fused K-quant gate/up pass, chained: gate||up rows against the
    oracle's expert rows, h against SwiGLU of the GPU's own rows, the codes
    bit-exact against the oracle's quantization of the GPU's h."""
    torch = torch_cuda()
    E = 5
    bank, stride = gen_bank(wt, E, 2 * d_ff, d_model, 860 + wt + d_model)
    ids = np.array([4, 0, 4, 2], np.int32)
    n = ids.size
    x = inputs.gen_activation(1, d_model, 861 + d_model)
    rq, rd, _ = oracle.quantize_act(x)
    qh = torch.full((n, d_ff), 0x55, dtype=torch.int8, device="cuda")
    dh, sh = nan_f32(n, d_ff // 32), sentinel_i32(n, d_ff // 32)
    h, gu = nan_f32(n, d_ff), nan_f32(n, 2 * d_ff)
    status = sentinel_i32(1, value=0)
    assert zq.zq_moe_gate_up(wt, dev(bank), stride, E, d_model, d_ff, dev(ids), n, dev(x), qh, dh,
                             sh, h, gu, status) == 0
    gu_h = host(gu)
    for s, e in enumerate(ids):
        y_ref, S = oracle.expert_rows_any(wt, bank, stride, 2 * d_ff, d_model, int(e), rq, rd)
        check_rows(gu_h[s], y_ref, S, "%s gate/up slot %d, %d -> %d" % (NAME[wt], s, d_model, d_ff))
    h_h = host(h)
    assert np.allclose(h_h, oracle.swiglu(gu_h, d_ff), rtol=1e-6, atol=0)
    rqh, rdh, rsh = oracle.quantize_act(h_h)
    assert np.array_equal(host(qh), rqh)
    assert np.array_equal(host(dh).view(np.uint32), rdh.view(np.uint32))
    assert np.array_equal(host(sh), rsh)
    assert int(host(status)[0]) == 0
    # slots of one expert give the same bits; without the debug outputs too
    assert np.array_equal(gu_h[0].view(np.uint32), gu_h[2].view(np.uint32))
    qh2 = torch.zeros((n, d_ff), dtype=torch.int8, device="cuda")
    dh2 = nan_f32(n, d_ff // 32)
    zq.zq_moe_gate_up(wt, dev(bank), stride, E, d_model, d_ff, dev(ids), n, dev(x), qh2, dh2)
    assert np.array_equal(host(qh2), host(qh))
    assert np.array_equal(host(dh2).view(np.uint32), host(dh).view(np.uint32))


@pytest.mark.parametrize("wt", [Q4_K, Q6_K], ids=lambda t: NAME[t])
def test_moe_gate_up_kquant_bad_id_and_route(zq, wt):
    """A bad expert id is skipped and reported; the routed form equals the
    router followed by the plain pass, output by output."""
    torch = torch_cuda()
    d_model, d_ff, n_routed, top_k = 2048, 256, 16, 4
    bank, stride = gen_bank(wt, n_routed + 1, 2 * d_ff, d_model, 870 + wt)
    bank_d = dev(bank)
    x = dev(inputs.gen_activation(1, d_model, 871))
    status = sentinel_i32(1, value=0)
    qh = torch.full((3, d_ff), 0x55, dtype=torch.int8, device="cuda")
    dh = nan_f32(3, d_ff // 32)
    zq.zq_moe_gate_up(wt, bank_d, stride, n_routed + 1, d_model, d_ff,
                      dev(np.array([1, 17, 3], np.int32)), 3, x, qh, dh, None, None, None, status)
    assert int(host(status)[0]) == zq.ZQ_ERANGE
    dhh = host(dh)
    assert np.isnan(dhh[1]).all() and not np.isnan(dhh[0]).any() and not np.isnan(dhh[2]).any()
    assert (host(qh)[1] == 0x55).all()

    logits, g = inputs.gen_router(n_routed, 872)
    gd = dev(np.array([g], np.float32))
    n_sel = top_k + 1
    outs = []
    for routed in (True, False):
        ids, wts = sentinel_i32(n_sel), nan_f32(n_sel)
        qh = torch.empty((n_sel, d_ff), dtype=torch.int8, device="cuda")
        dh, sh = nan_f32(n_sel, d_ff // 32), sentinel_i32(n_sel, d_ff // 32)
        gu = nan_f32(n_sel, 2 * d_ff)
        if routed:
            zq.zq_moe_gate_up_route(wt, bank_d, stride, n_routed + 1, d_model, d_ff, dev(logits),
                                    n_routed, top_k, gd, x, ids, wts, qh, dh, sh, None, gu)
        else:
            zq.zq_moe_route(dev(logits), n_routed, top_k, gd, ids, wts)
            zq.zq_moe_gate_up(wt, bank_d, stride, n_routed + 1, d_model, d_ff, ids, n_sel, x, qh,
                              dh, sh, None, gu)
        outs.append([host(t).copy() for t in (ids, wts, qh, dh, sh, gu)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert outs[0][0][top_k] == n_routed


def run_mixed(zq, fmt, banks, d_model, d_ff, n_routed, top_k, logits, g, x, y=None, flags=0):
    torch = torch_cuda()
    (gwt, gu_d, gs), (dwt, dn_d, ds), (swt, sgu_d, sdn_d) = banks
    n_sel = top_k + (1 if g is not None else 0)
    ws_bytes = zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ids, wts = sentinel_i32(n_sel), nan_f32(n_sel)
    y = nan_f32(d_model) if y is None else y
    gd = None if g is None else dev(np.array([g], np.float32))
    zq.zq_moe_ffn_mixed(gwt, gu_d, gs, dwt, dn_d, ds, swt, sgu_d, sdn_d, d_model, d_ff, dev(logits),
                        n_routed, top_k, gd, dev(x), ids, wts, ws, ws_bytes, y, flags)
    return host(ids), host(wts), y


def make_banks(fmt, n_routed, d_model, d_ff, seed):
    gwt, dwt, swt = fmt
    gu, gs = gen_bank(gwt, n_routed, 2 * d_ff, d_model, seed)
    dn, ds = gen_bank(dwt, n_routed, d_model, d_ff, seed + 1)
    sgu, _ = gen_bank(swt, 1, 2 * d_ff, d_model, seed + 2)
    sdn, _ = gen_bank(swt, 1, d_model, d_ff, seed + 3)
    host_b = ((gwt, gu, gs), (dwt, dn, ds), (swt, sgu, sdn))
    dev_b = ((gwt, dev(gu), gs), (dwt, dev(dn), ds), (swt, dev(sgu), dev(sdn)))
    return host_b, dev_b


def oracle_mixed(host_b, n_routed, d_model, d_ff, ids, wts, x):
    (gwt, gu, gs), (dwt, dn, ds), (swt, sgu, sdn) = host_b
    return oracle.moe_ffn_mixed(gwt, gu, gs, dwt, dn, ds, swt, sgu, sdn, n_routed, d_model, d_ff,
                                ids, wts, x)


PAGES = (Q4_K, Q5_K, Q8_0)


@pytest.mark.parametrize("fmt", [PAGES, (Q4_0, Q4_0, Q8_0), (Q6_K, Q4_K, Q4_0), (Q5_K, Q6_K, Q4_K),
                                 (Q8_0, Q4_K, Q6_K)],
                         ids=lambda f: "-".join(NAME[t] for t in f))
@pytest.mark.parametrize("d_model", [512, 1024, 2048, 4096])
# 512: the staged path; 1024 / 2048: routed and shared gate/up in one launch;
# 4096: the routed pass and the shared pass in two launches.  The down pass
# folds a block-format shared expert into K-quant routed rows.
def test_moe_ffn_mixed_small(zq, fmt, d_model):
    d_ff, n_routed, top_k = 256, 16, 4
    host_b, dev_b = make_banks(fmt, n_routed, d_model, d_ff, 830 + sum(fmt))
    logits, g = inputs.gen_router(n_routed, 831)
    x = inputs.gen_activation(1, d_model, 832)
    ids, wts, y = run_mixed(zq, fmt, dev_b, d_model, d_ff, n_routed, top_k, logits, g, x)
    rids, _ = oracle.moe_route(logits, top_k, g)
    assert np.array_equal(ids, rids)
    y_ref, S = oracle_mixed(host_b, n_routed, d_model, d_ff, ids, wts, x)
    check_rows(host(y), y_ref, S, "mixed moe %s" % (fmt,), tol=1e-3)
    # accumulate onto y
    prev = host(y).copy()
    run_mixed(zq, fmt, dev_b, d_model, d_ff, n_routed, top_k, logits, g, x, y=y, flags=1)
    assert np.allclose(host(y), 2 * prev, rtol=1e-6, atol=0)


@pytest.mark.parametrize("d_model", [512, 2048])
def test_moe_ffn_mixed_equals_its_stages(zq, d_model):
    """The composite against the same stages run through the public entry
    points one by one.  d_model 512: router, quantize, routed and shared
    gate||up gathers, SwiGLU + re-quantize; 2048: router, routed and shared
    zq_moe_gate_up (the composite runs both in one launch, with the same
    arithmetic); then the routed and the shared down stages, which the
    composite folds into one reduction.  The expert list and weights bit for
    bit; y within 1e-5 of the oracle's scale S (two summation orders of the
    same terms on the same h codes)."""
    torch = torch_cuda()
    d_ff, n_routed, top_k = 256, 16, 4
    host_b, dev_b = make_banks(PAGES, n_routed, d_model, d_ff, 840)
    (gwt, gu_d, gs), (dwt, dn_d, ds), (swt, sgu_d, sdn_d) = dev_b
    logits, g = inputs.gen_router(n_routed, 841)
    x = inputs.gen_activation(1, d_model, 842)
    ids, wts, y = run_mixed(zq, PAGES, dev_b, d_model, d_ff, n_routed, top_k, logits, g, x)
    n_sel = top_k + 1
    ids_d, wts_d = sentinel_i32(n_sel), nan_f32(n_sel)
    zq.zq_moe_route(dev(logits), n_routed, top_k, dev(np.array([g], np.float32)), ids_d, wts_d)
    zero = dev(np.zeros(1, np.int32))
    sgu_bytes, sdn_bytes = sgu_d.numel(), sdn_d.numel()   # one expert: stride = its size
    qh = torch.empty((n_sel, d_ff), dtype=torch.int8, device="cuda")
    dh, sh = nan_f32(n_sel, d_ff // 32), sentinel_i32(n_sel, d_ff // 32)
    if d_model == 512:
        qx, dx, sx = quantize_gpu(zq, x)
        gu = nan_f32(n_sel, 2 * d_ff)
        zq.zq_dmmv_moe(gwt, gu_d, n_routed, gs, 2 * d_ff, d_model, ids_d, None, top_k, qx, dx, sx,
                       0, zq.ZQ_MOE_GATHER, gu)
        zq.zq_dmmv_moe(swt, sgu_d, 1, sgu_bytes, 2 * d_ff, d_model, zero, None, 1, qx, dx, sx, 0,
                       zq.ZQ_MOE_GATHER, gu[top_k:])
        zq.zq_swiglu_quantize(gu, n_sel, d_ff, qh, dh, sh)
    else:
        xd = dev(x)
        zq.zq_moe_gate_up(gwt, gu_d, gs, n_routed, d_model, d_ff, ids_d, top_k, xd, qh, dh, sh)
        zq.zq_moe_gate_up(swt, sgu_d, sgu_bytes, 1, d_model, d_ff, zero, 1, xd, qh[top_k:],
                          dh[top_k:], sh[top_k:])
        # the composite's one-launch stage gives the same bits
        ids_m, wts_m = sentinel_i32(n_sel), nan_f32(n_sel)
        qh_m = torch.empty((n_sel, d_ff), dtype=torch.int8, device="cuda")
        dh_m, sh_m = nan_f32(n_sel, d_ff // 32), sentinel_i32(n_sel, d_ff // 32)
        zq.zq_moe_gate_up_mixed(gwt, gu_d, gs, swt, sgu_d, d_model, d_ff, dev(logits), n_routed,
                                top_k, dev(np.array([g], np.float32)), xd, ids_m, wts_m, qh_m,
                                dh_m, sh_m)
        for a_, b_ in ((ids_m, ids_d), (wts_m, wts_d), (qh_m, qh), (dh_m, dh), (sh_m, sh)):
            assert np.array_equal(host(a_).view(np.uint8), host(b_).view(np.uint8))
    y2 = nan_f32(d_model)
    zq.zq_dmmv_moe(dwt, dn_d, n_routed, ds, d_model, d_ff, ids_d, wts_d, top_k, qh, dh, sh, d_ff,
                   zq.ZQ_MOE_WEIGHTED_SUM, y2)
    zq.zq_dmmv_moe(swt, sdn_d, 1, sdn_bytes, d_model, d_ff, zero, wts_d[top_k:], 1, qh[top_k:],
                   dh[top_k:], sh[top_k:], d_ff, zq.ZQ_MOE_WEIGHTED_SUM, y2, zq.ZQ_ACCUMULATE)
    assert np.array_equal(host(ids_d), ids)
    assert np.array_equal(host(wts_d).view(np.uint32), wts.view(np.uint32))
    _, S = oracle_mixed(host_b, n_routed, d_model, d_ff, ids, wts, x)
    check_rows(host(y), host(y2).astype(np.float64), S, "fused down vs stages", tol=1e-5)


def test_moe_ffn_mixed_pages_shape(zq):
    """The pages' expert shapes: 128 routed experts of 2048 -> 512 -> 2048 in
    Q4_K / Q5_K, top-8, a Q8_0 shared expert."""
    d_model, d_ff, n_routed, top_k = 2048, 512, 128, 8
    host_b, dev_b = make_banks(PAGES, n_routed, d_model, d_ff, 850)
    for s in range(2):
        logits, g = inputs.gen_router(n_routed, 851 + s)
        x = inputs.gen_activation(1, d_model, 853 + s)
        ids, wts, y = run_mixed(zq, PAGES, dev_b, d_model, d_ff, n_routed, top_k, logits, g, x)
        assert np.array_equal(ids, oracle.moe_route(logits, top_k, g)[0])
        y_ref, S = oracle_mixed(host_b, n_routed, d_model, d_ff, ids, wts, x)
        check_rows(host(y), y_ref, S, "pages-format moe", tol=1e-3)


@pytest.mark.parametrize("fmt", [PAGES, (Q5_K, Q6_K, Q8_0)],
                         ids=lambda f: "-".join(NAME[t] for t in f))
def test_moe_ffn_mixed_no_shared_expert(zq, fmt):
    """Without a shared gate: top_k routed slots only, on the fused pass."""
    d_model, d_ff, n_routed, top_k = 4096, 256, 32, 6
    host_b, dev_b = make_banks(fmt, n_routed, d_model, d_ff, 880 + sum(fmt))
    logits, _ = inputs.gen_router(n_routed, 881)
    x = inputs.gen_activation(1, d_model, 882)
    ids, wts, y = run_mixed(zq, fmt, dev_b, d_model, d_ff, n_routed, top_k, logits, None, x)
    rids, rw = oracle.moe_route(logits, top_k, None)
    assert np.array_equal(ids, rids) and ids.size == top_k
    assert np.allclose(wts, rw, rtol=1e-6, atol=0)
    y_ref, S = oracle_mixed(host_b, n_routed, d_model, d_ff, ids, wts, x)
    check_rows(host(y), y_ref, S, "mixed moe without shared expert", tol=1e-3)
