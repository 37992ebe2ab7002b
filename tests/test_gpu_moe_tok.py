"""GPU parity of the several-token MoE block (zq_moe_ffn_tokens): 1..8
tokens, each with its own router logits, through one pass over the union of
their experts.

Per token, against the oracle:
  - the router: ids exactly, weights within 1e-6 (and bit for bit those of
    zq_moe_route on the same logits);
  - chained: the down rows and weighted sum against the oracle's on the
    single-token gate/up stage's codes of that token (zq_moe_gate_up with the
    same ids, whose codes the several-token gate/up reproduces bit for bit),
    at the row bar;
  - unchained: the whole block against the oracle's composition from x at
    the end-to-end MoE bar (an exp ulp may flip one re-quantized code).
"""
import numpy as np
import pytest

import oracle
from block_quant_matrix_amd import inputs
from gpuhelp import check_rows, dev, host, nan_f32, sentinel_i32, torch_cuda

pytestmark = pytest.mark.gpu

Q4_0, Q8_0 = 4, 8
MOE_E2E_TOL = 1e-3


@pytest.fixture(scope="module")
def zq():
    torch_cuda()
    from block_quant_matrix_amd import zq as _zq
    assert _zq.zq_device_check(0) == 0
    return _zq


_BANKS = {}


def banks(wt, n_experts, d_model, d_ff, seed):
    key = (wt, n_experts, d_model, d_ff, seed)
    if key not in _BANKS:
        gu, gs, dn, ds = inputs.moe_banks(seed, n_experts, d_model, d_ff, wt)
        _BANKS.clear()
        _BANKS[key] = dict(gu=gu, gs=gs, dn=dn, ds=ds, gu_d=dev(gu), dn_d=dev(dn))
    return _BANKS[key]


def run_tokens(zq, wt, B, n_exp, d_model, d_ff, logits, n_routed, top_k, gates, x, y=None,
               flags=0):
    torch = torch_cuda()
    n_tok = x.shape[0]
    n_sel = top_k + (1 if gates is not None else 0)
    ids = sentinel_i32(n_tok, n_sel)
    wts = nan_f32(n_tok, n_sel)
    ws_bytes = zq.zq_moe_ffn_tokens_workspace_bytes(d_model, d_ff, n_tok, n_sel)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)  # stale bytes: the plan and every stage must overwrite what they read
    xd = dev(x)
    y = nan_f32(n_tok, d_model) if y is None else y
    gd = None if gates is None else dev(np.asarray(gates, np.float32))
    zq.zq_moe_ffn_tokens(wt, B["gu_d"], B["gs"], B["dn_d"], B["ds"], n_exp, d_model, d_ff,
                         dev(logits), n_routed, top_k, gd, xd, n_tok, ids, wts, ws, ws_bytes, y,
                         flags)
    torch.cuda.synchronize()
    return host(ids), host(wts), host(y)


def check_token(zq, wt, B, n_exp, d_model, d_ff, n_routed, top_k, lg, g, xt, ids, wts, y, what):
    """The checks of one token of a several-token call."""
    torch = torch_cuda()
    rids, rw = oracle.moe_route(lg, top_k, g)
    assert np.array_equal(ids, rids), what + " ids"
    assert np.allclose(wts, rw, rtol=1e-6, atol=0), what + " weights"
    # the single-token router gives the same bits
    m = ids.size
    i1, w1 = sentinel_i32(m), nan_f32(m)
    zq.zq_moe_route(dev(lg), n_routed, top_k, None if g is None else dev(np.array([g], np.float32)),
                    i1, w1)
    # the single-token gate/up stage on the same ids: its codes are the
    # several-token stage's, bit for bit
    qh = torch.zeros((m, d_ff), dtype=torch.int8, device="cuda")
    dh = nan_f32(m, d_ff // 32)
    sh = sentinel_i32(m, d_ff // 32)
    zq.zq_moe_gate_up(wt, B["gu_d"], B["gs"], n_exp, d_model, d_ff, dev(ids), m, dev(xt), qh, dh,
                      sh)
    torch.cuda.synchronize()
    assert np.array_equal(host(i1), ids) and np.array_equal(host(w1).view(np.uint32),
                                                            wts.view(np.uint32))
    y_ref, S = oracle.moe_down_weighted(wt, B["dn"], B["ds"], d_model, d_ff, ids,
                                        wts.astype(np.float64), host(qh), host(dh))
    check_rows(y, y_ref, S, what + " chained down + weighted sum")
    y_u, S_u = oracle.moe_ffn(wt, B["gu"], B["gs"], B["dn"], B["ds"], d_model, d_ff, ids, wts, xt)
    check_rows(y, y_u, S_u, what + " unchained block", tol=MOE_E2E_TOL)


# The pages' widths (128 routed experts of 512, top 8, a shared expert) at
# 1, 2, 5 and 8 tokens.
@pytest.mark.parametrize("n_tok", [1, 2, 5, 8])
def test_tokens_pages_shape(zq, n_tok):
    n_routed, top_k, d_model, d_ff = 128, 8, 2048, 512
    B = banks(Q4_0, n_routed + 1, d_model, d_ff, inputs.seed_for(4))
    rng = np.random.default_rng(9300 + n_tok)
    logits = rng.standard_normal((n_tok, n_routed)).astype(np.float32)
    gates = rng.standard_normal(n_tok).astype(np.float32)
    x = inputs.gen_activation(n_tok, d_model, 9310 + n_tok).reshape(n_tok, d_model)
    ids, wts, y = run_tokens(zq, Q4_0, B, n_routed + 1, d_model, d_ff, logits, n_routed, top_k,
                             gates, x)
    for t in range(n_tok):
        check_token(zq, Q4_0, B, n_routed + 1, d_model, d_ff, n_routed, top_k, logits[t],
                    gates[t], x[t], ids[t], wts[t], y[t], "%d tokens, token %d" % (n_tok, t))


def test_tokens_shared_experts_and_accumulate(zq):
    """Tokens with identical logits share every expert (each entry has
    several members); others share none.  Accumulate onto the activation
    itself (y is x): y = x + block(x)."""
    n_routed, top_k, d_model, d_ff = 64, 6, 1024, 256
    B = banks(Q4_0, n_routed + 1, d_model, d_ff, 9400)
    rng = np.random.default_rng(9401)
    base = rng.standard_normal(n_routed).astype(np.float32)
    logits = np.stack([base, base, rng.standard_normal(n_routed).astype(np.float32), base])
    gates = np.array([0.5, -1.0, 0.25, 0.5], np.float32)
    x = inputs.gen_activation(4, d_model, 9402).reshape(4, d_model)
    ids, wts, y = run_tokens(zq, Q4_0, B, n_routed + 1, d_model, d_ff, logits, n_routed, top_k,
                             gates, x)
    assert np.array_equal(ids[0], ids[1]) and np.array_equal(ids[0], ids[3])
    for t in range(4):
        check_token(zq, Q4_0, B, n_routed + 1, d_model, d_ff, n_routed, top_k, logits[t],
                    gates[t], x[t], ids[t], wts[t], y[t], "shared experts, token %d" % t)
    xy = dev(x)
    _, _, y2 = run_tokens(zq, Q4_0, B, n_routed + 1, d_model, d_ff, logits, n_routed, top_k,
                          gates, x, y=xy, flags=1)
    assert np.array_equal(y2.view(np.uint32), (x + y).astype(np.float32).view(np.uint32))


# Q8_0 experts, every d_ff the call takes, no shared expert, top 1, a wide
# router, slots whose hidden codes are too many for the down pass to stage
# in LDS (8 x 17 slots of 1024, and the most slots a call takes: 8 tokens x
# 65), and activations wider than 64 blocks (two blocks per lane in gate/up,
# the second partly past the row at 3072).
@pytest.mark.parametrize("wt,n_routed,top_k,d_model,d_ff,n_tok,shared", [
    (Q8_0, 16, 4, 1024, 256, 3, True),
    (Q8_0, 32, 2, 512, 1024, 8, False),
    (Q4_0, 20, 1, 2048, 2048, 6, True),
    (Q4_0, 1024, 64, 256, 256, 2, True),
    (Q4_0, 64, 16, 512, 1024, 8, True),
    (Q8_0, 256, 64, 256, 256, 8, True),
    (Q4_0, 8, 2, 4096, 512, 3, True),
    (Q8_0, 8, 2, 3072, 256, 2, False),
])
def test_tokens_shapes(zq, wt, n_routed, top_k, d_model, d_ff, n_tok, shared):
    n_exp = n_routed + (1 if shared else 0)
    B = banks(wt, n_exp, d_model, d_ff, 9500 + d_ff + wt)
    rng = np.random.default_rng(9501 + n_routed)
    logits = rng.standard_normal((n_tok, n_routed)).astype(np.float32)
    gates = rng.standard_normal(n_tok).astype(np.float32) if shared else None
    x = inputs.gen_activation(n_tok, d_model, 9502).reshape(n_tok, d_model)
    ids, wts, y = run_tokens(zq, wt, B, n_exp, d_model, d_ff, logits, n_routed, top_k, gates, x)
    for t in range(n_tok):
        check_token(zq, wt, B, n_exp, d_model, d_ff, n_routed, top_k, logits[t],
                    None if gates is None else gates[t], x[t], ids[t], wts[t], y[t],
                    "wt %d d_ff %d token %d" % (wt, d_ff, t))
