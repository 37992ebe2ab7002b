"""HIP graph replay of the per-token decode chain: every replay, with eager
work and synchronizations in between, must give the bits of an eager run
on the same input."""
import numpy as np
import pytest

from block_quant_matrix_amd import inputs
from gpuhelp import dev, host, torch_cuda

pytestmark = pytest.mark.gpu

D_MODEL, N_ROUTED, TOP_K, D_FF, VOCAB, LAYERS = 2048, 16, 4, 512, 4096, 3


@pytest.fixture(scope="module")
def chain():
    torch = torch_cuda()
    from block_quant_matrix_amd import zq
    from block_quant_matrix_amd.chain import DecodeChain
    assert zq.zq_device_check(0) == 0
    router, banks, gates, norms = [], [], [], []
    rng = np.random.default_rng(45)
    for layer in range(LAYERS):
        router.append(dev(inputs.gen_weights(inputs.Q8_0, N_ROUTED, D_MODEL, 40 + layer)))
        gu, gs, dn, ds = inputs.moe_banks(50 + layer, N_ROUTED + 1, D_MODEL, D_FF)
        banks.append((dev(gu), gs, dev(dn), ds, N_ROUTED + 1))
        gates.append(dev(np.array([0.3 * (layer - 1)], np.float32)))
        norms.append(dev((1 + 0.1 * rng.standard_normal(D_MODEL)).astype(np.float32)))
    lm = dev(inputs.gen_weights(inputs.Q4_0, VOCAB, D_MODEL, 60))
    final = dev((1 + 0.1 * rng.standard_normal(D_MODEL)).astype(np.float32))
    return DecodeChain(torch, router, banks, lm, norms, final, d_model=D_MODEL, n_routed=N_ROUTED,
                       top_k=TOP_K, d_ff=D_FF, vocab=VOCAB, shared_gate=gates)


def outputs(c):
    return host(c.x).copy(), host(c.y_lm).copy(), int(host(c.idx)[0]), host(c.ids).copy()


def run_eager(torch, c, x0):
    c.x.copy_(x0)
    c.step()
    torch.cuda.synchronize()
    return outputs(c)


def run_graph(torch, c, x0):
    c.x.copy_(x0)
    c.replay()
    torch.cuda.synchronize()
    return outputs(c)


def same(a, b):
    xa, ya, ia, ida = a
    xb, yb, ib, idb = b
    return (np.array_equal(xa.view(np.uint32), xb.view(np.uint32)) and
            np.array_equal(ya.view(np.uint32), yb.view(np.uint32)) and ia == ib and
            np.array_equal(ida, idb))


def test_graph_replay_matches_eager(chain):
    torch = torch_cuda()
    c = chain
    x0 = dev(inputs.gen_activation(1, D_MODEL, 70))
    x1 = dev(inputs.gen_activation(1, D_MODEL, 71))
    ref0 = run_eager(torch, c, x0)
    ref1 = run_eager(torch, c, x1)
    assert not same(ref0, ref1)
    # the chain's own invariants: finite state and logits, argmax of the logits
    for xf, yl, idx, _ in (ref0, ref1):
        assert np.isfinite(xf).all() and np.isfinite(yl).all()
        assert idx == int(np.argmax(yl))
    c.x.copy_(x0)
    c.capture()
    for rep in range(4):
        xin, ref = (x0, ref0) if rep % 2 == 0 else (x1, ref1)
        # eager work between replays: clobber the outputs, run the other
        # input eagerly, synchronize
        c.y_lm.fill_(float("nan"))
        c.idx.fill_(-1)
        other = run_eager(torch, c, x1 if rep % 2 == 0 else x0)
        assert same(other, ref1 if rep % 2 == 0 else ref0)
        got = run_graph(torch, c, xin)
        assert same(got, ref), "replay %d differs from the eager run" % rep


def test_graph_launch_count(chain):
    assert chain.launches_per_step() == 3 * LAYERS + 2
