"""Pins for the CPU oracle: closed forms, exhaustive decodes, brute force and
invariants that fix its arithmetic independently of the oracle itself.

Each test names the oracle step it pins.  A plausible slip anywhere in the
oracle (a dropped term, a wrong sign, a swapped nibble, a wrong rounding mode,
a transposed operand) fails at least one of these.
"""
import math
import os

import numpy as np
import pytest

from block_quant_matrix_amd import inputs

Q4, Q8 = 4, 8
Q4_K, Q5_K, Q6_K = 12, 13, 14
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers --

def f16_bytes(v: float) -> bytes:
    return np.array([v], "<f2").tobytes()


def q8_block(d: float, q) -> np.ndarray:
    q = np.asarray(q, np.int8)
    assert q.size == 32
    return np.frombuffer(f16_bytes(d) + q.tobytes(), np.uint8).copy()


def q4_block_from_elements(d: float, nib) -> np.ndarray:
    """nib[0..31] unsigned nibbles in element order -> 18-byte block
    (element j<16 in the low nibble of qs[j], element j+16 in the high nibble)."""
    nib = np.asarray(nib, np.uint8)
    assert nib.size == 32 and nib.max() < 16
    qs = (nib[:16] | (nib[16:] << 4)).astype(np.uint8)
    return np.frombuffer(f16_bytes(d) + qs.tobytes(), np.uint8).copy()


def lossless_activation(rng, k, e=7):
    """x = kint * 2^-e per block with some |kint| = 127 in every block, so that
    quantization is exact: d = 2^-e, q = kint."""
    kint = rng.integers(-127, 128, size=k).astype(np.int64)
    for b in range(k // 32):
        j = b * 32 + int(rng.integers(0, 32))
        kint[j] = 127 if rng.integers(0, 2) else -127
    return (kint * 2.0 ** -e).astype(np.float32), kint


# ----------------------------------------------- P1: the dot primitive -----

def test_p1_golden_dp4a_70(ref):
    """The pages' own worked example: 1*5+2*6+3*7+4*8 = 70 (tests/golden/dp4a_70.txt)."""
    with open(os.path.join(GOLDEN, "dp4a_70.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert rows
    for line in rows:
        a, b, want = line.split("|")
        a = [int(v) for v in a.split()]
        b = [int(v) for v in b.split()]
        want = int(want)
        qa = np.zeros(32, np.int8)
        qb = np.zeros(32, np.int8)
        qa[:4] = a
        qb[:4] = b
        assert ref.block_isum(Q8, q8_block(1.0, qa), qb) == want
        # the same four products through the Q4_0 encoding (value = nib - 8)
        nib = np.full(32, 8, np.uint8)
        nib[:4] = np.array(a) + 8
        assert ref.block_isum(Q4, q4_block_from_elements(1.0, nib), qb) == want


def test_p1_dot_extremes(ref):
    qa = np.zeros(32, np.int8)
    qb = np.zeros(32, np.int8)
    qa[:4] = -128
    qb[:4] = -128
    assert ref.block_isum(Q8, q8_block(1.0, qa), qb) == 65536
    qa[:4] = 127
    assert ref.block_isum(Q8, q8_block(1.0, qa), qb) == -65024
    # the largest possible |isum| of a whole block still fits int32
    qa[:] = -128
    qb[:] = -128
    assert ref.block_isum(Q8, q8_block(1.0, qa), qb) == 32 * 128 * 128


# ---------------------------------------------------- P2: fp16 decode ------

def test_p2_fp16_decode_exhaustive(ref):
    """All 65536 binary16 patterns against numpy's own float16 conversion."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = ref.fp16_to_f64(h)
    want = h.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zero is kept
    assert math.copysign(1.0, ref.fp16_to_f64(np.array([0x8000], np.uint16))[0]) == -1.0


def test_p2_block_decode_layout(ref):
    """Scale is the first two bytes, little-endian; then the quants."""
    d, vals = ref.decode_block(Q8, q8_block(-0.375, np.arange(-16, 16)))
    assert d == -0.375
    assert list(vals) == list(range(-16, 16))
    d, vals = ref.decode_block(Q4, q4_block_from_elements(2.0 ** -20, np.arange(32) % 16))
    assert d == 2.0 ** -20  # an fp16 subnormal
    assert list(vals) == [(j % 16) - 8 for j in range(32)]


# --------------------------------------------- P3: activation quantizer ----

def quant_block(ref, x):
    q, d, s = ref.quantize_act(np.asarray(x, np.float32))
    return q, float(d[0]), int(s[0])


def test_p3a_zero_block(ref):
    q, d, s = quant_block(ref, np.zeros(32))
    assert d == 0.0 and s == 0 and not q.any()
    q, d, s = quant_block(ref, -np.zeros(32))
    assert d == 0.0 and s == 0 and not q.any()


@pytest.mark.parametrize("e", [0, 3, 7, 20, 100])
def test_p3b_lossless(ref, e):
    rng = np.random.default_rng(e)
    x, kint = lossless_activation(rng, 32, e)
    q, d, s = quant_block(ref, x)
    assert d == 2.0 ** -e
    assert np.array_equal(q.astype(np.int64), kint)
    assert s == kint.sum()


@pytest.mark.parametrize("c", [1.0, 0.3, 1e-3, 7.5, 1e30])
def test_p3c_constant_block(ref, c):
    q, d, s = quant_block(ref, np.full(32, c))
    assert (q == 127).all() and s == 32 * 127
    assert d == np.float32(np.float32(c) / np.float32(127.0))
    q, d, s = quant_block(ref, np.full(32, -c))
    assert (q == -127).all() and s == -32 * 127


def test_p3d_half_way_rounds_away_from_zero(ref):
    """amax = 127 * 2^-e; elements at +-2.5, +-0.5, +-1.5 units of 2^-e.
    Half away from zero gives +-3, +-1, +-2 (half to even would give 2, 0, 2)."""
    e = 5
    u = 2.0 ** -e
    x = np.zeros(32)
    x[0] = 127 * u
    x[1], x[2] = 2.5 * u, -2.5 * u
    x[3], x[4] = 0.5 * u, -0.5 * u
    x[5], x[6] = 1.5 * u, -1.5 * u
    q, d, s = quant_block(ref, x)
    assert d == u
    assert list(q[:7]) == [127, 3, -3, 1, -1, 2, -2]
    assert s == 127


def test_p3e_invariants(ref):
    rng = np.random.default_rng(33)
    x = rng.standard_normal((64, 32 * 16)).astype(np.float32)
    x[3] *= 1e-30
    x[4] *= 1e30
    qx, dx, sx = ref.quantize_act(x)
    assert np.abs(qx.astype(np.int32)).max() <= 127
    xb = x.reshape(64, 16, 32).astype(np.float64)
    qb = qx.reshape(64, 16, 32).astype(np.int64)
    assert np.array_equal(qb.sum(-1), sx)
    amax_pos = np.abs(xb).argmax(-1)
    assert (np.abs(np.take_along_axis(qb, amax_pos[..., None], -1)) == 127).all()
    err = np.abs(xb - dx[..., None].astype(np.float64) * qb)
    assert (err <= dx[..., None] / 2 * (1 + 1e-6)).all()
    # sign symmetry: -x quantizes to -q with the same scale (used again in P9)
    qn, dn, sn = ref.quantize_act(-x)
    assert np.array_equal(qn, -qx) and np.array_equal(dn, dx) and np.array_equal(sn, -sx)


def test_p3_rejects_non_finite(ref):
    x = np.zeros(32, np.float32)
    x[7] = np.inf
    with pytest.raises(RuntimeError):
        ref.quantize_act(x)
    x[7] = np.nan
    with pytest.raises(RuntimeError):
        ref.quantize_act(x)


# --------------------------------------------------- P4: all ones ----------

@pytest.mark.parametrize("wtype", [Q8, Q4])
def test_p4_all_ones(ref, wtype):
    """q = 1 everywhere (Q4_0 nibble 9), d_w = 1.0, x = 127/128 -> d_x = 1/128,
    q_x = 127, isum = 4064, t_b = 31.75 and y = K*127/128 = 2032 exactly."""
    k, rows = 2048, 4
    blk = q8_block(1.0, np.ones(32)) if wtype == Q8 else q4_block_from_elements(1.0, np.full(32, 9))
    w = np.tile(blk, rows * (k // 32))
    x = np.full(k, 127 / 128, np.float32)
    qx, dx, sx = ref.quantize_act(x)
    assert (qx == 127).all() and (dx == 1 / 128).all() and (sx == 32 * 127).all()
    y, S, isums = ref.dmmv(wtype, w, rows, k, qx, dx, want_isums=True)
    assert (isums == 4064).all()
    assert (y == 2032.0).all() and (S == 2032.0).all()


# -------------------------------------------- P5: single nonzero block -----

@pytest.mark.parametrize("wtype", [Q8, Q4])
def test_p5_single_nonzero_block(ref, wtype):
    rows, k = 130, 32 * 66
    nb = k // 32
    rng = np.random.default_rng(5)
    x, kint = lossless_activation(rng, k, e=6)
    qx, dx, _ = ref.quantize_act(x)
    assert np.array_equal(qx.astype(np.int64), kint) and (dx == 2.0 ** -6).all()
    base = inputs.gen_weights(wtype, rows, k, 77)
    bb = inputs.BLOCK_BYTES[wtype]
    for rstar, bstar in [(0, 0), (0, nb - 1), (rows - 1, 0), (rows - 1, nb - 1), (63, 31),
                         (64, 32), (65, 64), (127, 1), (128, 65)]:
        w = base.copy().reshape(rows * nb, bb)
        w[:, 0:2] = np.frombuffer(f16_bytes(0.0), np.uint8)
        w[rstar * nb + bstar, 0:2] = np.frombuffer(f16_bytes(0.125), np.uint8)
        blk = w[rstar * nb + bstar]
        if wtype == Q8:
            vals = blk[2:].view(np.int8).astype(np.int64)
        else:
            qs = blk[2:].astype(np.int64)
            vals = np.concatenate([qs & 15, qs >> 4]) - 8
        isum = int(np.dot(vals, kint[bstar * 32:(bstar + 1) * 32]))
        y, S = ref.dmmv(wtype, w.reshape(-1), rows, k, qx, dx)
        want = np.zeros(rows)
        want[rstar] = 0.125 * 2.0 ** -6 * isum
        assert np.array_equal(y, want), (rstar, bstar)


# ------------------------------------------------ P6: Q4_0 identity -------

def test_p6_q4_identity_random_blocks(ref):
    """The oracle evaluates sum (nib-8)*q and sum nib*q - 8*sum q and fails on a
    mismatch; run it over many random blocks and activations."""
    rng = np.random.default_rng(6)
    w = inputs.gen_weights(Q4, 64, 32 * 64, 606)
    x = rng.standard_normal(32 * 64).astype(np.float32)
    qx, dx, _ = ref.quantize_act(x)
    ref.dmmv(Q4, w, 64, 32 * 64, qx, dx)  # raises on an identity failure


# ---------------------------------------------------- P7: nibble order ----

def test_p7_nibble_order(ref):
    """qs[0] = 0x0F, all other nibbles 8: element 0 = 15-8 = 7, element 16 = 0-8 = -8."""
    qs = np.full(16, 0x88, np.uint8)
    qs[0] = 0x0F
    blk = np.frombuffer(f16_bytes(1.0) + qs.tobytes(), np.uint8).copy()
    e0 = np.zeros(32, np.int8)
    e0[0] = 127
    e16 = np.zeros(32, np.int8)
    e16[16] = 127
    assert ref.block_isum(Q4, blk, e0) == 889
    assert ref.block_isum(Q4, blk, e16) == -1016
    e1 = np.zeros(32, np.int8)
    e1[1] = 127
    assert ref.block_isum(Q4, blk, e1) == 0


# --------------------------------------------------- P8: brute force ------

@pytest.mark.parametrize("wtype", [Q8, Q4])
@pytest.mark.parametrize("k", [32, 64, 256])
def test_p8_bruteforce_tiny(ref, wtype, k):
    rows = 8
    w = inputs.gen_weights(wtype, rows, k, 800 + k)
    x = inputs.gen_activation(1, k, 900 + k)
    qx, dx, _ = ref.quantize_act(x)
    y, S = ref.dmmv(wtype, w, rows, k, qx, dx)
    ybf = ref.dmmv_bruteforce(wtype, w, rows, k, qx, dx)
    assert (np.abs(y - ybf) <= 1e-12 * S).all()


@pytest.mark.parametrize("wl", [1, 2, 3, 13])
def test_p8_bruteforce_sampled_workloads(ref, wl):
    cfg = inputs.WORKLOADS[wl]
    w = inputs.gen_weights(cfg["wtype"], cfg["rows"], cfg["k"], inputs.seed_for(wl))
    x = inputs.gen_activation(1, cfg["k"], inputs.seed_for(wl) + 1)
    qx, dx, _ = ref.quantize_act(x)
    rng = np.random.default_rng(wl)
    rows = np.unique(np.concatenate([[0, cfg["rows"] - 1],
                                     rng.integers(0, cfg["rows"], 254)])).astype(np.int64)
    y, S = ref.dmmv(cfg["wtype"], w, cfg["rows"], cfg["k"], qx, dx, rows_eval=rows)
    ybf = ref.dmmv_bruteforce(cfg["wtype"], w, cfg["rows"], cfg["k"], qx, dx, rows_eval=rows)
    assert (np.abs(y - ybf) <= 1e-12 * S).all()


def test_p8_bruteforce_gemm_entries(ref):
    n, k, m = 40, 32 * 10, 6
    w = inputs.gen_weights(Q4, n, k, 81)
    x = inputs.gen_activation(m, k, 82)
    qx, dx, _ = ref.quantize_act(x)
    mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y, S = ref.gemm_entries(Q4, w, n, k, qx, dx, m, mi.ravel(), ni.ravel())
    for t in range(m):
        ybf = ref.dmmv_bruteforce(Q4, w, n, k, qx[t], dx[t])
        assert (np.abs(y.reshape(m, n)[t] - ybf) <= 1e-12 * S.reshape(m, n)[t]).all()


# ------------------------------------------------------ P9: linearity -----

@pytest.mark.parametrize("wtype", [Q8, Q4])
def test_p9_linearity(ref, wtype):
    rows, k = 33, 32 * 12
    nb = k // 32
    bb = inputs.BLOCK_BYTES[wtype]
    w = inputs.gen_weights(wtype, rows, k, 91)
    x = inputs.gen_activation(1, k, 92)
    qx, dx, sx = ref.quantize_act(x)
    y, S, isums = ref.dmmv(wtype, w, rows, k, qx, dx, want_isums=True)
    # doubling every weight scale doubles y exactly
    w2 = w.copy().reshape(rows * nb, bb)
    d = w2[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
    w2[:, 0:2] = (d * 2).astype("<f2").view(np.uint8).reshape(-1, 2)
    y2, _ = ref.dmmv(wtype, w2.reshape(-1), rows, k, qx, dx)
    assert np.array_equal(y2, 2 * y)
    # negating x negates qx, sx and every isum; y flips sign exactly
    qn, dn, sn = ref.quantize_act(-x)
    assert np.array_equal(qn, -qx) and np.array_equal(dn, dx) and np.array_equal(sn, -sx)
    yn, _, isn = ref.dmmv(wtype, w, rows, k, qn, dn, want_isums=True)
    assert np.array_equal(isn, -isums) and np.array_equal(yn, -y)
    # permuting rows permutes y
    perm = np.random.default_rng(9).permutation(rows)
    wp = w.reshape(rows, nb * bb)[perm].reshape(-1)
    yp, _ = ref.dmmv(wtype, wp, rows, k, qx, dx)
    assert np.array_equal(yp, y[perm])


def test_p9_accumulate_adds_previous(ref):
    rows, k = 16, 64
    w = inputs.gen_weights(Q4, rows, k, 95)
    qx, dx, _ = ref.quantize_act(inputs.gen_activation(1, k, 96))
    y, S = ref.dmmv(Q4, w, rows, k, qx, dx)
    prev = np.linspace(-3, 3, rows).astype(np.float32)
    ya, Sa = ref.dmmv(Q4, w, rows, k, qx, dx, y_prev=prev)
    assert np.array_equal(ya, y + prev.astype(np.float64))
    assert np.array_equal(Sa, S + np.abs(prev.astype(np.float64)))


# ---------------------------------------------------------- P11: MoE ------

def test_p11_route_against_full_sort(ref):
    for seed in range(20):
        logits, g = inputs.gen_router(128, seed)
        if seed == 3:
            logits[10] = logits[20] = logits[30] = 5.0  # a three-way tie at the top
        ids, wts = ref.moe_route(logits, 8, g)
        order = np.lexsort((np.arange(128), -logits.astype(np.float64)))  # by -logit, then id
        assert list(ids[:8]) == list(order[:8])
        assert ids[8] == 128
        assert abs(wts[:8].sum() - 1.0) < 1e-15
        sel = logits[order[:8]].astype(np.float64)
        want = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.allclose(wts[:8], want, rtol=1e-14, atol=0)
        assert wts[8] == pytest.approx(1 / (1 + math.exp(-float(g))), rel=1e-15)
        assert (np.diff(wts[:8]) <= 0).all()
    ids, wts = ref.moe_route(np.zeros(128, np.float32), 8, np.float32(0.0))
    assert list(ids) == list(range(8)) + [128]
    assert (wts[:8] == 0.125).all() and wts[8] == 0.5
    ids, wts = ref.moe_route(np.zeros(128, np.float32), 8, None)
    assert ids.size == 8


def test_p11_swiglu_closed_forms(ref):
    gu = np.array([[0.0, 1.0, -30.0, 3.0, 5.0, 2.0, 7.0, 1.0]], np.float32)  # f = 4
    h = ref.swiglu(gu, 4)[0]
    assert h[0] == 0.0
    assert h[1] == np.float32(1.0 / (1.0 + math.exp(-1.0)) * 2.0)
    assert h[2] == np.float32(-30.0 / (1.0 + math.exp(30.0)) * 7.0) and abs(h[2]) < 1e-10
    assert h[3] == np.float32(3.0 / (1.0 + math.exp(-3.0)))
    # silu(z) - silu(-z) = z
    z = np.linspace(-8, 8, 64).astype(np.float32)
    gu = np.concatenate([z, -z, np.ones(64), np.ones(64)]).astype(np.float32).reshape(1, -1)
    h = ref.swiglu(gu, 128)[0]
    assert np.allclose(h[:64].astype(np.float64) - h[64:].astype(np.float64), z, rtol=0, atol=4e-6)


def test_p11_moe_identical_and_one_hot_experts(ref):
    d_model, d_ff, E = 256, 64, 5
    bank_gu, gs, bank_d, ds = inputs.moe_banks(1100, E, d_model, d_ff)
    # make every expert a copy of expert 0
    bank_gu = np.tile(bank_gu[:gs], E)
    bank_d = np.tile(bank_d[:ds], E)
    x = inputs.gen_activation(1, d_model, 1101)
    ids = np.array([0, 1, 2, 3, 4], np.int32)
    wts = np.array([0.1, 0.2, 0.3, 0.25, 0.15])
    y, S = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids, wts, x)
    y1, S1 = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids[:1], np.ones(1), x)
    assert (np.abs(y - y1) <= 1e-12 * S1).all()
    # one-hot weights pick that expert alone; permuting (id, w) pairs changes nothing
    bank_gu, gs, bank_d, ds = inputs.moe_banks(1200, E, d_model, d_ff)
    y3, S3 = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids, np.eye(5)[3], x)
    y3b, _ = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids[3:4], np.ones(1), x)
    assert (np.abs(y3 - y3b) <= 1e-12 * S3).all()
    ya, Sa = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids, wts, x)
    p = np.array([4, 2, 0, 3, 1])
    yb, _ = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids[p], wts[p], x)
    assert (np.abs(ya - yb) <= 1e-12 * Sa).all()


def _bf_expert(ref, wt, w, rows, k, qx, dx):
    """Rows of one matrix by the element-wise brute force (fp64 dequantize
    then dot), for block formats and K-quants alike."""
    if wt in (Q4, Q8):
        return ref.dmmv_bruteforce(wt, w, rows, k, qx, dx)
    return ref.k_bruteforce(wt, w, rows, k, qx, dx)


def _mixed_case(seed, gu_wt, down_wt, sh_wt, n_routed=6, d_model=256, d_ff=256):
    """Routed banks of one format pair and a shared expert of its own format
    whose matrices differ from every routed one."""
    if gu_wt in (Q4, Q8):
        gu, gs, _, _ = inputs.moe_banks(seed, n_routed, d_model, d_ff, gu_wt)
    else:
        gu, gs, _, _ = inputs.moe_banks_k(seed, n_routed, d_model, d_ff, gu_wt, Q4_K)
    if down_wt in (Q4, Q8):
        _, _, dn, ds = inputs.moe_banks(seed + 1, n_routed, d_model, d_ff, down_wt)
    else:
        _, _, dn, ds = inputs.moe_banks_k(seed + 1, n_routed, d_model, d_ff, Q4_K, down_wt)
    if sh_wt in (Q4, Q8):
        sgu, _, sdn, _ = inputs.moe_banks(seed + 2, 1, d_model, d_ff, sh_wt)
    else:
        sgu, _, sdn, _ = inputs.moe_banks_k(seed + 2, 1, d_model, d_ff, sh_wt, sh_wt)
    return gu, gs, dn, ds, sgu, sdn


def test_p11_mixed_reduces_to_single_format_bank(ref):
    """moe_ffn_mixed with every matrix Q4_0 and the shared expert's matrices
    equal to slot n_routed of the routed banks is moe_ffn over that bank of
    n_routed + 1 experts (itself pinned above)."""
    d_model, d_ff, n_routed = 256, 64, 7
    bank_gu, gs, bank_d, ds = inputs.moe_banks(1300, n_routed + 1, d_model, d_ff)
    sh_gu = bank_gu[n_routed * gs:(n_routed + 1) * gs].copy()
    sh_dn = bank_d[n_routed * ds:(n_routed + 1) * ds].copy()
    x = inputs.gen_activation(1, d_model, 1301)
    logits, g = inputs.gen_router(n_routed, 1302)
    ids, wts = ref.moe_route(logits, 3, g)
    assert ids[-1] == n_routed
    y0, S0 = ref.moe_ffn(Q4, bank_gu, gs, bank_d, ds, d_model, d_ff, ids, wts, x)
    y1, S1 = ref.moe_ffn_mixed(Q4, bank_gu[:n_routed * gs], gs, Q4, bank_d[:n_routed * ds], ds, Q4,
                               sh_gu, sh_dn, n_routed, d_model, d_ff, ids, wts, x)
    assert np.all(np.abs(y1 - y0) <= 1e-12 * S0) and np.allclose(S1, S0, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmts", [(Q4_K, Q5_K, Q8), (Q4, Q8, Q6_K), (Q5_K, Q6_K, Q4)])
def test_p11_mixed_one_hot_slots_against_bruteforce(ref, fmts):
    """One-hot weights on a slot give that expert alone, computed here by the
    element-wise brute force from its own matrices: the shared slot (id
    n_routed) must use the shared expert's matrices in the shared format, a
    routed slot its bank's matrices in the routed formats."""
    gu_wt, down_wt, sh_wt = fmts
    d_model, d_ff, n_routed = 256, 256, 6
    gu, gs, dn, ds, sgu, sdn = _mixed_case(1400 + gu_wt, gu_wt, down_wt, sh_wt, n_routed,
                                           d_model, d_ff)
    x = inputs.gen_activation(1, d_model, 1401)
    ids = np.array([4, 1, n_routed], np.int32)
    qx, dx, _ = ref.quantize_act(x)
    for slot in range(3):
        w1 = np.eye(3)[slot] * 0.625
        y, S = ref.moe_ffn_mixed(gu_wt, gu, gs, down_wt, dn, ds, sh_wt, sgu, sdn, n_routed,
                                 d_model, d_ff, ids, w1, x)
        e = int(ids[slot])
        if e == n_routed:
            mg, md, tg, td = sgu, sdn, sh_wt, sh_wt
        else:
            mg, md, tg, td = gu[e * gs:(e + 1) * gs], dn[e * ds:(e + 1) * ds], gu_wt, down_wt
        gu_rows = _bf_expert(ref, tg, mg, 2 * d_ff, d_model, qx, dx)
        h = ref.swiglu(gu_rows.astype(np.float32).reshape(1, -1), d_ff)[0]
        qh, dh, _ = ref.quantize_act(h)
        expect = 0.625 * _bf_expert(ref, td, md, d_model, d_ff, qh, dh)
        assert np.all(np.abs(y - expect) <= 1e-12 * S), (fmts, slot)
        assert np.any(y != 0)


def test_p11_mixed_decomposes_into_weighted_slots(ref):
    """The block's output is the weighted sum of its slots' one-hot outputs,
    and permuting the (id, weight) pairs changes nothing."""
    gu_wt, down_wt, sh_wt = Q4_K, Q5_K, Q8
    d_model, d_ff, n_routed = 256, 256, 8
    gu, gs, dn, ds, sgu, sdn = _mixed_case(1500, gu_wt, down_wt, sh_wt, n_routed, d_model, d_ff)
    x = inputs.gen_activation(1, d_model, 1501)
    logits, g = inputs.gen_router(n_routed, 1502)
    ids, wts = ref.moe_route(logits, 4, g)
    args = (gu_wt, gu, gs, down_wt, dn, ds, sh_wt, sgu, sdn, n_routed, d_model, d_ff)
    y, S = ref.moe_ffn_mixed(*args, ids, wts, x)
    parts = sum(float(wts[s]) * ref.moe_ffn_mixed(*args, ids, np.eye(len(ids))[s], x)[0]
                for s in range(len(ids)))
    assert np.all(np.abs(y - parts) <= 1e-12 * S)
    p = np.array([3, 0, 4, 2, 1])
    yp, _ = ref.moe_ffn_mixed(*args, ids[p], wts[p], x)
    assert np.all(np.abs(y - yp) <= 1e-12 * S)
    # the shared slot's weight is the sigmoid of the gate, the routed ones
    # sum to one
    assert abs(wts[-1] - 1.0 / (1.0 + math.exp(-float(g)))) < 1e-7
    assert abs(float(np.sum(wts[:-1])) - 1.0) < 1e-6


# -------------------------------------------------------- P12: argmax -----

def test_p12_argmax_cases(ref):
    y = np.zeros(100, np.float32)
    y[5] = y[7] = 3.0
    assert ref.argmax_f32(y) == 5
    y = -np.arange(1, 130, dtype=np.float32)
    assert ref.argmax_f32(y) == 0
    y = np.arange(67, dtype=np.float32)
    assert ref.argmax_f32(y) == 66
    y = np.full(1, -7.0, np.float32)
    assert ref.argmax_f32(y) == 0
    y = np.random.default_rng(12).standard_normal(1000).astype(np.float32)
    assert ref.argmax_f32(y) == int(np.argmax(y))
    assert ref.argmax_f32(np.zeros(0, np.float32)) == -1


# ---------------------------------------------------- P13: determinism ----

def test_p13_deterministic(ref):
    w = inputs.gen_weights(Q4, 64, 512, 131)
    x = inputs.gen_activation(1, 512, 132)
    a = ref.quantize_act(x)
    b = ref.quantize_act(x)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    y1, S1 = ref.dmmv(Q4, w, 64, 512, a[0], a[1])
    y2, S2 = ref.dmmv(Q4, w, 64, 512, b[0], b[1])
    assert np.array_equal(y1, y2) and np.array_equal(S1, S2)
    # the generators are seeded
    assert np.array_equal(inputs.gen_weights(Q8, 4, 64, 7), inputs.gen_weights(Q8, 4, 64, 7))


# ------------------------------------------- P14: quantization error ------

@pytest.mark.parametrize("wtype", [Q8, Q4])
def test_p14_quantization_error_bound(ref, wtype):
    rows, k = 64, 2048
    w = inputs.gen_weights(wtype, rows, k, 141)
    x = inputs.gen_activation(1, k, 142)
    qx, dx, _ = ref.quantize_act(x)
    y, _ = ref.dmmv(wtype, w, rows, k, qx, dx)
    yt = ref.dmmv_true(wtype, w, rows, k, x)
    bound = ref.quant_error_bound(wtype, w, rows, k, dx)
    assert (np.abs(y - yt) <= bound * (1 + 1e-6)).all()
    # and the bound is not vacuous: the typical error is well inside it
    assert np.median(np.abs(y - yt) / bound) < 0.2
    # the unquantized reference really uses the fp32 activation: the error is
    # there on (almost) every row
    assert np.median(np.abs(y - yt) / bound) > 1e-3
    assert np.count_nonzero(y != yt) >= rows - 1


def test_p14_unquantized_reference_closed_forms(ref):
    """dmmv_true on cases with a known answer: (a) an activation that the
    quantizer represents exactly gives the quantized reference's rows; (b) a
    one-element weight against an activation element that quantizes to zero
    gives that element itself, where the quantized reference gives 0."""
    rng = np.random.default_rng(143)
    rows, k = 8, 256
    w = inputs.gen_weights(Q8, rows, k, 144)
    x, _ = lossless_activation(rng, k)
    qx, dx, _ = ref.quantize_act(x)
    y, S = ref.dmmv(Q8, w, rows, k, qx, dx)
    assert np.all(np.abs(ref.dmmv_true(Q8, w, rows, k, x) - y) <= 1e-12 * S)
    q = np.zeros(32, np.int8)
    q[0] = 1
    w1 = q8_block(1.0, q)
    xb = np.zeros(32, np.float32)
    xb[1] = 127.0
    xb[0] = np.float32(0.3)
    qx1, dx1, _ = ref.quantize_act(xb)
    assert qx1[0] == 0 and ref.dmmv(Q8, w1, 1, 32, qx1, dx1)[0][0] == 0.0
    assert ref.dmmv_true(Q8, w1, 1, 32, xb)[0] == float(np.float32(0.3))


# ----------------------------------------------- generators' recipe -------

def test_generator_distributions():
    w = inputs.gen_weights(Q4, 512, 2048, 1).reshape(-1, 18)
    d = w[:, :2].copy().view("<f2").astype(np.float64).ravel()
    assert (d >= 0).all() and abs(d.mean() - 0.02 * math.sqrt(2 / math.pi)) < 2e-4
    nib = np.concatenate([w[:, 2:] & 15, w[:, 2:] >> 4]).ravel()
    assert abs(nib.mean() - 7.5) < 0.05 and nib.min() == 0 and nib.max() == 15
    w = inputs.gen_weights(Q8, 512, 2048, 1).reshape(-1, 34)
    q = w[:, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127
    d = w[:, :2].copy().view("<f2").astype(np.float64).ravel()
    assert abs(d.mean() - 0.01 * math.sqrt(2 / math.pi)) < 1e-4
    # some scales are fp16 subnormals; they must be kept as such
    assert (d < 2.0 ** -14).any()


def test_p3f_halfway_after_rounding(ref):
    """Elements whose fp32 product x*id rounds to exactly c + 1/2 (the exact
    product lies below it) must quantize to c + 1: the product is rounded to
    fp32 before the half-away-from-zero decision."""
    from cases import halfway_after_rounding
    x, hits = halfway_after_rounding(11)
    assert len(hits) > 1000
    q, d, s = ref.quantize_act(x)
    for i, want in hits:
        assert int(q[i]) == want, (i, want, int(q[i]))


# ------------------------------------------------------- K-quants (P15) ----
# An encoder written here from the byte and bit positions of the published
# layouts (element index -> byte, nibble, bit), independent of the oracle's
# decoder, which walks the other way.

KBB = {Q4_K: 144, Q5_K: 176, Q6_K: 210}


def k_encode(wtype, d, dmin, sc, mn, q):
    """Pack one super-block.  sc/mn: 8 values in 0..63 (Q4_K, Q5_K) or 16
    int8 scales (Q6_K); q: 256 codes (0..15, 0..31 or 0..63)."""
    out = np.zeros(KBB[wtype], np.uint8)
    if wtype in (Q4_K, Q5_K):
        out[0:2] = np.frombuffer(np.float16(d).astype("<f2").tobytes(), np.uint8)
        out[2:4] = np.frombuffer(np.float16(dmin).astype("<f2").tobytes(), np.uint8)
        s = np.zeros(12, np.int64)
        for j in range(4):
            s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
            s[j + 4] = mn[j] | ((mn[j + 4] >> 4) << 6)
            s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
        out[4:16] = s
        code0 = 16 if wtype == Q4_K else 48
        for e in range(256):
            g, w = divmod(e, 64)
            hi, l = divmod(w, 32)
            out[code0 + 32 * g + l] |= (q[e] & 15) << (4 * hi)
            if wtype == Q5_K:
                out[16 + l] |= ((q[e] >> 4) & 1) << (2 * g + hi)
    else:
        for e in range(256):
            h, rest = divmod(e, 128)
            c, l = divmod(rest, 32)
            out[64 * h + 32 * (c % 2) + l] |= (q[e] & 15) << (4 * (c // 2))
            out[128 + 32 * h + l] |= ((q[e] >> 4) & 3) << (2 * c)
        out[192:208] = np.asarray(sc, np.int64).astype(np.int8).view(np.uint8)
        out[208:210] = np.frombuffer(np.float16(d).astype("<f2").tobytes(), np.uint8)
    return out


def golden_kquant():
    rows = []
    for line in open(os.path.join(GOLDEN, "kquant_superblocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        typ, head, code, high, vals = [f.strip() for f in line.split("|")]
        wt = {"Q4_K": Q4_K, "Q5_K": Q5_K, "Q6_K": Q6_K}[typ]
        hb = []
        for tok in head.split():
            hb += list(bytes.fromhex(tok))   # 4-digit tokens: little-endian fp16 bytes as written
        sb = np.zeros(KBB[wt], np.uint8)
        if wt == Q4_K:
            sb[0:16] = hb
            sb[16:] = int(code, 16)
        elif wt == Q5_K:
            sb[0:16] = hb
            sb[16:48] = int(high, 16)
            sb[48:] = int(code, 16)
        else:
            sb[0:128] = int(code, 16)
            sb[128:192] = int(high, 16)
            sb[192:210] = hb
        exp = {int(a): float(b) for a, b in (t.split(":") for t in vals.split())}
        rows.append((wt, sb, exp))
    return rows


def dequant_one(ref, wt, sb, e):
    """Element e of super-block sb through the oracle's brute-force path:
    activation one-hot at e with code 1 and scale 1."""
    qx = np.zeros(256, np.int8)
    qx[e] = 1
    dx = np.ones(8, np.float32)
    return float(ref.k_bruteforce(wt, sb, 1, 256, qx, dx)[0])


def test_p15_golden_superblocks(ref):
    """Hand-worked super-blocks (tests/golden/kquant_superblocks.txt): the
    decoder and the brute-force path give the values derived by hand."""
    g = golden_kquant()
    assert [w for w, _, _ in g] == [Q4_K, Q5_K, Q6_K]
    for wt, sb, exp in g:
        d, dmin, sc, mn, q = ref.k_decode(wt, sb)
        for e, v in exp.items():
            if wt == Q6_K:
                assert d * sc[e // 16] * (q[e] - 32) == v, (wt, e)
            else:
                assert d * sc[e // 32] * q[e] - dmin * mn[e // 32] == v, (wt, e)
            assert dequant_one(ref, wt, sb, e) == v, (wt, e)
    # the scales of the Q4_K example, spelled out in the fixture
    d, dmin, sc, mn, _ = ref.k_decode(Q4_K, g[0][1])
    assert (d, dmin) == (1.0, 0.5)
    assert list(sc) == [1, 2, 3, 4, 17, 35, 53, 7] and list(mn) == [5, 6, 7, 8, 18, 36, 54, 8]


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K])
def test_p15_encode_decode_round_trip(ref, wt):
    rng = np.random.default_rng(wt)
    for _ in range(50):
        d, dmin = float(np.float16(rng.uniform(0.01, 2))), float(np.float16(rng.uniform(0, 2)))
        if wt == Q6_K:
            sc = rng.integers(-128, 128, 16)
            mn = np.zeros(16, np.int64)
            q = rng.integers(0, 64, 256)
            dmin = 0.0
        else:
            sc = rng.integers(0, 64, 8)
            mn = rng.integers(0, 64, 8)
            q = rng.integers(0, 32 if wt == Q5_K else 16, 256)
        dd, dm, s2, m2, q2 = ref.k_decode(wt, k_encode(wt, d, dmin, sc, mn, q))
        assert dd == d and dm == dmin
        assert np.array_equal(s2, sc) and np.array_equal(m2, mn) and np.array_equal(q2, q)


def test_p15_scale_min_exhaustive(ref):
    """Every 6-bit (scale, min) pair at every sub-block position."""
    for j in range(8):
        for v in range(64):
            sc = np.zeros(8, np.int64)
            mn = np.zeros(8, np.int64)
            sc[j] = v
            mn[j] = 63 - v
            _, _, s2, m2, _ = ref.k_decode(Q4_K, k_encode(Q4_K, 1.0, 1.0, sc, mn, np.zeros(256, np.int64)))
            assert np.array_equal(s2, sc) and np.array_equal(m2, mn), (j, v)


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K])
def test_p15_single_element_positions(ref, wt):
    """A lone code at each of the 256 positions lands at that element (and
    nowhere else) with the scale of its sub-block."""
    top = {Q4_K: 15, Q5_K: 31, Q6_K: 63}[wt]
    base = 32 if wt == Q6_K else 0
    sc = np.arange(1, 17) if wt == Q6_K else np.arange(1, 9)
    for e in range(256):
        q = np.full(256, base, np.int64)
        q[e] = top
        sb = k_encode(wt, 0.5, 0.0, sc, np.zeros(len(sc), np.int64), q)
        _, _, _, _, q2 = ref.k_decode(wt, sb)
        assert np.array_equal(q2, q), (wt, e)
        sub = e // 16 if wt == Q6_K else e // 32
        assert dequant_one(ref, wt, sb, e) == 0.5 * sc[sub] * (top - base)


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K])
def test_p15_closed_form_rows(ref, wt):
    """Unit scales and a constant code: every weight equals one number c, so
    each row is c * sum_b dx_b * s_b, exactly."""
    rows, k = 3, 512
    if wt == Q6_K:
        sb = k_encode(wt, 1.0, 0.0, np.ones(16, np.int64), np.zeros(16, np.int64),
                      np.full(256, 33, np.int64))            # value 1*1*(33-32) = 1
        c = 1.0
    else:
        sb = k_encode(wt, 1.0, 0.5, np.ones(8, np.int64), np.full(8, 2, np.int64),
                      np.full(256, 3, np.int64))             # value 3 - 1 = 2
        c = 2.0
    w = np.tile(sb, rows * (k // 256))
    x = inputs.gen_activation(1, k, 31)
    qx, dx, sx = ref.quantize_act(x)
    y, S = ref.k_dmmv(wt, w, rows, k, qx, dx)
    expect = c * sum(float(dx[b]) * int(sx[b]) for b in range(k // 32))
    assert np.all(np.abs(y - expect) <= 1e-12 * S)


@pytest.mark.parametrize("wt", [Q4_K, Q5_K, Q6_K])
def test_p15_bruteforce_and_isums(ref, wt):
    """Random super-blocks: the per-block references equal the element-wise
    brute force, and the integer sums equal numpy's on the encoder's codes."""
    rng = np.random.default_rng(100 + wt)
    rows, k = 4, 768
    sbs, codes, scs = [], [], []
    for _ in range(rows * k // 256):
        if wt == Q6_K:
            sc, mn, q = rng.integers(-128, 128, 16), np.zeros(16, np.int64), rng.integers(0, 64, 256)
        else:
            sc, mn = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
            q = rng.integers(0, 32 if wt == Q5_K else 16, 256)
        sbs.append(k_encode(wt, float(np.float16(rng.uniform(0.001, 0.01))),
                            float(np.float16(rng.uniform(0, 0.01))), sc, mn, q))
        codes.append(q)
        scs.append(sc)
    w = np.concatenate(sbs)
    x = inputs.gen_activation(1, k, 32)
    qx, dx, sx = ref.quantize_act(x)
    y, S, isums = ref.k_dmmv(wt, w, rows, k, qx, dx, want_isums=True)
    yb = ref.k_bruteforce(wt, w, rows, k, qx, dx)
    assert np.all(np.abs(y - yb) <= 1e-12 * S)
    nsb = k // 256
    for r in range(rows):
        for b in range(k // 32):
            u, j = divmod(b, 8)
            q = codes[r * nsb + u][32 * j:32 * j + 32].astype(np.int64)
            xb = qx[32 * b:32 * b + 32].astype(np.int64)
            if wt == Q6_K:
                s16 = scs[r * nsb + u][np.arange(32 * j, 32 * j + 32) // 16].astype(np.int64)
                expect = int(np.sum(s16 * (q - 32) * xb))
            else:
                expect = int(np.sum(q * xb))
            assert isums[r, b] == expect, (r, b)


def test_p15_generator_layout():
    """gen_weights_k: the fp16 super-block scales sit where the layouts put
    them, with the stated distribution."""
    for wt in (Q4_K, Q5_K, Q6_K):
        w = inputs.gen_weights_k(wt, 64, 1024, 5).reshape(-1, KBB[wt])
        off = 208 if wt == Q6_K else 0
        d = w[:, off:off + 2].copy().view("<f2").astype(np.float64).ravel()
        assert np.all(d >= 0) and 0.0004 < d.mean() < 0.0012


# ------------------------------------------------------- P16: rms_norm ----

def test_p16_rms_norm_golden(ref):
    """Hand-derived values (tests/golden/rms_norm.txt)."""
    n = 0
    for line in open(os.path.join(GOLDEN, "rms_norm.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        xs, ws, eps, exp = [p.split() for p in line.split("|")]
        x = np.array([float(v) for v in xs], np.float32)
        w = np.array([float(v) for v in ws], np.float32)
        got = ref.rms_norm(x, w, float(eps[0]))
        assert np.allclose(got, [float(v) for v in exp], rtol=1e-15, atol=0), line
        n += 1
    assert n == 4


def test_p16_rms_norm_invariants(ref):
    rng = np.random.default_rng(16)
    k = 2048
    x = rng.standard_normal(k).astype(np.float32)
    one = np.ones(k, np.float32)
    xn = ref.rms_norm(x, one, 0.0)
    # unit root mean square: sum of squares = k
    assert abs(float(np.sum(xn * xn)) - k) <= 1e-9 * k
    # scale invariance (eps = 0): a power of two scales x and the root mean
    # square alike, exactly
    assert np.array_equal(ref.rms_norm(4 * x, one, 0.0), xn)
    assert np.array_equal(ref.rms_norm(0.5 * x, one, 0.0), xn)
    # the weight multiplies elementwise, at its own index
    w = rng.standard_normal(k).astype(np.float32)
    assert np.allclose(ref.rms_norm(x, w, 0.0), xn * w.astype(np.float64), rtol=1e-15, atol=0)
    # eps enters under the root: a constant vector c gives c / sqrt(c^2 + eps)
    c = np.full(k, 0.75, np.float32)
    assert np.allclose(ref.rms_norm(c, one, 0.4375), 0.75 / math.sqrt(0.5625 + 0.4375),
                       rtol=1e-15, atol=0)
    # a constant vector with eps = 0 normalizes to its sign
    assert np.array_equal(ref.rms_norm(-c, one, 0.0), -np.ones(k))
    # zero input: zero output with eps > 0, refused with eps = 0
    assert np.array_equal(ref.rms_norm(np.zeros(k, np.float32), one, 1e-6), np.zeros(k))
    with pytest.raises(RuntimeError):
        ref.rms_norm(np.zeros(k, np.float32), one, 0.0)
    # tokens are independent
    x2 = rng.standard_normal((3, 64)).astype(np.float32)
    xn2 = ref.rms_norm(x2, np.ones(64, np.float32), 1e-6)
    for t in range(3):
        assert np.array_equal(xn2[t], ref.rms_norm(x2[t], np.ones(64, np.float32), 1e-6))


# -------------------------------------------------- P17: float weights ----
# The F16 / F32 DMMV over the fp32 activation.

F16, F32 = 16, 32


def _float_bytes(wt, vals):
    return np.ascontiguousarray(np.asarray(vals, np.float64).astype("<f2" if wt == F16 else "<f4")
                                ).view(np.uint8).reshape(-1)


@pytest.mark.parametrize("wt", [F16, F32])
def test_p17_all_ones_and_single_element(ref, wt):
    rows, k = 5, 96
    w = _float_bytes(wt, np.ones((rows, k)))
    y, S = ref.float_dmmv(wt, w, rows, k, np.full(k, 0.75, np.float32))
    assert np.all(y == 0.75 * k) and np.all(S == 0.75 * k)
    rng = np.random.default_rng(170)
    x = rng.standard_normal(k).astype(np.float32)
    for r0, j0, h in [(0, 0, -1.5), (4, 95, 0.0009765625), (2, 33, 65504.0), (3, 7, 2.0 ** -24)]:
        vals = np.zeros((rows, k))
        vals[r0, j0] = h
        y, S = ref.float_dmmv(wt, _float_bytes(wt, vals), rows, k, x)
        expect = np.zeros(rows)
        expect[r0] = h * float(x[j0])   # exact: 11 (or 24) x 24 significant bits
        assert np.array_equal(y, expect) and np.array_equal(S, np.abs(expect))


def test_p17_f16_byte_order_and_subnormals(ref):
    """Little-endian binary16: bytes (0x00, 0x3C) are 1.0; (0x3C, 0x00) is
    the subnormal 60 * 2^-24.  Subnormals decode exactly."""
    x = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0], np.float32)
    w = np.zeros(16, np.uint8)
    w[1] = 0x3C
    assert ref.float_dmmv(F16, w, 1, 8, x)[0][0] == 1.0
    w[:] = 0
    w[0] = 0x3C
    assert ref.float_dmmv(F16, w, 1, 8, x)[0][0] == 60 * 2.0 ** -24
    w = np.tile(np.array([0x01, 0x00], np.uint8), 8)   # every weight 2^-24
    assert ref.float_dmmv(F16, w, 1, 8, x)[0][0] == 36 * 2.0 ** -24


@pytest.mark.parametrize("wt", [F16, F32])
def test_p17_bruteforce_against_numpy(ref, wt):
    """Random rows against numpy's own float16/float32 decode and a float64
    dot product, within 1e-12 of the error scale; accumulate adds y_prev."""
    rows, k = 7, 1000
    w = inputs.gen_weights_float(wt, rows, k, 171)
    x = inputs.gen_activation(1, k, 172)
    wd = w.view("<f2" if wt == F16 else "<f4").astype(np.float64).reshape(rows, k)
    yb = wd @ x.astype(np.float64)
    y, S = ref.float_dmmv(wt, w, rows, k, x)
    assert np.all(np.abs(y - yb) <= 1e-12 * S)
    assert np.allclose(S, np.abs(wd * x.astype(np.float64)).sum(1), rtol=1e-12, atol=0)
    prev = np.arange(rows, dtype=np.float32) - 3
    y2, S2 = ref.float_dmmv(wt, w, rows, k, x, y_prev=prev)
    assert np.all(np.abs(y2 - (y + prev)) <= 1e-12 * S2)
    # negating x negates y exactly; a subset of rows is those rows
    assert np.array_equal(ref.float_dmmv(wt, w, rows, k, -x)[0], -y)
    idx = np.array([6, 0, 3])
    assert np.array_equal(ref.float_dmmv(wt, w, rows, k, x, rows_eval=idx)[0], y[idx])


def test_p17_refuses_non_finite(ref):
    w = _float_bytes(F16, np.ones((1, 8)))
    x = np.ones(8, np.float32)
    x[3] = np.inf
    with pytest.raises(RuntimeError):
        ref.float_dmmv(F16, w, 1, 8, x)
    w = _float_bytes(F32, [[1, 1, np.nan, 1, 1, 1, 1, 1]])
    with pytest.raises(RuntimeError):
        ref.float_dmmv(F32, w, 1, 8, np.ones(8, np.float32))
