"""CPU oracle for the block-quantized DMMV path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.

The arithmetic lives in ``zqref.c`` (plain C, fp64 references, built with
``gcc -O2 -ffp-contract=off``).  This module only loads it with ctypes and
marshals numpy arrays; the MoE chain composes the C primitives in the order
the pages give: routing (softmax_topk), expert gate/up DMMV, swiglu, activation
re-quantization, expert down DMMV and the weighted accumulate ("Bringing ZINC
to NVIDIA", section "The roadmap: from 70 to a coherent token"; "CUDA backend
for ZINC", section 5, milestone M1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zqref.c")
_LIB = os.path.join(_HERE, "libzqref.so")

Q4_0 = 4
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
F16 = 16
F32 = 32
FLOAT_BYTES = {F16: 2, F32: 4}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}
K_BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}

_ERR = {0: "ok", -1: "invalid argument", -2: "non-finite input",
        -3: "int32 overflow", -4: "Q4_0 identity failed"}

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile zqref.c with gcc into libzqref.so (next to the source)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.zqref_fp16_to_f64.restype = ctypes.c_double
        L.zqref_fp16_to_f64.argtypes = [ctypes.c_uint16]
        L.zqref_fp16_to_f64_array.argtypes = [P, I64, P]
        L.zqref_decode_block.argtypes = [I, P, P, P]
        L.zqref_quantize_block.argtypes = [P, P, P, P]
        L.zqref_quantize_act.argtypes = [P, I64, I64, I64, P, P, P]
        L.zqref_block_isum.argtypes = [I, P, P, P]
        L.zqref_dmmv_rows.argtypes = [I, P, I64, I64, P, P, P, P, I64, P, P, P]
        L.zqref_dmmv_bruteforce.argtypes = [I, P, I64, I64, P, P, P, I64, P]
        L.zqref_dmmv_true.argtypes = [I, P, I64, I64, P, P, I64, P]
        L.zqref_quant_error_bound.argtypes = [I, P, I64, I64, P, P, I64, P]
        L.zqref_argmax_f32.restype = I64
        L.zqref_argmax_f32.argtypes = [P, I64]
        L.zqref_moe_route.argtypes = [P, I, I, P, P, P]
        L.zqref_swiglu.argtypes = [P, I64, I64, P]
        L.zqref_rms_norm.argtypes = [P, P, ctypes.c_double, I64, I64, I64, P]
        L.zqref_gemm_entries.argtypes = [I, P, I64, I64, P, P, I64, P, P, I64, P, P]
        L.zqref_k_block_bytes.restype = I64
        L.zqref_k_block_bytes.argtypes = [I]
        L.zqref_k_decode.argtypes = [I, P, P, P, P, P, P]
        L.zqref_k_dmmv_rows.argtypes = [I, P, I64, I64, P, P, P, P, I64, P, P, P]
        L.zqref_k_bruteforce.argtypes = [I, P, I64, I64, P, P, P, I64, P]
        L.zqref_float_dmmv_rows.argtypes = [I, P, I64, I64, P, P, P, I64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("oracle %s failed: %s" % (what, _ERR.get(rc, rc)))


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def fp16_to_f64(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().zqref_fp16_to_f64_array(_p(h), h.size, _p(out))
    return out


def decode_block(wtype: int, blk: bytes | np.ndarray):
    b = _c(np.frombuffer(bytes(blk), np.uint8) if isinstance(blk, (bytes, bytearray)) else blk,
           np.uint8)
    d = ctypes.c_double()
    vals = np.empty(32, np.int32)
    _check(lib().zqref_decode_block(wtype, _p(b), ctypes.byref(d), _p(vals)), "decode_block")
    return d.value, vals


def quantize_act(x: np.ndarray):
    """x: [T][K] or [K] fp32 -> (qx int8 same shape, dx fp32 [..][K/32], sx int32)."""
    x = _c(x, np.float32)
    squeeze = x.ndim == 1
    x2 = x.reshape(1, -1) if squeeze else x
    t, k = x2.shape
    qx = np.empty((t, k), np.int8)
    dx = np.empty((t, k // 32), np.float32)
    sx = np.empty((t, k // 32), np.int32)
    _check(lib().zqref_quantize_act(_p(x2), t, k, k, _p(qx), _p(dx), _p(sx)), "quantize_act")
    if squeeze:
        return qx[0], dx[0], sx[0]
    return qx, dx, sx


def block_isum(wtype: int, blk: np.ndarray, qx32: np.ndarray) -> int:
    b = _c(blk, np.uint8)
    q = _c(qx32, np.int8)
    out = ctypes.c_int32()
    _check(lib().zqref_block_isum(wtype, _p(b), _p(q), ctypes.byref(out)), "block_isum")
    return out.value


def dmmv(wtype: int, w: np.ndarray, rows: int, k: int, qx, dx, rows_eval=None, y_prev=None,
         want_isums: bool = False):
    """fp64 reference rows: returns (y_ref, S) or (y_ref, S, isums[n_eval][K/32])."""
    w = _c(w, np.uint8)
    assert w.size >= rows * (k // 32) * BLOCK_BYTES[wtype]
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    yp = None if y_prev is None else _c(y_prev, np.float32)
    isums = np.empty((n, k // 32), np.int32) if want_isums else None
    _check(lib().zqref_dmmv_rows(wtype, _p(w), rows, k, _p(qx), _p(dx), _p(yp), _p(idx), n,
                                 _p(y), _p(S), _p(isums)), "dmmv_rows")
    return (y, S, isums) if want_isums else (y, S)


def dmmv_bruteforce(wtype, w, rows, k, qx, dx, rows_eval=None):
    w = _c(w, np.uint8)
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    _check(lib().zqref_dmmv_bruteforce(wtype, _p(w), rows, k, _p(qx), _p(dx), _p(idx), n, _p(y)),
           "dmmv_bruteforce")
    return y


def dmmv_true(wtype, w, rows, k, x, rows_eval=None):
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    _check(lib().zqref_dmmv_true(wtype, _p(w), rows, k, _p(x), _p(idx), n, _p(y)), "dmmv_true")
    return y


def quant_error_bound(wtype, w, rows, k, dx, rows_eval=None):
    w = _c(w, np.uint8)
    dx = _c(dx, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    out = np.empty(n, np.float64)
    _check(lib().zqref_quant_error_bound(wtype, _p(w), rows, k, _p(dx), _p(idx), n, _p(out)),
           "quant_error_bound")
    return out


def k_decode(wtype: int, sb: np.ndarray):
    """One K-quant super-block -> (d, dmin, scales, mins, codes[256])."""
    b = _c(sb, np.uint8)
    d, dmin = ctypes.c_double(), ctypes.c_double()
    sc = np.zeros(16, np.int32)
    mn = np.zeros(16, np.int32)
    q = np.empty(256, np.int32)
    _check(lib().zqref_k_decode(wtype, _p(b), ctypes.byref(d), ctypes.byref(dmin), _p(sc), _p(mn),
                                _p(q)), "k_decode")
    n = 16 if wtype == Q6_K else 8
    return d.value, dmin.value, sc[:n], mn[:n], q


def k_dmmv(wtype: int, w: np.ndarray, rows: int, k: int, qx, dx, rows_eval=None, y_prev=None,
           want_isums: bool = False):
    """fp64 reference rows over K-quant weights: (y_ref, S) or
    (y_ref, S, isums[n_eval][K/32])."""
    w = _c(w, np.uint8)
    assert w.size >= rows * (k // 256) * K_BLOCK_BYTES[wtype]
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    yp = None if y_prev is None else _c(y_prev, np.float32)
    isums = np.empty((n, k // 32), np.int32) if want_isums else None
    _check(lib().zqref_k_dmmv_rows(wtype, _p(w), rows, k, _p(qx), _p(dx), _p(yp), _p(idx), n,
                                   _p(y), _p(S), _p(isums)), "k_dmmv_rows")
    return (y, S, isums) if want_isums else (y, S)


def k_bruteforce(wtype, w, rows, k, qx, dx, rows_eval=None):
    w = _c(w, np.uint8)
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    _check(lib().zqref_k_bruteforce(wtype, _p(w), rows, k, _p(qx), _p(dx), _p(idx), n, _p(y)),
           "k_bruteforce")
    return y


def float_dmmv(wtype: int, w: np.ndarray, rows: int, k: int, x, rows_eval=None, y_prev=None):
    """fp64 reference rows of a float (F16 / F32) weight matrix times the fp32
    activation: (y_ref, S)."""
    w = _c(w, np.uint8)
    assert w.size >= rows * k * FLOAT_BYTES[wtype]
    x = _c(x, np.float32)
    idx = None if rows_eval is None else _c(rows_eval, np.int64)
    n = rows if idx is None else idx.size
    y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    yp = None if y_prev is None else _c(y_prev, np.float32)
    _check(lib().zqref_float_dmmv_rows(wtype, _p(w), rows, k, _p(x), _p(yp), _p(idx), n, _p(y),
                                       _p(S)), "float_dmmv_rows")
    return y, S


def argmax_f32(y: np.ndarray) -> int:
    y = _c(y, np.float32)
    return int(lib().zqref_argmax_f32(_p(y), y.size))


def moe_route(logits: np.ndarray, top_k: int, shared_gate: float | None):
    logits = _c(logits, np.float32)
    n = logits.size
    m = top_k + (1 if shared_gate is not None else 0)
    ids = np.empty(m, np.int32)
    wts = np.empty(m, np.float64)
    g = None if shared_gate is None else np.array([shared_gate], np.float32)
    _check(lib().zqref_moe_route(_p(logits), n, top_k, _p(g), _p(ids), _p(wts)), "moe_route")
    return ids, wts


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """xn = x / sqrt(mean(x^2) + eps) * w per token, in fp64: x [T][K] or [K]
    fp32, w [K] fp32 -> fp64 of x's shape."""
    x = _c(x, np.float32)
    squeeze = x.ndim == 1
    x2 = x.reshape(1, -1) if squeeze else x
    t, k = x2.shape
    w = _c(w, np.float32)
    assert w.size == k
    xn = np.empty((t, k), np.float64)
    _check(lib().zqref_rms_norm(_p(x2), _p(w), float(eps), t, k, k, _p(xn)), "rms_norm")
    return xn[0] if squeeze else xn


def swiglu(gu: np.ndarray, f: int) -> np.ndarray:
    gu = _c(gu, np.float32).reshape(-1, 2 * f)
    h = np.empty((gu.shape[0], f), np.float32)
    _check(lib().zqref_swiglu(_p(gu), gu.shape[0], f, _p(h)), "swiglu")
    return h


def gemm_entries(wtype, w, n_rows, k, qx, dx, m_tok, mi, ni):
    w = _c(w, np.uint8)
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    y = np.empty(mi.size, np.float64)
    S = np.empty(mi.size, np.float64)
    _check(lib().zqref_gemm_entries(wtype, _p(w), n_rows, k, _p(qx), _p(dx), m_tok, _p(mi),
                                    _p(ni), mi.size, _p(y), _p(S)), "gemm_entries")
    return y, S


# ------------------------------------------------------------------ MoE ----

def moe_expert_rows(wtype, bank: np.ndarray, expert_stride: int, rows: int, k: int, eid: int,
                    qx, dx, rows_eval=None):
    """Reference rows of expert ``eid`` of a bank of stacked matrices."""
    nbytes = rows * (k // 32) * BLOCK_BYTES[wtype]
    w = bank[eid * expert_stride: eid * expert_stride + nbytes]
    return dmmv(wtype, w, rows, k, qx, dx, rows_eval=rows_eval)


def moe_gate_up(wtype, gu_bank, gu_stride, d_model, d_ff, ids, qx, dx):
    """Stage (i): gu[s] = W_gu[ids[s]] . x for every selected expert (fp64 + S)."""
    ys, Ss = [], []
    for e in ids:
        y, S = moe_expert_rows(wtype, gu_bank, gu_stride, 2 * d_ff, d_model, int(e), qx, dx)
        ys.append(y)
        Ss.append(S)
    return np.stack(ys), np.stack(Ss)


def moe_down_weighted(wtype, down_bank, down_stride, d_model, d_ff, ids, wts, qh, dh,
                      rows_eval=None):
    """Stage (iii): y = sum_s wts[s] * (W_d[ids[s]] . h_s); S = sum_s |w_s| * S_s."""
    n = d_model if rows_eval is None else len(rows_eval)
    y = np.zeros(n, np.float64)
    S = np.zeros(n, np.float64)
    for s, e in enumerate(ids):
        ye, Se = moe_expert_rows(wtype, down_bank, down_stride, d_model, d_ff, int(e), qh[s],
                                 dh[s], rows_eval=rows_eval)
        y += float(wts[s]) * ye
        S += abs(float(wts[s])) * Se
    return y, S


def expert_rows_any(wtype, bank: np.ndarray, expert_stride: int, rows: int, k: int, eid: int,
                    qx, dx, rows_eval=None):
    """Reference rows of expert ``eid`` of a bank in any weight type (Q4_0 /
    Q8_0 blocks or K-quant super-blocks)."""
    if wtype in K_BLOCK_BYTES:
        nbytes = rows * (k // 256) * K_BLOCK_BYTES[wtype]
        w = bank[eid * expert_stride: eid * expert_stride + nbytes]
        return k_dmmv(wtype, w, rows, k, qx, dx, rows_eval=rows_eval)
    return moe_expert_rows(wtype, bank, expert_stride, rows, k, eid, qx, dx, rows_eval=rows_eval)


def moe_ffn_mixed(gu_wtype, gu_bank, gu_stride, down_wtype, down_bank, down_stride, sh_wtype,
                  sh_gu, sh_down, n_routed, d_model, d_ff, ids, wts, x):
    """Unchained end-to-end reference of one token through routed experts of
    one format pair and a shared expert (id n_routed) of its own format, in
    its own matrices: quantize x, gate||up rows per selected expert, swiglu,
    quantize h, weighted sum of the down rows.  Returns (y, S)."""
    qx, dx, _ = quantize_act(x)
    gus = []
    for e in ids:
        if int(e) == n_routed:
            ye, _ = expert_rows_any(sh_wtype, sh_gu, 0, 2 * d_ff, d_model, 0, qx, dx)
        else:
            ye, _ = expert_rows_any(gu_wtype, gu_bank, gu_stride, 2 * d_ff, d_model, int(e), qx, dx)
        gus.append(ye)
    h = swiglu(np.stack(gus).astype(np.float32), d_ff)
    qh, dh, _ = quantize_act(h)
    y = np.zeros(d_model, np.float64)
    S = np.zeros(d_model, np.float64)
    for s, e in enumerate(ids):
        if int(e) == n_routed:
            ye, Se = expert_rows_any(sh_wtype, sh_down, 0, d_model, d_ff, 0, qh[s], dh[s])
        else:
            ye, Se = expert_rows_any(down_wtype, down_bank, down_stride, d_model, d_ff, int(e),
                                     qh[s], dh[s])
        y += float(wts[s]) * ye
        S += abs(float(wts[s])) * Se
    return y, S


def moe_ffn(wtype, gu_bank, gu_stride, down_bank, down_stride, d_model, d_ff, ids, wts, x):
    """Unchained end-to-end reference of one token through the selected experts."""
    qx, dx, _ = quantize_act(x)
    gu, _ = moe_gate_up(wtype, gu_bank, gu_stride, d_model, d_ff, ids, qx, dx)
    h = swiglu(gu.astype(np.float32), d_ff)
    qh, dh, _ = quantize_act(h)
    return moe_down_weighted(wtype, down_bank, down_stride, d_model, d_ff, ids, wts, qh, dh)
