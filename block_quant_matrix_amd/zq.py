"""ctypes binding of libzq (include/zq.h): same names, argument marshalling only.

Every function takes device tensors (torch, on the GPU) or raw integer device
pointers, passes their addresses and sizes to the C ABI, and raises ZQError
on a non-zero status.  ``stream`` defaults to torch's current stream.  There
is no fallback: if libzq.so is missing or the device is not gfx950, calls fail.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzq.so")

ZQ_OK, ZQ_EINVAL, ZQ_ENULL, ZQ_EALIGN, ZQ_ERANGE, ZQ_EDEVICE, ZQ_ELAUNCH = 0, -1, -2, -3, -4, -5, -6
ZQ_ACCUMULATE = 1
ZQ_Q4_0, ZQ_Q8_0, ZQ_Q4_K, ZQ_Q5_K, ZQ_Q6_K, ZQ_F16, ZQ_F32 = 4, 8, 12, 13, 14, 16, 32
ZQ_MOE_GATHER, ZQ_MOE_WEIGHTED_SUM = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_INT = ctypes.c_int

# name -> (restype, argtypes); mirrors include/zq.h
SIGNATURES = {
    "zq_version": (_INT, []),
    "zq_strerror": (ctypes.c_char_p, [_INT]),
    "zq_device_check": (_INT, [_INT]),
    "zq_quantize_act": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "zq_dmmv_q8_0": (_INT, [_P, _I64, _I64, _P, _P, _P, _U32, _P]),
    "zq_dmmv_q4_0": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _U32, _P]),
    "zq_dmmv_q4_k": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _U32, _P]),
    "zq_dmmv_q5_k": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _U32, _P]),
    "zq_dmmv_q6_k": (_INT, [_P, _I64, _I64, _P, _P, _P, _U32, _P]),
    "zq_rms_norm_quantize": (_INT, [_P, _P, ctypes.c_float, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "zq_rms_norm_dmmv_f32": (_INT, [_INT, _P, _I64, _I64, _P, _P, ctypes.c_float, _P, _U32, _P, _P,
                                    _P, _P, _P]),
    "zq_rms_norm_dmmv_f32_argmax": (_INT, [_INT, _P, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P,
                                           _SZ, _P]),
    "zq_dmmv_tokens": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P, _I32, _P, _U32, _P]),
    "zq_dmmv_f32": (_INT, [_INT, _P, _I64, _I64, _P, _P, _U32, _P, _P, _P, _P]),
    "zq_dmmv_float": (_INT, [_INT, _P, _I64, _I64, _P, _P, _U32, _P]),
    "zq_moe_ffn_norm_route": (_INT, [_INT, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P, ctypes.c_float, _P,
                                     _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P, _U32, _P]),
    "zq_dmmv_k_f32": (_INT, [_INT, _P, _I64, _I64, _P, _P, _U32, _P, _P, _P, _P]),
    "zq_dmmv_tokens_f32": (_INT, [_INT, _P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _U32, _P]),
    "zq_dmmv_isums": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P, _P]),
    "zq_argmax_workspace_bytes": (_SZ, [_I64]),
    "zq_argmax_f32": (_INT, [_P, _I64, _P, _P, _SZ, _P]),
    "zq_dmmv_f32_argmax_workspace_bytes": (_SZ, []),
    "zq_dmmv_f32_argmax": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "zq_dmmv_f32_argmax_noalloc": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P, _P]),
    "zq_moe_route": (_INT, [_P, _I32, _I32, _P, _P, _P, _P]),
    "zq_dmmv_moe": (_INT, [_INT, _P, _I64, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _P, _I64,
                           _INT, _P, _U32, _P, _P]),
    "zq_swiglu_quantize": (_INT, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "zq_moe_gate_up": (_INT, [_INT, _P, _I64, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, _P,
                              _P, _P]),
    "zq_moe_ffn_workspace_bytes": (_SZ, [_I64, _I64, _I32]),
    "zq_moe_ffn": (_INT, [_INT, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _SZ,
                          _P, _U32, _P, _P]),
    "zq_moe_gate_up_route": (_INT, [_INT, _P, _I64, _I64, _I64, _I64, _P, _I32, _I32, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P]),
    "zq_moe_gate_up_mixed": (_INT, [_INT, _P, _I64, _INT, _P, _I64, _I64, _P, _I32, _I32, _P, _P,
                                    _P, _P, _P, _P, _P, _P]),
    "zq_moe_ffn_route": (_INT, [_INT, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I32, _I32, _P, _P,
                                _P, _P, _P, _SZ, _P, _U32, _P]),
    "zq_moe_ffn_mixed": (_INT, [_INT, _P, _I64, _INT, _P, _I64, _INT, _P, _P, _I64, _I64, _P, _I32,
                                _I32, _P, _P, _P, _P, _P, _SZ, _P, _U32, _P]),
    "zq_moe_ffn_tokens_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32]),
    "zq_moe_ffn_tokens": (_INT, [_INT, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I32, _I32, _P, _P,
                                 _I32, _P, _P, _P, _SZ, _P, _U32, _P]),
    "zq_gemm_prefill": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P, _I64, _P, _U32, _P]),
    "zq_gemm_isums": (_INT, [_INT, _P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "zq_read_probe": (_INT, [_P, _I64, _P, _P]),
}


class ZQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, strerror(status), status))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libzq.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libzq.so is not built (%s); run __graft_entry__.build() or "
                               "python -m block_quant_matrix_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().zq_strerror(status).decode()


def ptr(t) -> int | None:
    """Device address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name: str, *args) -> int:
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise ZQError(name, rc)
    return rc


def zq_version() -> int:
    return lib().zq_version()


def zq_device_check(device: int = 0) -> int:
    return lib().zq_device_check(device)


def zq_quantize_act(x, n_tok, k, x_stride, qx, dx, sx=None, stream=None):
    return _call("zq_quantize_act", ptr(x), n_tok, k, x_stride, ptr(qx), ptr(dx), ptr(sx),
                 _stream(stream))


def zq_dmmv_q8_0(w, rows, k, qx, dx, y, flags=0, stream=None):
    return _call("zq_dmmv_q8_0", ptr(w), rows, k, ptr(qx), ptr(dx), ptr(y), flags, _stream(stream))


def zq_dmmv_q4_0(w, rows, k, qx, dx, sx, y, flags=0, stream=None):
    return _call("zq_dmmv_q4_0", ptr(w), rows, k, ptr(qx), ptr(dx), ptr(sx), ptr(y), flags,
                 _stream(stream))


def zq_dmmv_q4_k(w, rows, k, qx, dx, sx, y, flags=0, stream=None):
    return _call("zq_dmmv_q4_k", ptr(w), rows, k, ptr(qx), ptr(dx), ptr(sx), ptr(y), flags,
                 _stream(stream))


def zq_dmmv_q5_k(w, rows, k, qx, dx, sx, y, flags=0, stream=None):
    return _call("zq_dmmv_q5_k", ptr(w), rows, k, ptr(qx), ptr(dx), ptr(sx), ptr(y), flags,
                 _stream(stream))


def zq_dmmv_q6_k(w, rows, k, qx, dx, y, flags=0, stream=None):
    return _call("zq_dmmv_q6_k", ptr(w), rows, k, ptr(qx), ptr(dx), ptr(y), flags,
                 _stream(stream))


def zq_rms_norm_quantize(x, norm_w, eps, n_tok, k, x_stride, qx, dx, sx=None, xn_out=None,
                         stream=None):
    return _call("zq_rms_norm_quantize", ptr(x), ptr(norm_w), eps, n_tok, k, x_stride, ptr(qx),
                 ptr(dx), ptr(sx), ptr(xn_out), _stream(stream))


def zq_rms_norm_dmmv_f32(wtype, w, rows, k, x, norm_w, eps, y, flags=0, qx_out=None, dx_out=None,
                         sx_out=None, xn_out=None, stream=None):
    return _call("zq_rms_norm_dmmv_f32", wtype, ptr(w), rows, k, ptr(x), ptr(norm_w), eps, ptr(y),
                 flags, ptr(qx_out), ptr(dx_out), ptr(sx_out), ptr(xn_out), _stream(stream))


def zq_rms_norm_dmmv_f32_argmax(wtype, w, rows, k, x, norm_w, eps, y, out_idx, workspace,
                                workspace_bytes, stream=None):
    return _call("zq_rms_norm_dmmv_f32_argmax", wtype, ptr(w), rows, k, ptr(x), ptr(norm_w), eps,
                 ptr(y), ptr(out_idx), ptr(workspace), workspace_bytes, _stream(stream))


def zq_dmmv_tokens(wtype, w, rows, k, qx, dx, sx, n_tok, y, flags=0, stream=None):
    return _call("zq_dmmv_tokens", wtype, ptr(w), rows, k, ptr(qx), ptr(dx), ptr(sx), n_tok, ptr(y),
                 flags, _stream(stream))


def zq_dmmv_f32(wtype, w, rows, k, x, y, flags=0, qx_out=None, dx_out=None, sx_out=None,
                stream=None):
    return _call("zq_dmmv_f32", wtype, ptr(w), rows, k, ptr(x), ptr(y), flags, ptr(qx_out),
                 ptr(dx_out), ptr(sx_out), _stream(stream))


def zq_moe_ffn_norm_route(wtype, gu_bank, gu_stride, down_bank, down_stride, n_experts, d_model,
                          d_ff, router_w, norm_w, eps, x, n_routed, top_k, shared_gate, xn_out,
                          logits_out, ids, wts, workspace, workspace_bytes, y, flags=0,
                          stream=None):
    return _call("zq_moe_ffn_norm_route", wtype, ptr(gu_bank), gu_stride, ptr(down_bank),
                 down_stride, n_experts, d_model, d_ff, ptr(router_w), ptr(norm_w), eps, ptr(x),
                 n_routed, top_k, ptr(shared_gate), ptr(xn_out), ptr(logits_out), ptr(ids),
                 ptr(wts), ptr(workspace), workspace_bytes, ptr(y), flags, _stream(stream))


def zq_dmmv_k_f32(wtype, w, rows, k, x, y, flags=0, qx_out=None, dx_out=None, sx_out=None,
                  stream=None):
    return _call("zq_dmmv_k_f32", wtype, ptr(w), rows, k, ptr(x), ptr(y), flags, ptr(qx_out),
                 ptr(dx_out), ptr(sx_out), _stream(stream))


def zq_dmmv_tokens_f32(wtype, w, rows, k, x, n_tok, qx, dx, sx, y, flags=0, stream=None):
    return _call("zq_dmmv_tokens_f32", wtype, ptr(w), rows, k, ptr(x), n_tok, ptr(qx), ptr(dx),
                 ptr(sx), ptr(y), flags, _stream(stream))


def zq_dmmv_float(wtype, w, rows, k, x, y, flags=0, stream=None):
    return _call("zq_dmmv_float", wtype, ptr(w), rows, k, ptr(x), ptr(y), flags, _stream(stream))


def zq_dmmv_isums(wtype, w, rows, k, qx, sx, isums, stream=None):
    return _call("zq_dmmv_isums", wtype, ptr(w), rows, k, ptr(qx), ptr(sx), ptr(isums),
                 _stream(stream))


def zq_argmax_workspace_bytes(n: int) -> int:
    return lib().zq_argmax_workspace_bytes(n)


def zq_argmax_f32(y, n, out_idx, workspace, workspace_bytes, stream=None):
    return _call("zq_argmax_f32", ptr(y), n, ptr(out_idx), ptr(workspace), workspace_bytes,
                 _stream(stream))


def zq_dmmv_f32_argmax_workspace_bytes() -> int:
    return lib().zq_dmmv_f32_argmax_workspace_bytes()


def zq_dmmv_f32_argmax(wtype, w, rows, k, x, y, out_idx, workspace, workspace_bytes, stream=None):
    return _call("zq_dmmv_f32_argmax", wtype, ptr(w), rows, k, ptr(x), ptr(y), ptr(out_idx),
                 ptr(workspace), workspace_bytes, _stream(stream))


def zq_dmmv_f32_argmax_noalloc(wtype, w, rows, k, x, y, out_idx, stream=None):
    return _call("zq_dmmv_f32_argmax_noalloc", wtype, ptr(w), rows, k, ptr(x), ptr(y), ptr(out_idx),
                 _stream(stream))


def zq_moe_route(logits, n_routed, top_k, shared_gate, ids, wts, stream=None):
    return _call("zq_moe_route", ptr(logits), n_routed, top_k, ptr(shared_gate), ptr(ids), ptr(wts),
                 _stream(stream))


def zq_dmmv_moe(wtype, bank, n_experts, expert_stride_bytes, rows, k, ids, wts, n_sel, qx, dx, sx,
                x_stride, mode, y, flags=0, dev_status=None, stream=None):
    return _call("zq_dmmv_moe", wtype, ptr(bank), n_experts, expert_stride_bytes, rows, k, ptr(ids),
                 ptr(wts), n_sel, ptr(qx), ptr(dx), ptr(sx), x_stride, mode, ptr(y), flags,
                 ptr(dev_status), _stream(stream))


def zq_swiglu_quantize(gu, n, f, qh, dh, sh=None, h_out=None, stream=None):
    return _call("zq_swiglu_quantize", ptr(gu), n, f, ptr(qh), ptr(dh), ptr(sh), ptr(h_out),
                 _stream(stream))


def zq_moe_gate_up(wtype, gu_bank, gu_stride_bytes, n_experts, d_model, d_ff, ids, n_sel, x, qh,
                   dh, sh=None, h_out=None, gu_out=None, dev_status=None, stream=None):
    return _call("zq_moe_gate_up", wtype, ptr(gu_bank), gu_stride_bytes, n_experts, d_model, d_ff,
                 ptr(ids), n_sel, ptr(x), ptr(qh), ptr(dh), ptr(sh), ptr(h_out), ptr(gu_out),
                 ptr(dev_status), _stream(stream))


def zq_moe_gate_up_mixed(gu_wtype, gu_bank, gu_stride_bytes, sh_wtype, sh_gu, d_model, d_ff,
                         logits, n_routed, top_k, shared_gate, x, ids, wts, qh, dh, sh=None,
                         stream=None):
    return _call("zq_moe_gate_up_mixed", gu_wtype, ptr(gu_bank), gu_stride_bytes, sh_wtype,
                 ptr(sh_gu), d_model, d_ff, ptr(logits), n_routed, top_k, ptr(shared_gate),
                 ptr(x), ptr(ids), ptr(wts), ptr(qh), ptr(dh), ptr(sh), _stream(stream))


def zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel) -> int:
    return lib().zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)


def zq_moe_ffn(wtype, gu_bank, gu_stride_bytes, down_bank, down_stride_bytes, n_experts, d_model,
               d_ff, ids, wts, n_sel, x, workspace, workspace_bytes, y, flags=0, dev_status=None,
               stream=None):
    return _call("zq_moe_ffn", wtype, ptr(gu_bank), gu_stride_bytes, ptr(down_bank),
                 down_stride_bytes, n_experts, d_model, d_ff, ptr(ids), ptr(wts), n_sel, ptr(x),
                 ptr(workspace), workspace_bytes, ptr(y), flags, ptr(dev_status), _stream(stream))


def zq_moe_gate_up_route(wtype, gu_bank, gu_stride, n_experts, d_model, d_ff, logits, n_routed,
                         top_k, shared_gate, x, ids, wts, qh, dh, sh=None, h_out=None, gu_out=None,
                         stream=None):
    return _call("zq_moe_gate_up_route", wtype, ptr(gu_bank), gu_stride, n_experts, d_model, d_ff,
                 ptr(logits), n_routed, top_k, ptr(shared_gate), ptr(x), ptr(ids), ptr(wts),
                 ptr(qh), ptr(dh), ptr(sh), ptr(h_out), ptr(gu_out), _stream(stream))


def zq_moe_ffn_route(wtype, gu_bank, gu_stride, down_bank, down_stride, n_experts, d_model, d_ff,
                     logits, n_routed, top_k, shared_gate, x, ids, wts, workspace,
                     workspace_bytes, y, flags=0, stream=None):
    return _call("zq_moe_ffn_route", wtype, ptr(gu_bank), gu_stride, ptr(down_bank), down_stride,
                 n_experts, d_model, d_ff, ptr(logits), n_routed, top_k, ptr(shared_gate), ptr(x),
                 ptr(ids), ptr(wts), ptr(workspace), workspace_bytes, ptr(y), flags,
                 _stream(stream))


def zq_moe_ffn_tokens_workspace_bytes(d_model, d_ff, n_tok, n_sel) -> int:
    return lib().zq_moe_ffn_tokens_workspace_bytes(d_model, d_ff, n_tok, n_sel)


def zq_moe_ffn_tokens(wtype, gu_bank, gu_stride, down_bank, down_stride, n_experts, d_model, d_ff,
                      logits, n_routed, top_k, shared_gate, x, n_tok, ids, wts, workspace,
                      workspace_bytes, y, flags=0, stream=None):
    return _call("zq_moe_ffn_tokens", wtype, ptr(gu_bank), gu_stride, ptr(down_bank), down_stride,
                 n_experts, d_model, d_ff, ptr(logits), n_routed, top_k, ptr(shared_gate), ptr(x),
                 n_tok, ptr(ids), ptr(wts), ptr(workspace), workspace_bytes, ptr(y), flags,
                 _stream(stream))


def zq_gemm_prefill(wtype, w, n, k, qx, dx, sx, m, y, flags=0, stream=None):
    return _call("zq_gemm_prefill", wtype, ptr(w), n, k, ptr(qx), ptr(dx), ptr(sx), m, ptr(y), flags,
                 _stream(stream))


def zq_gemm_isums(wtype, w, n, k, qx, sx, m, m0, m1, n0, n1, isums, stream=None):
    return _call("zq_gemm_isums", wtype, ptr(w), n, k, ptr(qx), ptr(sx), m, m0, m1, n0, n1,
                 ptr(isums), _stream(stream))


def zq_moe_ffn_mixed(gu_wtype, gu_bank, gu_stride, down_wtype, down_bank, down_stride, sh_wtype,
                     sh_gu, sh_down, d_model, d_ff, logits, n_routed, top_k, shared_gate, x, ids,
                     wts, workspace, workspace_bytes, y, flags=0, stream=None):
    return _call("zq_moe_ffn_mixed", gu_wtype, ptr(gu_bank), gu_stride, down_wtype, ptr(down_bank),
                 down_stride, sh_wtype, ptr(sh_gu), ptr(sh_down), d_model, d_ff, ptr(logits),
                 n_routed, top_k, ptr(shared_gate), ptr(x), ptr(ids), ptr(wts), ptr(workspace),
                 workspace_bytes, ptr(y), flags, _stream(stream))


def zq_read_probe(buf, nbytes, sink, stream=None):
    return _call("zq_read_probe", ptr(buf), nbytes, ptr(sink), _stream(stream))
