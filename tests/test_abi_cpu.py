"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/zq.h declares, the binding mirrors the header, and argument errors
come back as the documented codes before anything touches a device.

Pointers here are fake non-zero addresses: every check below fails (or, for
valid arguments, reaches the device check) before any launch, so nothing is
ever dereferenced.
"""
import os
import re
import subprocess

import pytest

from block_quant_matrix_amd import zq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zq.h")

A = 0x10000   # 64 KiB-aligned fake device addresses
B = 0x20000
C = 0x30000
D = 0x40000


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zq_\w+)\s*\(", src)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 15
    L = zq.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", zq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (zq_\w+)", out))
    assert set(names) <= exported
    # nothing exported beyond the header's zq_ functions
    assert exported <= set(names)


def test_binding_mirrors_header():
    assert set(zq.SIGNATURES) == set(header_functions())
    for n in zq.SIGNATURES:
        if n.startswith("zq_") and n not in ("zq_strerror",):
            assert callable(getattr(zq, n)), n


def test_version_and_strerror():
    L = zq.lib()
    assert L.zq_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert zq.strerror(code)
    assert "unknown" in zq.strerror(-99)


def test_workspace_sizes():
    L = zq.lib()
    assert L.zq_argmax_workspace_bytes(1) >= 8
    assert L.zq_argmax_workspace_bytes(248320) >= 8 * 243
    ws = L.zq_moe_ffn_workspace_bytes(2048, 512, 9)
    assert ws >= 2048 + 9 * 1024 * 4 + 9 * 512 and ws % 256 == 0
    assert L.zq_moe_ffn_workspace_bytes(0, 512, 9) == 0
    assert L.zq_dmmv_f32_argmax_workspace_bytes() == 8 * 2048


def test_moe_ffn_route_argument_errors():
    L = zq.lib()
    ws = L.zq_moe_ffn_workspace_bytes(2048, 512, 9)
    gs, ds = 2 * 512 * 64 * 18, 2048 * 16 * 18

    def rc(wtype=4, n_experts=129, d_model=2048, d_ff=512, logits=B, n_routed=128, top_k=8,
           g=C, x=D, ids=A + 0x1000, wts=A + 0x2000, work=A + 0x4000, wsb=ws, y=A + 0x8000,
           flags=0):
        return L.zq_moe_ffn_route(wtype, A, gs, B, ds, n_experts, d_model, d_ff, logits, n_routed,
                                  top_k, g, x, ids, wts, work, wsb, y, flags, None)

    assert rc(wtype=3) == zq.ZQ_EINVAL
    assert rc(top_k=0) == zq.ZQ_EINVAL
    assert rc(top_k=65, n_routed=128) == zq.ZQ_EINVAL
    assert rc(n_routed=1025) == zq.ZQ_EINVAL
    assert rc(n_routed=7) == zq.ZQ_EINVAL              # fewer than top_k
    assert rc(n_experts=128) == zq.ZQ_EINVAL           # no room for the shared expert
    assert rc(d_model=2047) == zq.ZQ_EINVAL
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(wsb=ws - 1) == zq.ZQ_EINVAL
    assert rc(logits=None) == zq.ZQ_ENULL
    assert rc(ids=None) == zq.ZQ_ENULL
    assert rc(x=D + 4) == zq.ZQ_EALIGN
    assert rc(work=A + 0x4010) == zq.ZQ_EALIGN


def test_moe_gate_up_route_argument_errors():
    L = zq.lib()
    gs = 2 * 512 * 64 * 18

    def rc(d_model=2048, n_routed=128, top_k=8, g=C, logits=B, qh=A + 0x1000):
        return L.zq_moe_gate_up_route(4, A, gs, 129, d_model, 512, logits, n_routed, top_k, g, D,
                                      A + 0x2000, A + 0x3000, qh, A + 0x4000, None, None, None,
                                      None)

    assert rc(d_model=8192) == zq.ZQ_EINVAL     # wider than the fused stage takes
    assert rc(top_k=9, n_routed=8) == zq.ZQ_EINVAL
    assert rc(logits=None) == zq.ZQ_ENULL
    assert rc(qh=A + 0x1004) == zq.ZQ_EALIGN


def test_q4k_argument_errors():
    L = zq.lib()

    def rc(w=A, rows=4, k=512, qx=B, dx=C, sx=None, y=D, flags=0):
        return L.zq_dmmv_q4_k(w, rows, k, qx, dx, sx, y, flags, None)

    assert rc(k=288) == zq.ZQ_EINVAL           # not a whole super-block
    assert rc(rows=-1) == zq.ZQ_EINVAL
    assert rc(flags=4) == zq.ZQ_EINVAL
    assert rc(w=A + 8) == zq.ZQ_EALIGN         # super-blocks are read 16 bytes at a time
    assert rc(qx=B + 4) == zq.ZQ_EALIGN
    assert rc(y=None) == zq.ZQ_ENULL
    assert L.zq_dmmv_isums(12, A, 4, 288, B, None, C, None) == zq.ZQ_EINVAL
    assert L.zq_dmmv_isums(12, A + 4, 4, 512, B, None, C, None) == zq.ZQ_EALIGN


def test_q5k_q6k_argument_errors():
    L = zq.lib()

    def rc5(w=A, rows=4, k=512, qx=B, dx=C, sx=None, y=D, flags=0):
        return L.zq_dmmv_q5_k(w, rows, k, qx, dx, sx, y, flags, None)

    def rc6(w=A, rows=4, k=512, qx=B, dx=C, y=D, flags=0):
        return L.zq_dmmv_q6_k(w, rows, k, qx, dx, y, flags, None)

    for rc in (rc5, rc6):
        assert rc(k=480) == zq.ZQ_EINVAL        # not a whole super-block
        assert rc(rows=-1) == zq.ZQ_EINVAL
        assert rc(flags=2) == zq.ZQ_EINVAL
        assert rc(w=A + 2) == zq.ZQ_EALIGN
        assert rc(qx=B + 8) == zq.ZQ_EALIGN
        assert rc(dx=None) == zq.ZQ_ENULL
        assert rc(w=None) == zq.ZQ_ENULL
    assert rc5(sx=C + 2) == zq.ZQ_EALIGN
    for wt in (13, 14):
        assert L.zq_dmmv_isums(wt, A, 4, 480, B, None, C, None) == zq.ZQ_EINVAL
        assert L.zq_dmmv_isums(wt, A + 4, 4, 512, B, None, C, None) == zq.ZQ_EALIGN
        assert L.zq_dmmv_isums(wt, A, 4, 512, B, None, None, None) == zq.ZQ_ENULL
    assert L.zq_dmmv_isums(15, A, 4, 512, B, None, C, None) == zq.ZQ_EINVAL


def test_tokens_argument_errors():
    L = zq.lib()

    def rc(wt=4, w=A, rows=4, k=512, qx=B, dx=C, sx=None, n_tok=2, y=D, flags=0):
        return L.zq_dmmv_tokens(wt, w, rows, k, qx, dx, sx, n_tok, y, flags, None)

    assert rc(n_tok=0) == zq.ZQ_EINVAL
    assert rc(n_tok=9) == zq.ZQ_EINVAL
    assert rc(wt=12) == zq.ZQ_EINVAL          # K-quants have their own entry points
    assert rc(k=48) == zq.ZQ_EINVAL
    assert rc(rows=-1) == zq.ZQ_EINVAL
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(qx=B + 4) == zq.ZQ_EALIGN
    assert rc(w=A + 2) == zq.ZQ_EALIGN
    assert rc(sx=C + 1) == zq.ZQ_EALIGN
    assert rc(dx=None) == zq.ZQ_ENULL
    assert rc(y=None) == zq.ZQ_ENULL


def test_rms_norm_argument_errors():
    L = zq.lib()

    def rq(x=A, nw=B, eps=1e-6, n_tok=2, k=512, stride=512, qx=C, dx=D, sx=None, xn=None):
        return L.zq_rms_norm_quantize(x, nw, eps, n_tok, k, stride, qx, dx, sx, xn, None)

    assert rq(eps=-1.0) == zq.ZQ_EINVAL
    assert rq(eps=float("nan")) == zq.ZQ_EINVAL
    assert rq(eps=float("inf")) == zq.ZQ_EINVAL
    assert rq(k=48) == zq.ZQ_EINVAL
    assert rq(stride=256) == zq.ZQ_EINVAL       # shorter than k
    assert rq(n_tok=-1) == zq.ZQ_EINVAL
    assert rq(nw=None) == zq.ZQ_ENULL
    assert rq(nw=B + 4) == zq.ZQ_EALIGN        # read 16 bytes at a time
    assert rq(stride=514) == zq.ZQ_EALIGN
    assert rq(xn=D + 8) == zq.ZQ_EALIGN

    def rd(wt=4, w=A, rows=4, k=512, x=B, nw=C, eps=1e-6, y=D, flags=0, xn=None):
        return L.zq_rms_norm_dmmv_f32(wt, w, rows, k, x, nw, eps, y, flags, None, None, None, xn,
                                      None)

    assert rd(wt=12) == zq.ZQ_EINVAL
    assert rd(k=16416) == zq.ZQ_EINVAL
    assert rd(eps=-0.5) == zq.ZQ_EINVAL
    assert rd(flags=2) == zq.ZQ_EINVAL
    assert rd(nw=None) == zq.ZQ_ENULL
    assert rd(nw=C + 4) == zq.ZQ_EALIGN
    assert rd(xn=D + 4) == zq.ZQ_EALIGN
    ws = L.zq_dmmv_f32_argmax_workspace_bytes()
    assert L.zq_rms_norm_dmmv_f32_argmax(4, A, 4, 512, B, None, 1e-6, D, None, C, ws,
                                         None) == zq.ZQ_ENULL
    assert L.zq_rms_norm_dmmv_f32_argmax(4, A, 4, 512, B, C, 1e-6, D, None, C, ws - 8,
                                         None) == zq.ZQ_EINVAL
    assert L.zq_rms_norm_dmmv_f32_argmax(4, A, 0, 512, B, C, 1e-6, D, None, C, ws,
                                         None) == zq.ZQ_EINVAL


def test_moe_mixed_argument_errors():
    L = zq.lib()
    ws = L.zq_moe_ffn_workspace_bytes(512, 256, 5)

    def rc(gwt=12, gb=A, gs=2 * 256 * 2 * 144, dwt=13, db=B, ds=512 * 1 * 176, swt=8, sg=C,
           sd=D, dm=512, dff=256, logits=A + 0x100000, nr=16, k=4, g=B + 0x100000,
           x=C + 0x100000, wsb=ws, flags=0, wsp=D + 0x100000):
        return L.zq_moe_ffn_mixed(gwt, gb, gs, dwt, db, ds, swt, sg, sd, dm, dff, logits, nr, k, g,
                                  x, A + 0x200000, B + 0x200000, wsp, wsb, C + 0x200000, flags,
                                  None)

    assert rc(gwt=7) == zq.ZQ_EINVAL
    assert rc(swt=99) == zq.ZQ_EINVAL
    assert rc(dff=288) == zq.ZQ_EINVAL          # Q5_K down needs d_ff % 256 == 0
    assert rc(dm=288) == zq.ZQ_EINVAL           # Q4_K gate/up needs d_model % 256 == 0
    assert rc(gs=1000) == zq.ZQ_EINVAL          # stride shorter than an expert
    assert rc(k=0) == zq.ZQ_EINVAL
    assert rc(nr=3) == zq.ZQ_EINVAL             # fewer experts than top_k
    assert rc(wsb=ws - 1) == zq.ZQ_EINVAL
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(sg=None) == zq.ZQ_ENULL           # shared gate given, shared matrix missing
    assert rc(gb=A + 4) == zq.ZQ_EALIGN         # K-quant banks are 16-byte aligned
    assert rc(wsp=D + 0x100004) == zq.ZQ_EALIGN
    # no shared expert: its matrices may be NULL and its type is not checked
    assert rc(g=None, sg=None, sd=None, swt=99) == zq.ZQ_EDEVICE
    # the K-quant expert-indexed DMMV
    assert L.zq_dmmv_moe(12, A, 4, 144 * 64, 64, 288, B, None, 2, C, D, None, 0, 0, D, 0, None,
                         None) == zq.ZQ_EINVAL    # k not a multiple of 256
    assert L.zq_dmmv_moe(12, A + 8, 4, 144 * 64, 64, 256, B, None, 2, C, D, None, 0, 0, D, 0,
                         None, None) == zq.ZQ_EALIGN
    assert L.zq_dmmv_moe(12, A, 4, 144 * 63, 64, 256, B, None, 2, C, D, None, 0, 0, D, 0, None,
                         None) == zq.ZQ_EINVAL    # stride shorter than an expert


def test_lmhead_argument_errors():
    L = zq.lib()
    ws = L.zq_dmmv_f32_argmax_workspace_bytes()

    def rc(wtype=4, w=A, rows=248320, k=2048, x=B, y=C, out=D, work=A + 0x8000, wsb=ws):
        return L.zq_dmmv_f32_argmax(wtype, w, rows, k, x, y, out, work, wsb, None)

    assert rc(wtype=5) == zq.ZQ_EINVAL
    assert rc(rows=0) == zq.ZQ_EINVAL
    assert rc(rows=1 << 31) == zq.ZQ_EINVAL
    assert rc(k=2047) == zq.ZQ_EINVAL
    assert rc(k=16384 + 32) == zq.ZQ_EINVAL
    assert rc(wsb=ws - 8) == zq.ZQ_EINVAL
    assert rc(x=None) == zq.ZQ_ENULL
    assert rc(y=None) == zq.ZQ_ENULL
    assert rc(work=None) == zq.ZQ_ENULL
    assert rc(x=B + 4) == zq.ZQ_EALIGN
    assert rc(work=A + 0x8004) == zq.ZQ_EALIGN
    assert rc(y=C + 2) == zq.ZQ_EALIGN


def test_lmhead_noalloc_argument_errors():
    L = zq.lib()

    def rc(wtype=4, w=A, rows=248320, k=2048, x=B, y=C, out=D):
        return L.zq_dmmv_f32_argmax_noalloc(wtype, w, rows, k, x, y, out, None)

    assert rc(wtype=5) == zq.ZQ_EINVAL
    assert rc(rows=0) == zq.ZQ_EINVAL
    assert rc(rows=1 << 31) == zq.ZQ_EINVAL
    assert rc(k=2047) == zq.ZQ_EINVAL
    assert rc(k=16384 + 32) == zq.ZQ_EINVAL
    assert rc(x=None) == zq.ZQ_ENULL
    assert rc(y=None) == zq.ZQ_ENULL
    assert rc(out=None) == zq.ZQ_ENULL
    assert rc(x=B + 4) == zq.ZQ_EALIGN
    assert rc(y=C + 2) == zq.ZQ_EALIGN
    assert rc(out=D + 1) == zq.ZQ_EALIGN


def rc_dmmv_q4(**kw):
    a = dict(w=A, rows=4, k=64, qx=B, dx=C, sx=None, y=D, flags=0)
    a.update(kw)
    return zq.lib().zq_dmmv_q4_0(a["w"], a["rows"], a["k"], a["qx"], a["dx"], a["sx"], a["y"],
                                 a["flags"], None)


def test_dmmv_argument_errors():
    assert rc_dmmv_q4(k=33) == zq.ZQ_EINVAL
    assert rc_dmmv_q4(k=0) == zq.ZQ_EINVAL
    assert rc_dmmv_q4(rows=-1) == zq.ZQ_EINVAL
    assert rc_dmmv_q4(flags=2) == zq.ZQ_EINVAL
    assert rc_dmmv_q4(w=None) == zq.ZQ_ENULL
    assert rc_dmmv_q4(qx=None) == zq.ZQ_ENULL
    assert rc_dmmv_q4(y=None) == zq.ZQ_ENULL
    assert rc_dmmv_q4(w=A + 2) == zq.ZQ_EALIGN
    assert rc_dmmv_q4(qx=B + 8) == zq.ZQ_EALIGN
    assert rc_dmmv_q4(y=D + 1) == zq.ZQ_EALIGN
    assert rc_dmmv_q4(sx=C + 2) == zq.ZQ_EALIGN
    L = zq.lib()
    assert L.zq_dmmv_q8_0(A, 4, 48, B, C, D, 0, None) == zq.ZQ_EINVAL
    assert L.zq_dmmv_isums(5, A, 4, 64, B, None, D, None) == zq.ZQ_EINVAL
    assert L.zq_dmmv_isums(4, A, 4, 64, B, None, None, None) == zq.ZQ_ENULL


def test_fused_dmmv_argument_errors():
    L = zq.lib()
    assert L.zq_dmmv_f32(4, A, 4, 16416, B, C, 0, None, None, None, None) == zq.ZQ_EINVAL
    assert L.zq_dmmv_f32(6, A, 4, 64, B, C, 0, None, None, None, None) == zq.ZQ_EINVAL
    assert L.zq_dmmv_f32(4, A, 4, 64, B + 4, C, 0, None, None, None, None) == zq.ZQ_EALIGN
    assert L.zq_dmmv_f32(4, A, 4, 64, B, C, 0, D + 2, None, None, None) == zq.ZQ_EALIGN
    assert L.zq_dmmv_f32(4, A, 4, 64, None, C, 0, None, None, None, None) == zq.ZQ_ENULL
    assert L.zq_dmmv_f32(8, A, 4, 64, B, C, 4, None, None, None, None) == zq.ZQ_EINVAL


def test_other_argument_errors():
    L = zq.lib()
    # quantize: stride < k, misaligned x, stride not a multiple of 4
    assert L.zq_quantize_act(A, 1, 64, 32, B, C, None, None) == zq.ZQ_EINVAL
    assert L.zq_quantize_act(A + 4, 1, 64, 64, B, C, None, None) == zq.ZQ_EALIGN
    assert L.zq_quantize_act(A, 2, 64, 66, B, C, None, None) == zq.ZQ_EALIGN
    assert L.zq_quantize_act(None, 1, 64, 64, B, C, None, None) == zq.ZQ_ENULL
    # argmax: n = 0, workspace too small
    assert L.zq_argmax_f32(A, 0, B, C, 4096, None) == zq.ZQ_EINVAL
    assert L.zq_argmax_f32(A, 248320, B, C, 8, None) == zq.ZQ_EINVAL
    # router: top_k > n_routed, top_k > 64
    assert L.zq_moe_route(A, 4, 8, None, B, C, None) == zq.ZQ_EINVAL
    assert L.zq_moe_route(A, 128, 65, None, B, C, None) == zq.ZQ_EINVAL
    # moe: bad mode, gather with flags, weighted without weights, short stride
    args = dict(wtype=4, bank=A, n_experts=129, stride=1024 * 64 * 18, rows=1024, k=2048, ids=B,
                wts=C, n_sel=9, qx=D, dx=D + 4096, sx=None, x_stride=0, mode=0, y=D + 8192,
                flags=0, status=None)

    def moe(**kw):
        a = dict(args)
        a.update(kw)
        return L.zq_dmmv_moe(a["wtype"], a["bank"], a["n_experts"], a["stride"], a["rows"], a["k"],
                             a["ids"], a["wts"], a["n_sel"], a["qx"], a["dx"], a["sx"],
                             a["x_stride"], a["mode"], a["y"], a["flags"], a["status"], None)

    assert moe(mode=2) == zq.ZQ_EINVAL
    assert moe(flags=1) == zq.ZQ_EINVAL
    assert moe(mode=1, wts=None) == zq.ZQ_ENULL
    assert moe(stride=100) == zq.ZQ_EINVAL
    assert moe(x_stride=48) == zq.ZQ_EINVAL
    assert moe(n_sel=-1) == zq.ZQ_EINVAL
    # fused gate/up: model wider than 4096, missing outputs
    assert L.zq_moe_gate_up(4, A, 8192 * 256 * 18 * 2, 9, 8192, 256, B, 9, C, D, D + 65536, None,
                            None, None, None, None) == zq.ZQ_EINVAL
    assert L.zq_moe_gate_up(4, A, 1024 * 64 * 18, 9, 2048, 512, B, 9, C, None, D, None, None,
                            None, None, None) == zq.ZQ_ENULL
    assert L.zq_moe_gate_up(4, A, 1024 * 64 * 18, 9, 2048, 512, B, 9, C, D + 4, D + 65536, None,
                            None, None, None, None) == zq.ZQ_EALIGN
    # K-quant gate/up: d_model off the fused pass's widths, a bank or a
    # stride off 16 bytes, a stride short of one expert
    kgs = 2 * 512 * (2048 // 256) * 144
    assert L.zq_moe_gate_up(12, A, 2 * 512 * 2 * 144, 9, 512, 512, B, 9, C, D, D + 65536, None,
                            None, None, None, None) == zq.ZQ_EINVAL
    assert L.zq_moe_gate_up(12, A + 4, kgs, 9, 2048, 512, B, 9, C, D, D + 65536, None, None, None,
                            None, None) == zq.ZQ_EALIGN
    assert L.zq_moe_gate_up(12, A, kgs + 8, 9, 2048, 512, B, 9, C, D, D + 65536, None, None, None,
                            None, None) == zq.ZQ_EALIGN
    assert L.zq_moe_gate_up(13, A, kgs, 9, 2048, 512, B, 9, C, D, D + 65536, None, None, None,
                            None, None) == zq.ZQ_EINVAL
    assert L.zq_moe_gate_up(15, A, kgs, 9, 2048, 512, B, 9, C, D, D + 65536, None, None, None,
                            None, None) == zq.ZQ_EINVAL
    # mixed gate/up stage: no shared gate, a width it does not take
    assert L.zq_moe_gate_up_mixed(12, A, kgs, 8, B, 2048, 512, C, 16, 4, None, D, A, B, C, D, None,
                                  None) == zq.ZQ_ENULL
    assert L.zq_moe_gate_up_mixed(12, A, kgs, 8, B, 4096, 512, C, 16, 4, C, D, A, B, C, D, None,
                                  None) == zq.ZQ_EINVAL
    assert L.zq_moe_gate_up_mixed(12, A, kgs, 3, B, 2048, 512, C, 16, 4, C, D, A, B, C, D, None,
                                  None) == zq.ZQ_EINVAL
    # swiglu: f not a multiple of 32
    assert L.zq_swiglu_quantize(A, 9, 48, B, C, None, None, None) == zq.ZQ_EINVAL
    # moe_ffn: workspace too small
    assert L.zq_moe_ffn(4, A, 1024 * 64 * 18, B, 2048 * 16 * 18, 129, 2048, 512, C, C + 64, 9, D,
                        D + 65536, 16, D + 1 << 20, 0, None, None) == zq.ZQ_EINVAL
    # gemm: bad ranges
    assert L.zq_gemm_isums(4, A, 64, 64, B, None, 8, 4, 2, 0, 64, C, None) == zq.ZQ_EINVAL
    assert L.zq_gemm_isums(4, A, 64, 64, B, None, 8, 0, 8, 0, 65, C, None) == zq.ZQ_EINVAL
    assert L.zq_gemm_prefill(3, A, 64, 64, B, C, None, 8, D, 0, None) == zq.ZQ_EINVAL


def test_moe_ffn_tokens_argument_errors():
    L = zq.lib()
    ws = L.zq_moe_ffn_tokens_workspace_bytes(2048, 512, 8, 9)
    assert ws % 256 == 0 and ws >= 8 * 2048 + 72 * 512
    assert L.zq_moe_ffn_tokens_workspace_bytes(2048, 512, -1, 9) == 0
    gs, ds = 2 * 512 * 64 * 18, 2048 * 16 * 18

    def rc(wtype=4, n_experts=129, d_model=2048, d_ff=512, logits=B, n_routed=128, top_k=8,
           g=C, x=D, n_tok=8, ids=A + 0x1000, wts=A + 0x2000, work=A + 0x4000, wsb=ws,
           y=A + 0x8000, flags=0, gs=gs):
        return L.zq_moe_ffn_tokens(wtype, A, gs, B, ds, n_experts, d_model, d_ff, logits,
                                   n_routed, top_k, g, x, n_tok, ids, wts, work, wsb, y, flags,
                                   None)

    assert rc(wtype=12) == zq.ZQ_EINVAL
    assert rc(n_tok=0) == zq.ZQ_EINVAL
    assert rc(n_tok=9) == zq.ZQ_EINVAL
    assert rc(top_k=65, n_routed=128) == zq.ZQ_EINVAL
    assert rc(n_routed=1025, n_experts=1026) == zq.ZQ_EINVAL
    assert rc(n_routed=7) == zq.ZQ_EINVAL              # fewer than top_k
    assert rc(n_experts=128) == zq.ZQ_EINVAL           # no room for the shared expert
    assert rc(d_ff=768) == zq.ZQ_EINVAL                # d_ff outside 256 / 512 / 1024 / 2048
    assert rc(d_model=2047) == zq.ZQ_EINVAL
    assert rc(gs=gs - 18) == zq.ZQ_EINVAL              # expert stride shorter than an expert
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(wsb=ws - 1) == zq.ZQ_EINVAL
    assert rc(logits=None) == zq.ZQ_ENULL
    assert rc(work=None) == zq.ZQ_ENULL
    assert rc(x=D + 4) == zq.ZQ_EALIGN
    assert rc(work=A + 0x4010) == zq.ZQ_EALIGN
    if not os.path.exists("/dev/kfd"):
        assert rc(g=None, n_experts=128) == zq.ZQ_EDEVICE   # valid: the device check is last


def test_moe_ffn_norm_route_argument_errors():
    L = zq.lib()
    ws = L.zq_moe_ffn_workspace_bytes(2048, 512, 9)
    gs, ds = 2 * 512 * 64 * 18, 2048 * 16 * 18

    def rc(wtype=4, n_experts=129, d_model=2048, d_ff=512, router=B, norm=C, eps=1e-6, x=D,
           n_routed=128, top_k=8, g=C + 0x1000, xn=A + 0x1000, lg=A + 0x2000, ids=A + 0x3000,
           wts=A + 0x4000, work=A + 0x8000, wsb=ws, y=D, flags=1):
        return L.zq_moe_ffn_norm_route(wtype, A, gs, B, ds, n_experts, d_model, d_ff, router, norm,
                                       eps, x, n_routed, top_k, g, xn, lg, ids, wts, work, wsb, y,
                                       flags, None)

    assert rc(wtype=13) == zq.ZQ_EINVAL
    assert rc(top_k=0) == zq.ZQ_EINVAL
    assert rc(n_routed=7) == zq.ZQ_EINVAL
    assert rc(n_experts=128) == zq.ZQ_EINVAL           # no room for the shared expert
    assert rc(eps=float("nan")) == zq.ZQ_EINVAL
    assert rc(eps=-1.0) == zq.ZQ_EINVAL
    assert rc(d_model=16384 + 32) == zq.ZQ_EINVAL
    assert rc(wsb=ws - 1) == zq.ZQ_EINVAL
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(router=None) == zq.ZQ_ENULL
    assert rc(norm=None) == zq.ZQ_ENULL
    assert rc(xn=None) == zq.ZQ_ENULL                  # xn and the logits are always written
    assert rc(lg=None) == zq.ZQ_ENULL
    assert rc(norm=C + 4) == zq.ZQ_EALIGN
    assert rc(xn=A + 0x1004) == zq.ZQ_EALIGN
    assert rc(x=D + 4, y=D + 4) == zq.ZQ_EALIGN
    if not os.path.exists("/dev/kfd"):
        assert rc() == zq.ZQ_EDEVICE


def test_float_dmmv_argument_errors():
    L = zq.lib()

    def rc(wtype=16, w=A, rows=64, k=4096, x=B, y=C, flags=0):
        return L.zq_dmmv_float(wtype, w, rows, k, x, y, flags, None)

    assert rc(wtype=4) == zq.ZQ_EINVAL
    assert rc(k=0) == zq.ZQ_EINVAL
    assert rc(k=4100) == zq.ZQ_EINVAL
    assert rc(k=16384 + 8) == zq.ZQ_EINVAL
    assert rc(rows=-1) == zq.ZQ_EINVAL
    assert rc(flags=2) == zq.ZQ_EINVAL
    assert rc(w=None) == zq.ZQ_ENULL
    assert rc(x=None) == zq.ZQ_ENULL
    assert rc(y=None) == zq.ZQ_ENULL
    assert rc(w=A + 8) == zq.ZQ_EALIGN
    assert rc(x=B + 4) == zq.ZQ_EALIGN
    assert rc(y=C + 2) == zq.ZQ_EALIGN


def test_f32_input_forms_argument_errors():
    L = zq.lib()

    def rk(wtype=12, w=A, rows=64, k=4096, x=B, y=C, flags=0, qx=None, dx=None, sx=None):
        return L.zq_dmmv_k_f32(wtype, w, rows, k, x, y, flags, qx, dx, sx, None)

    assert rk(wtype=4) == zq.ZQ_EINVAL                  # block formats take zq_dmmv_f32
    assert rk(k=4096 + 32) == zq.ZQ_EINVAL             # not whole super-blocks
    assert rk(k=16384 + 256) == zq.ZQ_EINVAL
    assert rk(k=0) == zq.ZQ_EINVAL
    assert rk(rows=-1) == zq.ZQ_EINVAL
    assert rk(flags=2) == zq.ZQ_EINVAL
    assert rk(w=None) == zq.ZQ_ENULL
    assert rk(x=None) == zq.ZQ_ENULL
    assert rk(w=A + 4) == zq.ZQ_EALIGN
    assert rk(x=B + 4) == zq.ZQ_EALIGN
    assert rk(qx=D + 2) == zq.ZQ_EALIGN

    def rt(wtype=4, w=A, rows=4096, k=4096, x=B, n_tok=8, qx=C, dx=D, sx=D + 0x1000,
           y=D + 0x2000, flags=0):
        return L.zq_dmmv_tokens_f32(wtype, w, rows, k, x, n_tok, qx, dx, sx, y, flags, None)

    assert rt(wtype=12) == zq.ZQ_EINVAL
    assert rt(n_tok=0) == zq.ZQ_EINVAL
    assert rt(n_tok=9) == zq.ZQ_EINVAL
    assert rt(k=4100) == zq.ZQ_EINVAL
    assert rt(flags=2) == zq.ZQ_EINVAL
    assert rt(qx=None) == zq.ZQ_ENULL                  # the codes are always stored
    assert rt(sx=None) == zq.ZQ_ENULL
    assert rt(x=B + 8) == zq.ZQ_EALIGN
    assert rt(qx=C + 4) == zq.ZQ_EALIGN
    if not os.path.exists("/dev/kfd"):
        assert rk() == zq.ZQ_EDEVICE
        assert rt() == zq.ZQ_EDEVICE


def test_read_probe_argument_errors():
    L = zq.lib()
    assert L.zq_read_probe(A, 24, C, None) == zq.ZQ_EINVAL
    assert L.zq_read_probe(A, -16, C, None) == zq.ZQ_EINVAL
    assert L.zq_read_probe(None, 16, C, None) == zq.ZQ_ENULL
    assert L.zq_read_probe(A, 16, None, None) == zq.ZQ_ENULL
    assert L.zq_read_probe(A + 8, 16, C, None) == zq.ZQ_EALIGN
    assert L.zq_read_probe(A, 16, C + 2, None) == zq.ZQ_EALIGN


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_valid_arguments_without_gpu_report_no_device():
    """With every argument valid, the last check is the device: no GPU here."""
    assert rc_dmmv_q4() == zq.ZQ_EDEVICE
    assert zq.lib().zq_dmmv_q4_k(A, 4, 512, B, C, None, D, 0, None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_dmmv_q5_k(A, 4, 512, B, C, None, D, 0, None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_dmmv_q6_k(A, 4, 512, B, C, D, 0, None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_dmmv_tokens(4, A, 4, 512, B, C, None, 2, D, 0, None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_rms_norm_quantize(A, B, 1e-6, 2, 512, 512, C, D, None, None,
                                         None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_rms_norm_dmmv_f32(4, A, 4, 512, B, C, 1e-6, D, 0, None, None, None, None,
                                         None) == zq.ZQ_EDEVICE
    L = zq.lib()
    assert L.zq_dmmv_f32_argmax(4, A, 248320, 2048, B, C, D, A + 0x8000,
                                L.zq_dmmv_f32_argmax_workspace_bytes(), None) == zq.ZQ_EDEVICE
    assert L.zq_dmmv_f32_argmax(8, A, 7, 8192, B, C, D, A + 0x8000,
                                L.zq_dmmv_f32_argmax_workspace_bytes(), None) == zq.ZQ_EDEVICE
    assert L.zq_dmmv_f32_argmax(4, A, 7, 64, B, C, None, A + 0x8000,
                                L.zq_dmmv_f32_argmax_workspace_bytes(), None) == zq.ZQ_EDEVICE
    assert L.zq_dmmv_f32_argmax_noalloc(4, A, 248320, 2048, B, C, D, None) == zq.ZQ_EDEVICE
    ws = L.zq_moe_ffn_workspace_bytes(2048, 512, 8)
    assert L.zq_moe_ffn_route(4, A, 2 * 512 * 64 * 18, B, 2048 * 16 * 18, 128, 2048, 512, B, 128,
                              8, None, D, A + 0x1000, A + 0x2000, A + 0x4000, ws, A + 0x8000, 0,
                              None) == zq.ZQ_EDEVICE
    assert L.zq_read_probe(A, 1 << 20, C, None) == zq.ZQ_EDEVICE
    assert L.zq_dmmv_float(16, A, 64, 4096, B, C, 0, None) == zq.ZQ_EDEVICE
    assert L.zq_dmmv_float(32, A, 64, 1000, B, C, 1, None) == zq.ZQ_EDEVICE
    assert zq.lib().zq_device_check(0) == zq.ZQ_EDEVICE
