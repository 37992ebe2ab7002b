#!/usr/bin/env python3
"""Throughput of the block-quantized decode path on one MI355X.

Default (workload 2): one step = quantize one fp32 activation of 4096 to int8
blocks, then the Q4_0 DMMV of a 4096 x 4096 weight matrix.  Weights rotate
over distinct copies whose total is more than twice the 256 MB MALL, so every
step streams its weights from HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..13]

Timing: a GPU-side spin kernel is queued ahead of the timed region so that the
K steps are enqueued before the GPU reaches them and run back to back (host
launch cost is not what is measured); HIP events on the launch stream bracket
exactly the K steps.  A second pass times K back-to-back launches of the
dominant kernel alone the same way (roofline.achieved).  The CPU oracle is timed on
a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
MALL_BYTES = 256 << 20

METRIC = "DMMV achieved HBM GB/s (% of MI355X peak) + rows/s, Q4_0 4096x4096"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------- workloads --

class Workload:
    name = ""
    dominant_name = ""       # name of the dominant kernel
    bound = "hbm"
    steps = 2000
    warmup = 50

    def setup(self, torch, zq, inputs):
        raise NotImplementedError

    def step(self, i):
        raise NotImplementedError

    def prepare_dominant(self):
        """Produce the inputs the dominant kernel reads (outside any timing)."""
        raise NotImplementedError

    def dominant(self, i):
        """Launch only the dominant kernel, on the inputs of step i."""
        raise NotImplementedError

    def pct_of_peak(self, value, unit):
        """The step's rate as a percentage of the chip's peak for its unit."""
        return 100.0 * value / (HBM_PEAK_GBS if unit == "GB/s" else INT8_PEAK_TOPS)

    def value(self, ms_per_step):
        """(value, unit) of the whole step."""
        raise NotImplementedError

    def achieved(self, ms_per_launch):
        raise NotImplementedError

    def cpu_baseline(self, seconds):
        raise NotImplementedError


def copies_for(nbytes, lo=2):
    return max(lo, int(np.ceil(2 * MALL_BYTES / nbytes)) + 1)


class DmmvWorkload(Workload):
    """Quantize + DMMV (+ argmax for the LM head)."""

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.wtype, self.rows, self.k = cfg["wtype"], cfg["rows"], cfg["k"]
        self.argmax = wl in (3, 13)
        self.bb = inputs.BLOCK_BYTES[self.wtype]
        self.nb = self.k // 32
        self.wbytes = self.rows * self.nb * self.bb
        # small (decode) matrices: one fused launch quantizes x and runs the
        # DMMV; the LM head: one persistent fused launch whose workgroups
        # quantize x once, stream many row groups and leave argmax partials,
        # then the one-block final argmax
        self.fused = wl in (1, 2)
        # weights + fp32 activation in + fp32 rows out
        self.dmmv_bytes = self.wbytes + 4 * self.k + 4 * self.rows
        if self.fused:
            self.dominant_name = "dmmv_f32x_kernel (quantize + DMMV)"
        else:
            self.dominant_name = "dmmv_f32x_kernel (LM head: quantize + DMMV + argmax partials)"
        self.step_bytes = self.dmmv_bytes
        # (one launch per step: K stays inside one hardware queue)
        self.steps = {1: 3000, 2: 3000, 3: 200, 13: 100}[wl]
        self.warmup = {1: 500, 2: 200, 3: 10, 13: 5}[wl]

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for(self.wbytes)
        host = [inputs.gen_weights(self.wtype, self.rows, self.k, inputs.seed_for(self.wl, c))
                for c in range(self.ncopy)]
        self.w = [torch.from_numpy(h).to("cuda") for h in host]
        self.w_host0 = host[0]
        del host
        self.x_host = inputs.gen_activation(1, self.k, inputs.seed_for(self.wl) + 1)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.y = torch.empty(self.rows, dtype=torch.float32, device="cuda")
        if self.argmax:
            self.ws_bytes = zq.zq_dmmv_f32_argmax_workspace_bytes()
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
            self.idx = torch.empty(1, dtype=torch.int32, device="cuda")

    def step(self, i):
        if self.fused:
            self.zq.zq_dmmv_f32(self.wtype, self.w[i % self.ncopy], self.rows, self.k, self.x,
                                self.y)
        else:
            self.zq.zq_dmmv_f32_argmax(self.wtype, self.w[i % self.ncopy], self.rows, self.k,
                                       self.x, self.y, self.idx, self.ws, self.ws_bytes)

    def prepare_dominant(self):
        pass

    def dominant(self, i):
        if self.fused:
            self.step(i)
        else:
            # the DMMV launch alone (no final argmax block)
            self.zq.zq_dmmv_f32_argmax(self.wtype, self.w[i % self.ncopy], self.rows, self.k,
                                       self.x, self.y, None, self.ws, self.ws_bytes)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.dmmv_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.dmmv_bytes

    def extra(self, ms):
        return {"rows_per_s": self.rows / (ms * 1e-3)}

    def cpu_baseline(self, seconds):
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            qx, dx, sx = oracle.quantize_act(self.x_host)
            y, _ = oracle.dmmv(self.wtype, self.w_host0, self.rows, self.k, qx, dx)
            if self.argmax:
                oracle.argmax_f32(y.astype(np.float32))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=self.step_bytes / per / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d full steps (quantize + %d-row DMMV%s) of this workload on one "
                           "host thread, %.1f s" % (n, self.rows, " + argmax" if self.argmax else "",
                                                    el))


class DmmvKWorkload(Workload):
    """Quantize + DMMV over K-quant super-blocks (Q4_K / Q5_K / Q6_K; two
    launches)."""
    dominant_name = "dmmv_k_kernel"

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.wtype, self.rows, self.k = cfg["wtype"], cfg["rows"], cfg["k"]
        self.tname = {inputs.Q4_K: "Q4_K", inputs.Q5_K: "Q5_K", inputs.Q6_K: "Q6_K"}[self.wtype]
        self.dominant_name = "dmmv_k_kernel (%s)" % self.tname
        self.nb = self.k // 32
        self.wbytes = self.rows * (self.k // 256) * inputs.K_BLOCK_BYTES[self.wtype]
        # the DMMV reads the weights, the int8 codes, scales (and for Q4_K /
        # Q5_K the block sums), and writes fp32 rows; the step adds the fp32
        # activation the quantizer reads and the codes, scales and sums it
        # writes
        sums = 4 * self.nb if self.wtype != inputs.Q6_K else 0
        self.dmmv_bytes = self.wbytes + self.k + 4 * self.nb + sums + 4 * self.rows
        self.step_bytes = self.dmmv_bytes + 4 * self.k + self.k + 8 * self.nb
        # two launches per step: at most 2000 steps keep the timed region's
        # launches within one hardware queue, so all of them are enqueued
        # ahead of the GPU
        if self.wbytes > (64 << 20):
            self.steps, self.warmup = 300, 20
        else:
            self.steps, self.warmup = 2000, 100

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for(self.wbytes)
        host = [inputs.gen_weights_k(self.wtype, self.rows, self.k, inputs.seed_for(self.wl, c))
                for c in range(self.ncopy)]
        self.w = [torch.from_numpy(h).to("cuda") for h in host]
        self.w_host0 = host[0]
        del host
        self.x_host = inputs.gen_activation(1, self.k, inputs.seed_for(self.wl) + 1)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.qx = torch.empty(self.k, dtype=torch.int8, device="cuda")
        self.dx = torch.empty(self.nb, dtype=torch.float32, device="cuda")
        self.sx = torch.empty(self.nb, dtype=torch.int32, device="cuda")
        self.y = torch.empty(self.rows, dtype=torch.float32, device="cuda")

    def _dmmv(self, i):
        w = self.w[i % self.ncopy]
        if self.tname == "Q4_K":
            self.zq.zq_dmmv_q4_k(w, self.rows, self.k, self.qx, self.dx, self.sx, self.y)
        elif self.tname == "Q5_K":
            self.zq.zq_dmmv_q5_k(w, self.rows, self.k, self.qx, self.dx, self.sx, self.y)
        else:
            self.zq.zq_dmmv_q6_k(w, self.rows, self.k, self.qx, self.dx, self.y)

    def step(self, i):
        self.zq.zq_quantize_act(self.x, 1, self.k, self.k, self.qx, self.dx, self.sx)
        self._dmmv(i)

    def prepare_dominant(self):
        self.zq.zq_quantize_act(self.x, 1, self.k, self.k, self.qx, self.dx, self.sx)

    def dominant(self, i):
        self._dmmv(i)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.dmmv_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.dmmv_bytes

    def extra(self, ms):
        return {"rows_per_s": self.rows / (ms * 1e-3)}

    def cpu_baseline(self, seconds):
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            qx, dx, sx = oracle.quantize_act(self.x_host)
            oracle.k_dmmv(self.wtype, self.w_host0, self.rows, self.k, qx, dx)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=self.step_bytes / per / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d full steps (quantize + %d-row %s DMMV) of this workload on one "
                           "host thread, %.1f s" % (n, self.rows, self.tname, el))


class DmmvTokWorkload(Workload):
    """Quantize T tokens + one multi-token DMMV (two launches): the small-M
    decode shapes, Q4_0 4096 x 4096 (the tile form on the matrix cores) and
    the 248 320-row LM head (the tall form on the matrix cores)."""
    dominant_name = "dmmv_tok_kernel"

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.wtype, self.rows, self.k, self.T = cfg["wtype"], cfg["rows"], cfg["k"], cfg["n_tok"]
        self.nb = self.k // 32
        if self.rows >= 65536 and self.T >= 3:
            self.dominant_name = "dmmv_tok_mfma_kernel (matrix cores)"
        elif self.T >= 5 and 64 <= self.nb <= 128 and self.rows * self.k >= 8 << 20:
            # (the library's choice for these shapes; Q8_0 rows of more than
            # 88 blocks exceed its LDS and stay on the vector form)
            if self.wtype == 4 or self.nb <= 88:
                self.dominant_name = "dmmv_tok_tile_kernel (matrix cores)"
        self.wbytes = self.rows * self.nb * inputs.BLOCK_BYTES[self.wtype]
        # the DMMV reads the weights once and every token's codes, scales and
        # sums, and writes T rows of fp32; the step adds the quantizer's fp32
        # reads and its writes
        self.dmmv_bytes = self.wbytes + self.T * (self.k + 8 * self.nb) + 4 * self.T * self.rows
        self.step_bytes = self.dmmv_bytes + self.T * (4 * self.k + self.k + 8 * self.nb)
        self.steps, self.warmup = (2000, 100) if self.rows < 65536 else (400, 20)

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for(self.wbytes)
        host = [inputs.gen_weights(self.wtype, self.rows, self.k, inputs.seed_for(self.wl, c))
                for c in range(self.ncopy)]
        self.w = [torch.from_numpy(h).to("cuda") for h in host]
        self.w_host0 = host[0]
        del host
        self.x_host = inputs.gen_activation(self.T, self.k, inputs.seed_for(self.wl) + 1)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.qx = torch.empty((self.T, self.k), dtype=torch.int8, device="cuda")
        self.dx = torch.empty((self.T, self.nb), dtype=torch.float32, device="cuda")
        self.sx = torch.empty((self.T, self.nb), dtype=torch.int32, device="cuda")
        self.y = torch.empty((self.T, self.rows), dtype=torch.float32, device="cuda")

    def step(self, i):
        self.zq.zq_quantize_act(self.x, self.T, self.k, self.k, self.qx, self.dx, self.sx)
        self.dominant(i)

    def prepare_dominant(self):
        self.zq.zq_quantize_act(self.x, self.T, self.k, self.k, self.qx, self.dx, self.sx)

    def dominant(self, i):
        self.zq.zq_dmmv_tokens(self.wtype, self.w[i % self.ncopy], self.rows, self.k, self.qx,
                               self.dx, self.sx, self.T, self.y)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.dmmv_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.dmmv_bytes

    def extra(self, ms):
        return {"token_rows_per_s": self.T * self.rows / (ms * 1e-3), "us_per_token": ms * 1e3 / self.T}

    def cpu_baseline(self, seconds):
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            qx, dx, _ = oracle.quantize_act(self.x_host)
            for t in range(self.T):
                oracle.dmmv(self.wtype, self.w_host0, self.rows, self.k, qx[t], dx[t])
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=self.step_bytes / per / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d full steps (quantize %d tokens + %d-row DMMV per token) on one "
                           "host thread, %.1f s" % (n, self.T, self.rows, el))


class MoeMixedWorkload(Workload):
    """Router + one token through 8 routed experts stored as the pages' model
    stores them (gate/up Q4_K, down Q5_K) and a Q8_0 shared expert, through
    zq_moe_ffn_mixed (two launches: the gate/up pass over the 8 routed Q4_K
    experts, router folded in, and the Q8_0 shared expert; the Q5_K weighted
    down sum with the shared Q8_0 down rows in the same reduction)."""
    dominant_name = "moe_gate_up_mix_kernel (Q4_K routed + Q8_0 shared, router folded in)"

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.E, self.top_k, self.dm, self.dff = cfg["n_routed"], cfg["top_k"], cfg["d_model"], cfg["d_ff"]
        self.gwt, self.dwt, self.swt = cfg["gu_wtype"], cfg["down_wtype"], cfg["sh_wtype"]
        self.n_sel = self.top_k + 1
        kb = inputs.K_BLOCK_BYTES
        self.gu_m = 2 * self.dff * (self.dm // 256) * kb[self.gwt]
        self.dn_m = self.dm * (self.dff // 256) * kb[self.dwt]
        self.sgu_m = 2 * self.dff * (self.dm // 32) * inputs.BLOCK_BYTES[self.swt]
        self.sdn_m = self.dm * (self.dff // 32) * inputs.BLOCK_BYTES[self.swt]
        # weights a token reads: 8 routed experts' gate/up and down, the
        # shared expert's two matrices; plus the fp32 activation, logits, y
        self.step_bytes = (self.top_k * (self.gu_m + self.dn_m) + self.sgu_m + self.sdn_m +
                           4 * self.dm + 4 * self.E + 4 * self.dm)
        # the gate/up pass: 8 routed experts' and the shared expert's
        # gate||up rows, the fp32 x and the logits in; the quantized h
        # (codes, scales, sums) of 9 slots and the expert list out
        self.gather_bytes = (self.top_k * self.gu_m + self.sgu_m + 4 * self.dm + 4 * self.E +
                             self.n_sel * self.dff + 8 * self.n_sel * (self.dff // 32) +
                             8 * self.n_sel)
        self.steps, self.warmup = 2000, 200     # two launches per step

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for(self.E * (self.gu_m + self.dn_m))
        self.banks = []
        for c in range(self.ncopy):
            gu, gs, dn, ds = inputs.moe_banks_k(inputs.seed_for(self.wl, c), self.E, self.dm,
                                                self.dff, self.gwt, self.dwt)
            self.banks.append((torch.from_numpy(gu).to("cuda"), torch.from_numpy(dn).to("cuda")))
            if c == 0:
                self.host_bank = (gu, gs, dn, ds)
            del gu, dn
        self.gs, self.ds = gs, ds
        sgu = inputs.gen_weights(self.swt, 2 * self.dff, self.dm, inputs.seed_for(self.wl, 40))
        sdn = inputs.gen_weights(self.swt, self.dm, self.dff, inputs.seed_for(self.wl, 41))
        self.host_shared = (sgu, sdn)
        self.sgu, self.sdn = torch.from_numpy(sgu).to("cuda"), torch.from_numpy(sdn).to("cuda")
        lg = [inputs.gen_router(self.E, inputs.seed_for(self.wl, 100 + i)) for i in range(64)]
        self.logits = torch.from_numpy(np.stack([l for l, _ in lg])).to("cuda")
        self.gates = torch.from_numpy(np.array([g for _, g in lg], np.float32)).to("cuda")
        self.host_router = lg[0]
        self.x_host = inputs.gen_activation(1, self.dm, inputs.seed_for(self.wl) + 7)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.ids = torch.empty(self.n_sel, dtype=torch.int32, device="cuda")
        self.wts = torch.empty(self.n_sel, dtype=torch.float32, device="cuda")
        self.ws_bytes = zq.zq_moe_ffn_workspace_bytes(self.dm, self.dff, self.n_sel)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.y = torch.empty(self.dm, dtype=torch.float32, device="cuda")
        self.qh = torch.empty((self.n_sel, self.dff), dtype=torch.int8, device="cuda")
        self.dh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.float32, device="cuda")
        self.sh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.int32, device="cuda")

    def step(self, i):
        gu, dn = self.banks[i % self.ncopy]
        j = i % self.logits.shape[0]
        self.zq.zq_moe_ffn_mixed(self.gwt, gu, self.gs, self.dwt, dn, self.ds, self.swt, self.sgu,
                                 self.sdn, self.dm, self.dff, self.logits[j], self.E, self.top_k,
                                 self.gates[j:j + 1], self.x, self.ids, self.wts, self.ws,
                                 self.ws_bytes, self.y)

    def prepare_dominant(self):
        pass

    def dominant(self, i):
        # the step's gate/up launch, alone
        gu, _ = self.banks[i % self.ncopy]
        j = i % self.logits.shape[0]
        self.zq.zq_moe_gate_up_mixed(self.gwt, gu, self.gs, self.swt, self.sgu, self.dm, self.dff,
                                     self.logits[j], self.E, self.top_k, self.gates[j:j + 1],
                                     self.x, self.ids, self.wts, self.qh, self.dh, self.sh)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.gather_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.gather_bytes

    def extra(self, ms):
        return {"tokens_per_s": 1.0 / (ms * 1e-3)}

    def cpu_baseline(self, seconds):
        import oracle
        gu, gs, dn, ds = self.host_bank
        sgu, sdn = self.host_shared
        logits, g = self.host_router
        n, t0 = 0, time.perf_counter()
        while True:
            ids, wts = oracle.moe_route(logits, self.top_k, g)
            oracle.moe_ffn_mixed(self.gwt, gu, gs, self.dwt, dn, ds, self.swt, sgu, sdn, self.E,
                                 self.dm, self.dff, ids, wts, self.x_host)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=self.step_bytes / per / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d full MoE tokens (route + 8 K-quant experts + Q8_0 shared) on one "
                           "host thread, %.1f s" % (n, el))


class DecodeChainWorkload(Workload):
    """One token through 40 layers (RMS norm + Q8_0 router DMMV, routed MoE
    block of 128 + 1 Q4_0 experts added onto the state) and the LM head with
    its final norm and argmax: 122 launches, replayed as one HIP graph.  The
    eager time of the same chain is reported beside it."""
    dominant_name = "moe_gate_up_kernel (router folded in)"
    bound = "hbm"
    # each layer's gate/up launch is the 128-expert block's, shape for shape:
    # its counted traffic is that workload's
    traffic_workload = "q4_0_moe_128e_top8_shared_2048x512"

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.layers, self.nbanks = cfg["layers"], cfg["moe_banks"]
        self.E, self.top_k, self.dm, self.dff = cfg["n_routed"], cfg["top_k"], cfg["d_model"], cfg["d_ff"]
        self.vocab = cfg["vocab"]
        self.n_sel = self.top_k + 1
        bb = 18
        gu_w = self.n_sel * 2 * self.dff * (self.dm // 32) * bb
        down_w = self.n_sel * self.dm * (self.dff // 32) * bb
        router_w = self.E * (self.dm // 32) * 34
        lm_w = self.vocab * (self.dm // 32) * bb
        # bytes a token must read at least: every layer's router and selected
        # experts, the LM head; plus the fp32 state and logits traffic
        self.token_bytes = self.layers * (router_w + gu_w + down_w) + lm_w + 4 * self.vocab
        self.gate_up_bytes = (gu_w + 4 * self.dm + 4 * self.E + self.n_sel * self.dff +
                              8 * self.n_sel * (self.dff // 32) + 8 * self.n_sel)
        # each replay enqueues every kernel: 24 steps keep the timed region's
        # launches within one hardware queue
        self.steps, self.warmup = 24, 3

    def setup(self, torch, zq, inputs):
        from block_quant_matrix_amd.chain import DecodeChain
        self.torch, self.zq = torch, zq
        rng = np.random.default_rng(inputs.seed_for(self.wl, 9))
        banks, self.host_banks = [], []
        for c in range(self.nbanks):
            gu, gs, down, ds = inputs.moe_banks(inputs.seed_for(self.wl, c), self.E + 1, self.dm,
                                                self.dff)
            banks.append((torch.from_numpy(gu).to("cuda"), gs, torch.from_numpy(down).to("cuda"),
                          ds, self.E + 1))
            self.host_banks.append((gu, gs, down, ds))
        self.ncopy = self.nbanks
        routers = [inputs.gen_weights(inputs.Q8_0, self.E, self.dm, inputs.seed_for(self.wl, 20 + l))
                   for l in range(self.layers)]
        norms = [(1 + 0.1 * rng.standard_normal(self.dm)).astype(np.float32)
                 for _ in range(self.layers + 1)]
        gates = rng.standard_normal(self.layers).astype(np.float32)
        lm = inputs.gen_weights(inputs.Q4_0, self.vocab, self.dm, inputs.seed_for(self.wl, 30))
        self.host = dict(routers=routers, norms=norms, gates=gates, lm=lm)
        dev = lambda a: torch.from_numpy(a).to("cuda")
        self.chain = DecodeChain(torch, [dev(r) for r in routers], [banks[l % self.nbanks]
                                 for l in range(self.layers)], dev(lm),
                                 [dev(n) for n in norms[:-1]], dev(norms[-1]), d_model=self.dm,
                                 n_routed=self.E, top_k=self.top_k, d_ff=self.dff,
                                 vocab=self.vocab,
                                 shared_gate=[dev(gates[l:l + 1]) for l in range(self.layers)])
        self.x0_host = inputs.gen_activation(1, self.dm, inputs.seed_for(self.wl) + 1)
        self.x0 = dev(self.x0_host)
        self.chain.x.copy_(self.x0)
        self.chain.step()  # eager warm-up, then capture
        torch.cuda.synchronize()
        self.chain.x.copy_(self.x0)
        self.chain.capture()
        torch.cuda.synchronize()
        # dominant kernel alone: the gate/up pass of one layer's MoE
        self.qh = torch.empty((self.n_sel, self.dff), dtype=torch.int8, device="cuda")
        self.dh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.float32, device="cuda")
        self.sh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.int32, device="cuda")
        self.banks = banks

    def step(self, i):
        self.chain.replay()

    def prepare_dominant(self):
        pass

    def dominant(self, i):
        gu, gs, _, _, ne = self.banks[i % self.nbanks]
        c = self.chain
        self.zq.zq_moe_gate_up_route(4, gu, gs, ne, self.dm, self.dff, c.logits, self.E,
                                     self.top_k, c.shared_gate[0], c.xn, c.ids, c.wts, self.qh,
                                     self.dh, self.sh)

    def value(self, ms):
        return 1.0 / (ms * 1e-3), "tok/s"

    def pct_of_peak(self, value, unit):
        # the bytes one token must read, at that token rate, against HBM peak
        return 100.0 * self.token_bytes * value / 1e9 / HBM_PEAK_GBS

    def achieved(self, ms):
        return self.gate_up_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.gate_up_bytes

    def extra(self, ms):
        torch = self.torch
        K = self.steps
        # the same chain launched eagerly, timed the same way
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            self.chain.step()
        host_eager = (time.perf_counter() - t0) * 1e3 / K
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            self.chain.replay()
        host_graph = (time.perf_counter() - t0) * 1e3 / K
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        gpu_blocker(torch, 1.5 * host_eager * K + 5)
        e0.record()
        for i in range(K):
            self.chain.step()
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / K
        return {"launches_per_token": self.chain.launches_per_step(),
                "graph_us_per_token": ms * 1e3, "eager_us_per_token": eager_ms * 1e3,
                "host_submit_us_graph": host_graph * 1e3, "host_submit_us_eager": host_eager * 1e3,
                "token_GB_per_s": self.token_bytes / (ms * 1e-3) / 1e9}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        n, t0 = 0, time.perf_counter()
        while True:
            x = self.x0_host.astype(np.float32).copy()
            for l in range(self.layers):
                xn = oracle.rms_norm(x, h["norms"][l], 1e-6).astype(np.float32)
                qx, dx, _ = oracle.quantize_act(xn)
                logits, _ = oracle.dmmv(8, h["routers"][l], self.E, self.dm, qx, dx)
                ids, wts = oracle.moe_route(logits.astype(np.float32), self.top_k, h["gates"][l])
                gu, gs, down, ds = self.host_banks[l % self.nbanks]
                y, _ = oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, ids, wts, xn)
                x = (x + y).astype(np.float32)
            xn = oracle.rms_norm(x, h["norms"][-1], 1e-6).astype(np.float32)
            qx, dx, _ = oracle.quantize_act(xn)
            yl, _ = oracle.dmmv(4, h["lm"], self.vocab, self.dm, qx, dx)
            int(np.argmax(yl))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=1.0 / per, unit="tok/s", cores=1, kind="oracle",
                    sample="%d tokens through the %d-layer chain and the LM head on one host "
                           "thread, %.1f s" % (n, self.layers, el))


class MoeWorkload(Workload):
    """Router + one token through 8 routed + 1 shared Q4_0 experts, in two
    launches: gate/up with the router folded in, then down."""
    dominant_name = "moe_gate_up_kernel (router folded in)"
    steps = 2000
    warmup = 100

    def __init__(self):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[4]
        self.name = cfg["name"]
        self.E, self.top_k, self.dm, self.dff = cfg["n_routed"], cfg["top_k"], cfg["d_model"], cfg["d_ff"]
        self.n_sel = self.top_k + 1
        bb = 18
        self.gu_w = self.n_sel * 2 * self.dff * (self.dm // 32) * bb
        self.down_w = self.n_sel * self.dm * (self.dff // 32) * bb
        self.step_bytes = self.gu_w + self.down_w + 4 * self.dm + 4 * self.dm
        # fused gate/up pass: weights + fp32 x + router logits in, quantized h
        # out (codes, scales, sums) + the expert list and weights
        self.gate_up_bytes = (self.gu_w + 4 * self.dm + 4 * self.E + self.n_sel * self.dff +
                              8 * self.n_sel * (self.dff // 32) + 8 * self.n_sel)

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        bank_bytes = (self.E + 1) * (2 * self.dff * (self.dm // 32) + self.dm * (self.dff // 32)) * 18
        self.ncopy = copies_for(bank_bytes)
        self.banks = []
        for c in range(self.ncopy):
            gu, gs, down, ds = inputs.moe_banks(inputs.seed_for(4, c), self.E + 1, self.dm, self.dff)
            self.banks.append((torch.from_numpy(gu).to("cuda"), torch.from_numpy(down).to("cuda")))
            if c == 0:
                self.host_bank = (gu, gs, down, ds)
        self.gs, self.ds = gs, ds
        nlog = 64
        lg = [inputs.gen_router(self.E, inputs.seed_for(4, 100 + i)) for i in range(nlog)]
        self.logits = torch.from_numpy(np.stack([l for l, _ in lg])).to("cuda")
        self.gates = torch.from_numpy(np.array([g for _, g in lg], np.float32)).to("cuda")
        self.host_router = lg[0]
        self.x_host = inputs.gen_activation(1, self.dm, inputs.seed_for(4) + 7)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.ids = torch.empty(self.n_sel, dtype=torch.int32, device="cuda")
        self.wts = torch.empty(self.n_sel, dtype=torch.float32, device="cuda")
        self.ws_bytes = zq.zq_moe_ffn_workspace_bytes(self.dm, self.dff, self.n_sel)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.y = torch.empty(self.dm, dtype=torch.float32, device="cuda")
        # outputs of the gate/up pass when it is timed alone
        self.qh = torch.empty((self.n_sel, self.dff), dtype=torch.int8, device="cuda")
        self.dh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.float32, device="cuda")
        self.sh = torch.empty((self.n_sel, self.dff // 32), dtype=torch.int32, device="cuda")

    def step(self, i):
        gu, down = self.banks[i % self.ncopy]
        j = i % self.logits.shape[0]
        self.zq.zq_moe_ffn_route(4, gu, self.gs, down, self.ds, self.E + 1, self.dm, self.dff,
                                 self.logits[j], self.E, self.top_k, self.gates[j:j + 1], self.x,
                                 self.ids, self.wts, self.ws, self.ws_bytes, self.y)

    def prepare_dominant(self):
        pass

    def dominant(self, i):
        gu, _ = self.banks[i % self.ncopy]
        j = i % self.logits.shape[0]
        self.zq.zq_moe_gate_up_route(4, gu, self.gs, self.E + 1, self.dm, self.dff, self.logits[j],
                                     self.E, self.top_k, self.gates[j:j + 1], self.x, self.ids,
                                     self.wts, self.qh, self.dh, self.sh)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.gate_up_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.gate_up_bytes

    def extra(self, ms):
        return {"tokens_per_s": 1.0 / (ms * 1e-3)}

    def cpu_baseline(self, seconds):
        import oracle
        gu, gs, down, ds = self.host_bank
        logits, g = self.host_router
        n, t0 = 0, time.perf_counter()
        while True:
            ids, wts = oracle.moe_route(logits, self.top_k, g)
            oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, ids, wts, self.x_host)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per = el / n
        return dict(value=self.step_bytes / per / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d full MoE tokens (route + 9 experts) on one host thread, %.1f s"
                           % (n, el))


class GemmWorkload(Workload):
    dominant_name = "gemm_kernel"
    bound = "mfma"
    steps = 100
    warmup = 10

    def __init__(self):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[5]
        self.name = cfg["name"]
        self.m, self.n, self.k = cfg["m"], cfg["n"], cfg["k"]
        self.ops = 2 * self.m * self.n * self.k

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        wbytes = self.n * (self.k // 32) * 18
        self.ncopy = copies_for(wbytes)
        host = [inputs.gen_weights(4, self.n, self.k, inputs.seed_for(5, c)) for c in range(self.ncopy)]
        self.w = [torch.from_numpy(h).to("cuda") for h in host]
        self.w_host0 = host[0]
        del host
        self.x_host = inputs.gen_activation(self.m, self.k, inputs.seed_for(5) + 1)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.qx = torch.empty((self.m, self.k), dtype=torch.int8, device="cuda")
        self.dx = torch.empty((self.m, self.k // 32), dtype=torch.float32, device="cuda")
        self.y = torch.empty((self.m, self.n), dtype=torch.float32, device="cuda")

    def step(self, i):
        self.zq.zq_quantize_act(self.x, self.m, self.k, self.k, self.qx, self.dx, None)
        self.zq.zq_gemm_prefill(4, self.w[i % self.ncopy], self.n, self.k, self.qx, self.dx, None,
                                self.m, self.y)

    def prepare_dominant(self):
        self.zq.zq_quantize_act(self.x, self.m, self.k, self.k, self.qx, self.dx, None)

    def dominant(self, i):
        self.zq.zq_gemm_prefill(4, self.w[i % self.ncopy], self.n, self.k, self.qx, self.dx, None,
                                self.m, self.y)

    def value(self, ms):
        return self.ops / (ms * 1e-3) / 1e12, "TOP/s"

    def achieved(self, ms):
        return self.ops / (ms * 1e-3) / 1e12, INT8_PEAK_TOPS, "TOP/s", self.ops

    def extra(self, ms):
        # The ceiling the fp32 rescale sets: every (token, row, block) triple
        # needs a convert, a multiply and an FMA, unpacked, at 64 lanes per
        # clock per CU (256 CUs, 2.4 GHz).
        triples = self.m * self.n * (self.k // 32)
        valu_s = 3 * triples / (256 * 64 * 2.4e9)
        ceiling = 2 * self.m * self.n * self.k / valu_s / 1e12
        steps_tops = 2 * self.m * self.n * self.k / (ms * 1e-3) / 1e12
        return {"tokens_per_s": self.m / (ms * 1e-3),
                "valu_epilogue_ceiling_TOPs": round(ceiling, 1),
                "step_frac_of_epilogue_ceiling": round(steps_tops / ceiling, 4)}

    def cpu_baseline(self, seconds):
        import oracle
        rng = np.random.default_rng(0)
        qx, dx, _ = oracle.quantize_act(self.x_host)
        n_pairs, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            mi = rng.integers(0, self.m, 256)
            ni = rng.integers(0, self.n, 256)
            oracle.gemm_entries(4, self.w_host0, self.n, self.k, qx, dx, self.m, mi, ni)
            n_pairs += 256
        el = time.perf_counter() - t0
        ops_per_s = n_pairs * 2 * self.k / el
        return dict(value=ops_per_s / 1e12, unit="TOP/s", cores=1, kind="oracle",
                    sample="%d output entries (of %d) of this GEMM on one host thread, %.1f s"
                           % (n_pairs, self.m * self.n, el))


def counted_traffic(kernel_name, workload):
    """HBM bytes per launch of the kernel at this workload from the committed
    counter runs (profiles/traffic.json, keyed by workload), or None when
    there is none or the kernel's sources have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel_name:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        try:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sha256"] else None


def make_workload(wl):
    if wl in (1, 2, 3, 13):
        return DmmvWorkload(wl)
    if wl == 4:
        return MoeWorkload()
    if wl in (6, 7, 8):
        return DmmvKWorkload(wl)
    if wl in (9, 12):
        return DmmvTokWorkload(wl)
    if wl == 10:
        return DecodeChainWorkload(wl)
    if wl == 11:
        return MoeMixedWorkload(wl)
    return GemmWorkload()


# ----------------------------------------------------------------- timing --

_SLEEP_CYCLES_PER_MS = None


def gpu_blocker(torch, ms):
    """Queue about `ms` of GPU work (torch's spin kernel) so the launches that
    follow are all enqueued before the GPU reaches them."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:  # calibrate the spin kernel's clock once
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(10_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 10_000_000 / max(e0.elapsed_time(e1), 1e-3)
    ms = min(max(ms, 1.0), 2000.0)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def host_launch_ms(w, torch, n=50):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        w.step(i)
    el = (time.perf_counter() - t0) * 1e3 / n
    torch.cuda.synchronize()
    return el


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from block_quant_matrix_amd import inputs, zq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if zq.zq_device_check(0) != 0:
        print("device 0 is not gfx950", file=sys.stderr)
        sys.exit(1)

    w = make_workload(args.workload)
    K = args.steps if args.steps is not None else w.steps
    W = args.warmup if args.warmup is not None else w.warmup
    w.setup(torch, zq, inputs)

    if args.calibrate_copy:  # a plain copy of known size, for counter scaling
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst

    for i in range(W):
        w.step(i)
    torch.cuda.synchronize()
    h_ms = host_launch_ms(w, torch)

    # --- timed region: exactly K steps between two events ---
    t_ev0 = torch.cuda.Event(enable_timing=True)
    t_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_blocker(torch, 1.5 * h_ms * K + 5)
    t_ev0.record()
    for i in range(K):
        w.step(i)
    t_ev1.record()
    torch.cuda.synchronize()
    ms_per_step = t_ev0.elapsed_time(t_ev1) / K

    # --- dominant kernel alone: K back-to-back launches between two events.
    # (An event pair around each launch adds several microseconds of marker
    # processing to a microsecond-scale kernel; back-to-back launches include
    # only the dispatch gap, which the kernel-trace durations also carry.)
    w.prepare_dominant()
    d_ev0 = torch.cuda.Event(enable_timing=True)
    d_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_blocker(torch, 1.5 * h_ms * K + 5)
    d_ev0.record()
    for i in range(K):
        w.dominant(i)
    d_ev1.record()
    torch.cuda.synchronize()
    ms_kernel = d_ev0.elapsed_time(d_ev1) / K

    # --- the launch floor: K back-to-back launches of an empty kernel (torch's
    # spin kernel with a zero count, one thread) on the same stream.  What a
    # launch of any kernel costs before it reads a byte; at the 4096 x 4096
    # size it is a large part of the DMMV's time.
    f_ev0 = torch.cuda.Event(enable_timing=True)
    f_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_blocker(torch, 0.05 * K + 5)
    f_ev0.record()
    for i in range(K):
        torch.cuda._sleep(0)
    f_ev1.record()
    torch.cuda.synchronize()
    ms_floor = f_ev0.elapsed_time(f_ev1) / K

    value, unit = w.value(ms_per_step)
    ach, peak, runit, per_launch = w.achieved(ms_kernel)
    out = {
        "metric": METRIC if args.workload == 2 else "%s throughput (%s)" % (w.name, unit),
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "weight_copies": w.ncopy, "parallelism": "none"},
        "pct_of_peak": round(w.pct_of_peak(value, unit), 2),
    }
    out.update({k: round(v, 4 if abs(v) < 10 else 1) for k, v in w.extra(ms_per_step).items()})
    out["roofline"] = {"bound": w.bound, "kernel": w.dominant_name, "achieved": round(ach, 3),
                       "peak": peak, "unit": runit, "frac": round(ach / peak, 4),
                       "per_launch": per_launch, "ms_per_launch": round(ms_kernel, 6),
                       "empty_launch_ms": round(ms_floor, 6),
                       "frac_after_empty_launch": (round(per_launch / ((ms_kernel - ms_floor) * 1e-3)
                                                         / (1e9 if runit == "GB/s" else 1e12) / peak, 4)
                                                   if ms_kernel > ms_floor else None),
                       "traffic": counted_traffic(w.dominant_name,
                                                  getattr(w, "traffic_workload", w.name))}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = w.cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
