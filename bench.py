#!/usr/bin/env python3
"""Throughput of the block-quantized decode path on one MI355X.

Default (workload 2): one step = the fused quantize + Q4_0 DMMV of a 4096 x
4096 weight matrix from an fp32 activation (one launch).  Weights rotate over
distinct copies whose total is more than twice the 256 MB MALL, so every step
streams its weights from HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..13]

Timing: a GPU-side spin kernel is queued ahead of the timed region so that the
K steps are enqueued before the GPU reaches them and run back to back (host
launch cost is not what is measured); HIP events on the launch stream bracket
exactly the K steps.  When a step is one launch of the dominant kernel the
roofline comes from that same timed region; otherwise a second pass times K
back-to-back launches of the dominant kernel alone the same way.

The oracle leg (cpu_baseline) runs before the timed region: it checks the
GPU's outputs of the first step against the CPU oracle on the same inputs
(parity_checked) and times the oracle on a bounded sample of the workload,
on one host thread and on all of the host's cores (median of 3 runs each).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
MALL_BYTES = 256 << 20
ROW_TOL = 1e-4               # fp32 rows against the fp64 oracle (normwise and well-conditioned)
MOE_E2E_TOL = 1e-3           # an unchained MoE block (an exp ulp may flip one re-quantized code)

METRIC = "DMMV achieved HBM GB/s (% of MI355X peak) + rows/s, Q4_0 4096x4096"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=2, choices=list(range(1, 17)))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (no parity check, no CPU timing)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the rocm-smi clock readings (a child process; for profiler runs)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the LM-head measurement the default line carries")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="about how long the oracle leg's timing runs take in all")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------ parity bars --

def rows_within(y, y_ref, S, tol=ROW_TOL):
    """The fp32 row bar: every output written; normwise |y - y_ref| <= tol*S;
    elementwise |y - y_ref| <= tol*|y_ref| where |y_ref| >= 0.1*S.  Returns
    (ok, worst error in units of S)."""
    y = np.asarray(y, np.float64).ravel()
    y_ref = np.asarray(y_ref, np.float64).ravel()
    S = np.asarray(S, np.float64).ravel()
    if np.isnan(y).any():
        return False, float("nan")
    err = np.abs(y - y_ref)
    worst = float((err / np.maximum(S, 1e-300)).max()) if y.size else 0.0
    ok = bool((err <= tol * S).all())
    well = np.abs(y_ref) >= 0.1 * S
    ok = ok and bool((err[well] <= tol * np.abs(y_ref[well])).all())
    return ok, worst


def first_max(y):
    """Lowest index of the largest value."""
    return int(np.argmax(np.asarray(y)))


def argmax_ok(idx, y_gpu, y_ref, S, tol):
    """The GPU's index is the argmax of its own logits (ties to the lowest
    row), and the oracle's unless the oracle's top two are within tol of
    each other's error scales."""
    if idx != first_max(y_gpu):
        return False
    top = np.argsort(-np.asarray(y_ref), kind="stable")[:2]
    if y_ref[top[0]] - y_ref[top[1]] >= tol * (S[top[0]] + S[top[1]]):
        return idx == int(top[0])
    return True


# ------------------------------------------------------------- workloads --

class Workload:
    name = ""
    dominant_name = ""       # name of the dominant kernel
    bound = "hbm"
    steps = 2000
    warmup = 50
    step_is_dominant = False  # a step is exactly one launch of the dominant kernel
    step_is_graph = False     # a step is itself one graph replay (timed eagerly)
    dtype = "int8"            # the arithmetic the dominant kernel's products run in

    def setup(self, torch, zq, inputs):
        raise NotImplementedError

    def step(self, i):
        raise NotImplementedError

    def prepare_dominant(self):
        """Produce the inputs the dominant kernel reads (outside any timing)."""

    def dominant(self, i):
        """Launch only the dominant kernel, on the inputs of step i."""
        self.step(i)

    def pct_of_peak(self, value, unit):
        """The step's rate as a percentage of the chip's peak for its unit."""
        return 100.0 * value / (HBM_PEAK_GBS if unit == "GB/s" else INT8_PEAK_TOPS)

    def value(self, ms_per_step):
        """(value, unit) of the whole step."""
        raise NotImplementedError

    def achieved(self, ms_per_launch):
        raise NotImplementedError

    def extra(self, ms):
        return {}

    # the oracle leg
    def gpu_result(self):
        """Run step 0 on the GPU and return its outputs on the host."""
        raise NotImplementedError

    def oracle_step(self):
        """One step of the oracle on the inputs of step 0."""
        raise NotImplementedError

    def parity(self, gpu, ref):
        """(ok, detail): the GPU's outputs against the oracle's."""
        raise NotImplementedError

    def cpu_value(self, s_per_step):
        """The oracle's rate in the unit of the GPU's metric."""
        return self.step_bytes / s_per_step / 1e9, "GB/s"

    def cpu_sample(self):
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
        self.step_is_dominant = self.fused
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

    def gpu_result(self):
        self.y.fill_(float("nan"))
        if self.argmax:
            self.idx.fill_(-1)
        self.step(0)
        self.torch.cuda.synchronize()
        out = {"y": self.y.cpu().numpy().copy()}
        if self.argmax:
            out["idx"] = int(self.idx.cpu().numpy()[0])
        return out

    def oracle_step(self, rows_eval=None):
        import oracle
        qx, dx, _ = oracle.quantize_act(self.x_host)
        y, S = oracle.dmmv(self.wtype, self.w_host0, self.rows, self.k, qx, dx, rows_eval=rows_eval)
        out = {"y": y, "S": S}
        if self.argmax and rows_eval is None:
            out["idx"] = oracle.argmax_f32(y.astype(np.float32))
        return out

    def parity(self, gpu, ref, rows_eval=None):
        y = gpu["y"] if rows_eval is None else gpu["y"][rows_eval]
        ok, worst = rows_within(y, ref["y"], ref["S"])
        detail = "%d rows within %g*S (worst %.3g*S)" % (y.size, ROW_TOL, worst)
        if self.argmax:
            if "idx" in ref:
                ok = ok and argmax_ok(gpu["idx"], gpu["y"], ref["y"], ref["S"], ROW_TOL)
                detail += "; argmax %d = oracle's" % gpu["idx"]
            else:
                ok = ok and gpu["idx"] == first_max(gpu["y"])
                detail += "; argmax %d = argmax of the GPU's logits" % gpu["idx"]
        return ok, detail

    def cpu_sample(self):
        return "quantize + %d-row DMMV%s over this workload's first weight copy" % (
            self.rows, " + argmax" if self.argmax else "")


class DmmvKWorkload(Workload):
    """DMMV over K-quant super-blocks (Q4_K / Q5_K / Q6_K) from the fp32
    activation: one launch of zq_dmmv_k_f32, the quantization inside it."""
    dominant_name = "dmmv_k_f32_kernel"
    step_is_dominant = True

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.wtype, self.rows, self.k = cfg["wtype"], cfg["rows"], cfg["k"]
        self.tname = {inputs.Q4_K: "Q4_K", inputs.Q5_K: "Q5_K", inputs.Q6_K: "Q6_K"}[self.wtype]
        self.dominant_name = "dmmv_k_f32_kernel (%s, quantize + DMMV)" % self.tname
        self.nb = self.k // 32
        self.wbytes = self.rows * (self.k // 256) * inputs.K_BLOCK_BYTES[self.wtype]
        # the step reads the weights and the fp32 activation and writes fp32
        # rows (the codes live in each workgroup's LDS)
        self.dmmv_bytes = self.wbytes + 4 * self.k + 4 * self.rows
        self.step_bytes = self.dmmv_bytes
        if self.wbytes > (64 << 20):
            self.steps, self.warmup = 300, 20
        else:
            self.steps, self.warmup = 3000, 100

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

    def step(self, i):
        self.zq.zq_dmmv_k_f32(self.wtype, self.w[i % self.ncopy], self.rows, self.k, self.x,
                              self.y)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.dmmv_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.dmmv_bytes

    def extra(self, ms):
        return {"rows_per_s": self.rows / (ms * 1e-3)}

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.qx.fill_(0)
        self.zq.zq_dmmv_k_f32(self.wtype, self.w[0], self.rows, self.k, self.x, self.y, 0,
                              self.qx, self.dx, self.sx)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy(), "qx": self.qx.cpu().numpy().copy(),
                "dx": self.dx.cpu().numpy().copy(), "sx": self.sx.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        qx, dx, sx = oracle.quantize_act(self.x_host)
        y, S = oracle.k_dmmv(self.wtype, self.w_host0, self.rows, self.k, qx, dx)
        return {"y": y, "S": S, "qx": qx, "dx": dx, "sx": sx}

    def parity(self, gpu, ref):
        codes = (np.array_equal(gpu["qx"], ref["qx"]) and np.array_equal(gpu["sx"], ref["sx"])
                 and np.array_equal(gpu["dx"].view(np.uint32),
                                    np.asarray(ref["dx"], np.float32).view(np.uint32)))
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"])
        return ok and codes, "stored codes %s; %d rows within %g*S (worst %.3g*S)" % (
            "bit-exact" if codes else "DIFFER", self.rows, ROW_TOL, worst)

    def cpu_sample(self):
        return "quantize + %d-row %s DMMV over this workload's first weight copy" % (
            self.rows, self.tname)


class DmmvTokWorkload(Workload):
    """T fp32 tokens through zq_dmmv_tokens_f32 (two launches: the quantizer,
    then one multi-token DMMV): the small-M decode shapes, Q4_0 4096 x 4096
    (the tile form on the matrix cores) and the 248 320-row LM head (the tall
    form on the matrix cores)."""
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
        self.zq.zq_dmmv_tokens_f32(self.wtype, self.w[i % self.ncopy], self.rows, self.k, self.x,
                                   self.T, self.qx, self.dx, self.sx, self.y)

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

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        qx, dx, _ = oracle.quantize_act(self.x_host)
        ys, Ss = [], []
        for t in range(self.T):
            y, S = oracle.dmmv(self.wtype, self.w_host0, self.rows, self.k, qx[t], dx[t])
            ys.append(y)
            Ss.append(S)
        return {"y": np.stack(ys), "S": np.stack(Ss)}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"])
        return ok, "%d tokens x %d rows within %g*S (worst %.3g*S)" % (self.T, self.rows, ROW_TOL,
                                                                      worst)

    def cpu_sample(self):
        return "quantize %d tokens + a %d-row DMMV per token over the first weight copy" % (
            self.T, self.rows)


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

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy(), "ids": self.ids.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        gu, gs, down, ds = self.host_bank
        logits, g = self.host_router
        ids, wts = oracle.moe_route(logits, self.top_k, g)
        y, S = oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, ids, wts, self.x_host)
        return {"y": y, "S": S, "ids": ids}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"], MOE_E2E_TOL)
        ok = ok and np.array_equal(gpu["ids"], ref["ids"])
        return ok, ("expert ids equal; %d rows within the unchained MoE bar %g*S (worst %.3g*S)"
                    % (self.dm, MOE_E2E_TOL, worst))

    def cpu_sample(self):
        return "route + one token through 8 routed + 1 shared expert (the first bank copy)"


class MoeTokWorkload(Workload):
    """Eight tokens, each with its own router logits, through the MoE block of
    128 + 1 Q4_0 experts in one call (zq_moe_ffn_tokens: route, gate/up,
    down with the weighted sums; each distinct expert's weights read once).
    The step's bytes are the distinct experts the step's routing touches
    (counted from the GPU's own expert lists) plus the activations and
    outputs."""
    dominant_name = "several-token MoE block (route + gate/up + down launches)"
    step_is_dominant = True
    steps = 1000
    warmup = 50

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.E, self.top_k, self.dm, self.dff = cfg["n_routed"], cfg["top_k"], cfg["d_model"], cfg["d_ff"]
        self.T = cfg["n_tok"]
        self.n_sel = self.top_k + 1
        self.expert_bytes = (2 * self.dff * (self.dm // 32) + self.dm * (self.dff // 32)) * 18

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for((self.E + 1) * self.expert_bytes)
        self.banks = []
        for c in range(self.ncopy):
            gu, gs, down, ds = inputs.moe_banks(inputs.seed_for(self.wl, c), self.E + 1, self.dm,
                                                self.dff)
            self.banks.append((torch.from_numpy(gu).to("cuda"), torch.from_numpy(down).to("cuda")))
            if c == 0:
                self.host_bank = (gu, gs, down, ds)
        self.gs, self.ds = gs, ds
        self.nlog = 64
        rng = np.random.default_rng(inputs.seed_for(self.wl, 100))
        self.logits_host = rng.standard_normal((self.nlog, self.T, self.E)).astype(np.float32)
        self.gates_host = rng.standard_normal((self.nlog, self.T)).astype(np.float32)
        self.logits = torch.from_numpy(self.logits_host).to("cuda")
        self.gates = torch.from_numpy(self.gates_host).to("cuda")
        self.x_host = inputs.gen_activation(self.T, self.dm, inputs.seed_for(self.wl) + 7)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.ids = torch.empty((self.T, self.n_sel), dtype=torch.int32, device="cuda")
        self.wts = torch.empty((self.T, self.n_sel), dtype=torch.float32, device="cuda")
        self.ws_bytes = zq.zq_moe_ffn_tokens_workspace_bytes(self.dm, self.dff, self.T, self.n_sel)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.y = torch.empty((self.T, self.dm), dtype=torch.float32, device="cuda")
        # the distinct experts of each routing, from the GPU's own lists
        distinct = []
        for j in range(self.nlog):
            self.step(j)
            torch.cuda.synchronize()
            distinct.append(len(np.unique(self.ids.cpu().numpy())))
        self.distinct = float(np.mean(distinct))
        self.step_bytes = (self.distinct * self.expert_bytes + 4 * self.T * self.E +
                           8 * self.T * self.dm)

    def step(self, i):
        gu, down = self.banks[i % self.ncopy]
        j = i % self.nlog
        self.zq.zq_moe_ffn_tokens(4, gu, self.gs, down, self.ds, self.E + 1, self.dm, self.dff,
                                  self.logits[j], self.E, self.top_k, self.gates[j], self.x, self.T,
                                  self.ids, self.wts, self.ws, self.ws_bytes, self.y)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", int(self.step_bytes)

    def extra(self, ms):
        return {"tokens_per_s": self.T / (ms * 1e-3), "us_per_token": ms * 1e3 / self.T,
                "distinct_experts_per_step": self.distinct,
                "expert_slots_per_step": self.T * self.n_sel}

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy(), "ids": self.ids.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        gu, gs, down, ds = self.host_bank
        ys, Ss, idss = [], [], []
        for t in range(self.T):
            ids, wts = oracle.moe_route(self.logits_host[0, t], self.top_k, self.gates_host[0, t])
            y, S = oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, ids, wts, self.x_host[t])
            ys.append(y)
            Ss.append(S)
            idss.append(ids)
        return {"y": np.stack(ys), "S": np.stack(Ss), "ids": np.stack(idss)}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"], MOE_E2E_TOL)
        ok = ok and np.array_equal(gpu["ids"], ref["ids"])
        return ok, ("expert ids equal; %d tokens x %d rows within the unchained MoE bar %g*S "
                    "(worst %.3g*S)" % (self.T, self.dm, MOE_E2E_TOL, worst))

    def cpu_sample(self):
        return "route + %d tokens through 8 routed + 1 shared expert each (first bank copy)" % self.T


class GemmWorkload(Workload):
    dominant_name = "gemm_kernel"
    bound = "mfma"
    steps = 100
    warmup = 10
    SAMPLE = 256   # output entries per oracle step

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
        rng = np.random.default_rng(55)
        self.mi = rng.integers(0, self.m, self.SAMPLE)
        self.ni = rng.integers(0, self.n, self.SAMPLE)
        self._oq = None

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

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy()[self.mi, self.ni].copy()}

    def oracle_step(self):
        import oracle
        if self._oq is None:  # every token's codes, once (outside the timed sample)
            self._oq = oracle.quantize_act(self.x_host)[:2]
        qx, dx = self._oq
        y, S = oracle.gemm_entries(4, self.w_host0, self.n, self.k, qx, dx, self.m, self.mi,
                                   self.ni)
        return {"y": y, "S": S}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"])
        return ok, "%d sampled entries within %g*S (worst %.3g*S)" % (self.SAMPLE, ROW_TOL, worst)

    def cpu_value(self, s_per_step):
        return self.SAMPLE * 2 * self.k / s_per_step / 1e12, "TOP/s"

    def cpu_sample(self):
        return ("%d sampled output entries of the %d x %d x %d GEMM (tokens quantized once "
                "beforehand)" % (self.SAMPLE, self.m, self.n, self.k))


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

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy(), "ids": self.ids.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        gu, gs, dn, ds = self.host_bank
        sgu, sdn = self.host_shared
        logits, g = self.host_router
        ids, wts = oracle.moe_route(logits, self.top_k, g)
        y, S = oracle.moe_ffn_mixed(self.gwt, gu, gs, self.dwt, dn, ds, self.swt, sgu, sdn,
                                    self.E, self.dm, self.dff, ids, wts, self.x_host)
        return {"y": y, "S": S, "ids": ids}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"], MOE_E2E_TOL)
        ok = ok and np.array_equal(gpu["ids"], ref["ids"])
        return ok, ("expert ids equal; %d rows within the unchained MoE bar %g*S (worst %.3g*S)"
                    % (self.dm, MOE_E2E_TOL, worst))

    def cpu_sample(self):
        return "route + one token through 8 K-quant experts + the Q8_0 shared expert"


class DecodeChainWorkload(Workload):
    """One token through 40 layers (RMS norm + Q8_0 router DMMV, routed MoE
    block of 128 + 1 Q4_0 experts added onto the state) and the LM head with
    its final norm and argmax: 122 launches, replayed as one HIP graph.  The
    eager time of the same chain is reported beside it."""
    dominant_name = "moe_gate_up_kernel (router folded in)"
    bound = "hbm"
    step_is_graph = True
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

    def gpu_result(self):
        """The replayed graph's token (as timed), then the same token run
        eagerly one layer at a time, keeping every layer's input state and
        routing for the layer-by-layer oracle check."""
        torch = self.torch
        c = self.chain
        c.x.copy_(self.x0)
        c.y_lm.fill_(float("nan"))
        c.idx.fill_(-1)
        c.replay()
        torch.cuda.synchronize()
        out = {"y": c.y_lm.cpu().numpy().copy(), "idx": int(c.idx.cpu().numpy()[0])}
        c.x.copy_(self.x0)
        torch.cuda.synchronize()
        states, ids, wts = [], [], []
        for layer in range(self.layers):
            states.append(c.x.cpu().numpy().copy())
            c.step_layer(layer)
            torch.cuda.synchronize()
            ids.append(c.ids.cpu().numpy().copy())
            wts.append(c.wts.cpu().numpy().copy())
        states.append(c.x.cpu().numpy().copy())
        c.y_lm.fill_(float("nan"))
        c.idx.fill_(-1)
        c.lm_head()
        torch.cuda.synchronize()
        out.update(y_eager=c.y_lm.cpu().numpy().copy(), idx_eager=int(c.idx.cpu().numpy()[0]),
                   states=states, ids=ids, wts=wts)
        self.gpu_states = out
        return out

    def oracle_step(self):
        """The oracle through every layer from the GPU's input state of that
        layer (so that one layer's rounding cannot compound into the next):
        norm, Q8_0 router, top-k + shared expert, the MoE block, the residual
        add; then the final norm and LM head from the GPU's final state.  A
        layer whose GPU routing differs from the oracle's also gets the block
        with the GPU's experts, for the near-tie check."""
        import oracle
        h = self.host
        g = self.gpu_states
        layers = []
        for l in range(self.layers):
            x = g["states"][l].astype(np.float32)
            xn = oracle.rms_norm(x, h["norms"][l], 1e-6).astype(np.float32)
            qx, dx, _ = oracle.quantize_act(xn)
            logits, S_r = oracle.dmmv(8, h["routers"][l], self.E, self.dm, qx, dx)
            ids, wts = oracle.moe_route(logits.astype(np.float32), self.top_k, h["gates"][l])
            gu, gs, down, ds = self.host_banks[l % self.nbanks]
            y, S = oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, ids, wts, xn)
            rec = {"logits": logits, "S_r": S_r, "ids": ids, "x_out": x.astype(np.float64) + y,
                   "S": S + np.abs(x.astype(np.float64))}
            if not np.array_equal(np.sort(ids), np.sort(g["ids"][l])):
                y2, _ = oracle.moe_ffn(4, gu, gs, down, ds, self.dm, self.dff, g["ids"][l],
                                       g["wts"][l].astype(np.float64), xn)
                rec["x_out_gpu_ids"] = x.astype(np.float64) + y2
            layers.append(rec)
        x = g["states"][-1].astype(np.float32)
        xn = oracle.rms_norm(x, h["norms"][-1], 1e-6).astype(np.float32)
        qx, dx, _ = oracle.quantize_act(xn)
        yl, S = oracle.dmmv(4, h["lm"], self.vocab, self.dm, qx, dx)
        return {"layers": layers, "y": yl, "S": S}

    def near_tie(self, rec, gpu_ids):
        """The GPU's routed experts differ from the oracle's only by experts
        whose oracle logits lie within the row bar of the selection boundary."""
        k = self.top_k
        lg, Sr = rec["logits"], rec["S_r"]
        order = np.argsort(-lg, kind="stable")
        edge = lg[order[k - 1]] if k > 0 else np.inf
        routed_g = set(int(e) for e in gpu_ids[:k])
        routed_r = set(int(e) for e in rec["ids"][:k])
        for e in routed_g ^ routed_r:
            if e >= self.E or abs(lg[e] - edge) > ROW_TOL * (Sr[e] + Sr[order[k - 1]]):
                return False
        return True

    def parity(self, gpu, ref):
        if not (np.array_equal(gpu["y"].view(np.uint32), gpu["y_eager"].view(np.uint32)) and
                gpu["idx"] == gpu["idx_eager"]):
            return False, "the replayed graph's logits differ from the eager run's"
        worst, ties = 0.0, 0
        for l, rec in enumerate(ref["layers"]):
            x_out = rec["x_out"]
            if "x_out_gpu_ids" in rec:
                if not self.near_tie(rec, gpu["ids"][l]):
                    return False, "layer %d: the GPU's experts differ from the oracle's" % l
                ties += 1
                x_out = rec["x_out_gpu_ids"]
            err = np.abs(gpu["states"][l + 1].astype(np.float64) - x_out) / rec["S"]
            worst = max(worst, float(err.max()))
        err_lm = float((np.abs(gpu["y"].astype(np.float64) - ref["y"]) / ref["S"]).max())
        ok = (worst <= MOE_E2E_TOL and err_lm <= MOE_E2E_TOL and
              argmax_ok(gpu["idx"], gpu["y"], ref["y"], ref["S"], MOE_E2E_TOL))
        return ok, ("graph replay = eager run bit for bit; each of %d layers from the GPU's own "
                    "input state: experts equal to the oracle's (%d near ties), state after the "
                    "block within %g*S (worst %.3g*S); LM head from the GPU's final state within "
                    "%g*S (worst %.3g*S), token %d" % (self.layers, ties, MOE_E2E_TOL, worst,
                                                       MOE_E2E_TOL, err_lm, gpu["idx"]))

    def cpu_value(self, s_per_step):
        return 1.0 / s_per_step, "tok/s"

    def cpu_sample(self):
        return "one token through the %d-layer chain and the LM head" % self.layers


class FloatDmmvWorkload(Workload):
    """The F16 DMMV from the fp32 activation (one launch): the headline shape
    and the LM head."""
    step_is_dominant = True
    dtype = "f16 x f32 -> f32"

    def __init__(self, wl):
        from block_quant_matrix_amd import inputs
        cfg = inputs.WORKLOADS[wl]
        self.wl = wl
        self.name = cfg["name"]
        self.wtype, self.rows, self.k = cfg["wtype"], cfg["rows"], cfg["k"]
        self.wbytes = self.rows * self.k * inputs.FLOAT_BYTES[self.wtype]
        self.dominant_name = "dmmv_float_kernel (F16)"
        # weights + fp32 activation in + fp32 rows out
        self.step_bytes = self.wbytes + 4 * self.k + 4 * self.rows
        self.steps, self.warmup = (2000, 100) if self.wbytes < (256 << 20) else (60, 5)

    def setup(self, torch, zq, inputs):
        self.torch, self.zq = torch, zq
        self.ncopy = copies_for(self.wbytes)
        self.w = []
        for c in range(self.ncopy):
            h = inputs.gen_weights_float(self.wtype, self.rows, self.k, inputs.seed_for(self.wl, c))
            self.w.append(torch.from_numpy(h).to("cuda"))
            if c == 0:
                self.w_host0 = h
            del h
        self.x_host = inputs.gen_activation(1, self.k, inputs.seed_for(self.wl) + 1)
        self.x = torch.from_numpy(self.x_host).to("cuda")
        self.y = torch.empty(self.rows, dtype=torch.float32, device="cuda")

    def step(self, i):
        self.zq.zq_dmmv_float(self.wtype, self.w[i % self.ncopy], self.rows, self.k, self.x,
                              self.y)

    def value(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, "GB/s"

    def achieved(self, ms):
        return self.step_bytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", self.step_bytes

    def extra(self, ms):
        return {"rows_per_s": self.rows / (ms * 1e-3)}

    def gpu_result(self):
        self.y.fill_(float("nan"))
        self.step(0)
        self.torch.cuda.synchronize()
        return {"y": self.y.cpu().numpy().copy()}

    def oracle_step(self):
        import oracle
        y, S = oracle.float_dmmv(self.wtype, self.w_host0, self.rows, self.k, self.x_host)
        return {"y": y, "S": S}

    def parity(self, gpu, ref):
        ok, worst = rows_within(gpu["y"], ref["y"], ref["S"])
        return ok, "%d rows within %g*S (worst %.3g*S)" % (self.rows, ROW_TOL, worst)

    def cpu_sample(self):
        return "a %d-row F16 DMMV over this workload's first weight copy" % self.rows


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
    if wl in (14, 15):
        return FloatDmmvWorkload(wl)
    if wl == 16:
        return MoeTokWorkload(wl)
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


def host_launch_ms(fn, torch, n=50):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    el = (time.perf_counter() - t0) * 1e3 / n
    torch.cuda.synchronize()
    return el


def timed(torch, fn, K, h_ms, graph=True):
    """ms per call of K back-to-back calls of fn(i) between two events on the
    launch stream.

    With graph (the default) the K calls are captured once as a HIP graph and
    the timed region is one replay of it: the host then submits a node in well
    under a microsecond, so a kernel shorter than a Python-level call is not
    paced by the host.  The replay waits behind a GPU blocker longer than its
    own submission.  Without graph the K calls are made eagerly behind a
    blocker sized from h_ms (for steps that are themselves graph replays)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if not graph:
        gpu_blocker(torch, 1.5 * h_ms * K + 5)
        e0.record()
        for i in range(K):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        for i in range(K):
            fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()  # untimed: the replay's own host cost sizes the blocker
    h_replay = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    gpu_blocker(torch, 1.5 * h_replay + 5)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / K


def read_ceiling(torch, zq, nbytes=1 << 30, K=20):
    """The live streaming-read rate of the chip (GB/s): K back-to-back reads
    of 1 GiB (4x the MALL) by the library's read probe."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        zq.zq_read_probe(buf, nbytes, sink)
    h_ms = host_launch_ms(lambda i: zq.zq_read_probe(buf, nbytes, sink), torch, n=5)
    ms = timed(torch, lambda i: zq.zq_read_probe(buf, nbytes, sink), K, h_ms)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def read_floor(torch, zq, nbytes, ncopy, K):
    """The same-size read floor (ms per launch): K back-to-back launches of the
    library's read probe over nbytes, rotating over ncopy distinct buffers as
    the workload's weights rotate, so that each launch reads from HBM; the
    time any kernel needs to read that many bytes, its launch included."""
    n16 = nbytes // 16 * 16
    buf = torch.empty(ncopy * n16, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    fn = lambda i: zq.zq_read_probe(base + (i % ncopy) * n16, n16, sink)
    for i in range(3):
        fn(i)
    h_ms = host_launch_ms(fn, torch, n=5)
    ms = timed(torch, fn, K, h_ms)
    del buf
    return n16, ms


def gpu_clocks():
    """Current shader and memory clocks from rocm-smi (best effort)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(k for k in d if k.startswith("card"))[0]]
        pick = lambda key: next((v for k, v in card.items() if k.lower().startswith(key)), None)
        return {"sclk": pick("sclk"), "mclk": pick("mclk")}
    except Exception:  # noqa: BLE001 - a missing or changed tool only drops the field
        return None


# ------------------------------------------------------------- oracle leg --

def host_threads():
    """Threads the oracle may use: the process's CPUs, at most 16 (one GPU's
    share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_leg(w, seconds):
    """The GPU's first step against the oracle (parity), then the oracle's
    own rate on one thread and on all host threads (each the median of 3
    runs).  The oracle's C routines release the interpreter while they run,
    so threads that each run whole oracle steps run in parallel."""
    gpu = w.gpu_result()
    t0 = time.perf_counter()
    ref = w.oracle_step()
    t_one = time.perf_counter() - t0
    ok, detail = w.parity(gpu, ref)
    n = max(1, int(round(seconds / 6.0 / t_one)))

    def run(m):
        for _ in range(m):
            w.oracle_step()

    single = []
    for _ in range(3):
        t0 = time.perf_counter()
        run(n)
        single.append((time.perf_counter() - t0) / n)
    threads = host_threads()
    multi = []
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(run, [n] * threads))
            multi.append((time.perf_counter() - t0) / (n * threads))
    s1, sm = statistics.median(single), statistics.median(multi)
    v1, unit = w.cpu_value(s1)
    vm, _ = w.cpu_value(sm)
    cpu = {"value": round(vm, 4), "unit": unit, "cores": threads, "kind": "oracle",
           "sample": "%s; each run %d step(s) per thread, median of 3 runs, %d threads each "
                     "running whole steps" % (w.cpu_sample(), n, threads),
           "single_thread": {"value": round(v1, 4), "unit": unit, "s_per_step": round(s1, 6)},
           "all_cores_s_per_step": round(sm, 6), "runs": 3, "statistic": "median",
           "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    return cpu, {"ok": bool(ok), "detail": detail}


# ------------------------------------------------------------------ main --

def measure(w, torch, K, W):
    """Warm up, then the timed region and the dominant kernel's pass."""
    for i in range(W):
        w.step(i)
    torch.cuda.synchronize()
    h_ms = host_launch_ms(w.step, torch)
    ms_per_step = timed(torch, w.step, K, h_ms, graph=not w.step_is_graph)
    if w.step_is_dominant:
        ms_kernel = ms_per_step
    else:
        # the dominant kernel alone: K back-to-back launches between two
        # events (an event pair around each launch adds several microseconds
        # of marker processing to a microsecond-scale kernel)
        w.prepare_dominant()
        ms_kernel = timed(torch, w.dominant, K, h_ms)
    return ms_per_step, ms_kernel


def oracle_leg_sampled(s):
    """The oracle leg of a secondary line: the GPU's first step against the
    oracle on sampled rows, and its argmax against the GPU's own logits."""
    gpu = s.gpu_result()
    rng = np.random.default_rng(3)
    sel = np.unique(np.concatenate([[0, s.rows - 1, gpu["idx"]],
                                    rng.integers(0, s.rows, 2048)])).astype(np.int64)
    return s.parity(gpu, s.oracle_step(rows_eval=sel), rows_eval=sel)


def lmhead_secondary(torch, zq, inputs, with_oracle):
    """The LM-head step (Q4_0 248 320 x 2048 + argmax) measured beside the
    headline: step rate, the fused DMMV launch alone, and (with the oracle
    leg) a parity check of sampled rows and of the argmax."""
    s = DmmvWorkload(3)
    s.setup(torch, zq, inputs)
    ok, detail = oracle_leg_sampled(s) if with_oracle else (None, None)
    ms_step, ms_kernel = measure(s, torch, s.steps, s.warmup)
    gbs = s.dmmv_bytes / (ms_kernel * 1e-3) / 1e9
    out = {"workload": s.name, "steps": s.steps, "ms_per_step": round(ms_step, 6),
           "step_GBs": round(s.step_bytes / (ms_step * 1e-3) / 1e9, 1),
           "rows_per_s": round(s.rows / (ms_step * 1e-3), 1),
           "dmmv_kernel": {"kernel": s.dominant_name, "ms_per_launch": round(ms_kernel, 6),
                           "per_launch": s.dmmv_bytes, "achieved_GBs": round(gbs, 1),
                           "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": counted_traffic(s.dominant_name, s.name)},
           "parity_checked": None if ok is None else bool(ok), "parity": detail}
    del s
    return out


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

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = oracle_leg(w, args.cpu_seconds)

    clocks_before = None if args.no_clocks else gpu_clocks()
    ms_per_step, ms_kernel = measure(w, torch, K, W)
    clocks_after = None if args.no_clocks else gpu_clocks()

    # what a launch of any kernel costs before it reads a byte: K back-to-back
    # launches of an empty kernel (torch's spin kernel with a zero count) on
    # the same stream; a diagnostic beside the roofline, not part of it
    ms_floor = timed(torch, lambda i: torch.cuda._sleep(0), K, 0.01)
    ceiling = read_ceiling(torch, zq)

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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "weight_copies": w.ncopy, "parallelism": "none"},
        "pct_of_peak": round(w.pct_of_peak(value, unit), 2),
        "parity_checked": None if parity is None else parity["ok"],
    }
    if parity is not None:
        out["parity"] = parity["detail"]
    out.update({k: round(v, 4 if abs(v) < 10 else 1) for k, v in w.extra(ms_per_step).items()})
    out["roofline"] = {"bound": w.bound, "kernel": w.dominant_name, "achieved": round(ach, 3),
                       "peak": peak, "unit": runit, "frac": round(ach / peak, 4),
                       "traffic": counted_traffic(w.dominant_name,
                                                  getattr(w, "traffic_workload", w.name)),
                       "per_launch": per_launch, "ms_per_launch": round(ms_kernel, 6),
                       "timed_in": "the timed region" if w.step_is_dominant else
                                   "a pass of K back-to-back launches of this kernel alone"}
    out["read_ceiling"] = {"GBs": round(ceiling, 1),
                           "note": "live streaming read of 1 GiB by zq_read_probe"}
    if runit == "GB/s":
        out["read_ceiling"]["frac_of_ceiling"] = round(ach / ceiling, 4)
    if runit == "GB/s" and per_launch <= (64 << 20):
        # at sizes where a launch's fixed cost weighs, the time a read-only
        # kernel needs for the same bytes, measured the same way
        nf, ms_rf = read_floor(torch, zq, per_launch, w.ncopy, min(K, 2000))
        out["read_floor"] = {"bytes": nf, "us_per_launch": round(ms_rf * 1e3, 3),
                             "GBs": round(nf / (ms_rf * 1e-3) / 1e9, 1),
                             "kernel_us_per_launch": round(ms_kernel * 1e3, 3),
                             "frac_of_floor_rate": round(ms_rf / ms_kernel, 4),
                             "note": "zq_read_probe over the dominant kernel's algorithmic "
                                     "bytes, rotating over the workload's weight copies"}
    out["empty_launch_us"] = round(ms_floor * 1e3, 3)
    out["clocks"] = {"before": clocks_before, "after": clocks_after}
    if args.workload == 2:
        out["target_70pct_met"] = ach / peak >= 0.70
    if args.workload == 2 and not args.no_secondary:
        out["secondary"] = [lmhead_secondary(torch, zq, inputs, not args.no_cpu_baseline)]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
