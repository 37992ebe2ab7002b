"""A per-token decode chain over the zq kernels, for eager runs and HIP graph
replay.

One token passes through `layers` copies of the hot path and the LM head:
  per layer, zq_moe_ffn_norm_route: RMS-normalize the fp32 state and take
    the Q8_0 router DMMV of it (one launch; xn and the logits published),
    then the routed MoE block on xn (router top-k + softmax folded into the
    gate/up pass, SwiGLU + requantize, down with the weighted sum) added
    onto the state (two launches, ZQ_ACCUMULATE);
  then the LM head: final RMS norm, Q4_0 DMMV + argmax (two launches).
The layer order and the residual add follow the decode forward order of
"Bringing ZINC to NVIDIA: a CUDA backend, because WSL2 only speaks CUDA",
section "The roadmap: from 70 to a coherent token" (router DMMV,
softmax_topk, expert gate/up, swiglu, expert down with the weighted
accumulate, residual accumulate, rms_norm_mul, LM head, argmax), without
the attention and SSM stages that lie outside this path.  Replaying the whole
per-token chain as one graph is "RTX 5090: Batched Prefill & CUDA Graphs in
ZINC", section "CUDA graphs - the structural answer to launch latency";
here torch.cuda.CUDAGraph records the same launches through HIP stream
capture.

Every buffer is allocated in the constructor; step() only enqueues zq
kernels on the current stream (no allocation, copy, memset or sync), which
is what makes it capturable.  Host-side orchestration only: every step of
the arithmetic runs in the zq kernels.
"""
from __future__ import annotations

from . import zq as _zq


class DecodeChain:
    def __init__(self, torch, router_w, moe_banks, lm_w, norm_w, final_norm_w, *, d_model,
                 n_routed, top_k, d_ff, vocab, shared_gate, eps=1e-6):
        """router_w: per-layer Q8_0 [n_routed][d_model] device byte tensors;
        moe_banks: per-layer (gu_bank, gu_stride, down_bank, down_stride, n_experts);
        lm_w: Q4_0 [vocab][d_model] device bytes; norm_w: per-layer fp32
        [d_model] RMS-norm weights, final_norm_w the one before the LM head;
        shared_gate: per-layer fp32 device scalars (the shared expert's gate
        g) or None."""
        self.torch = torch
        self.layers = len(router_w)
        assert len(moe_banks) == self.layers and len(norm_w) == self.layers
        self.router_w, self.moe_banks, self.lm_w = router_w, moe_banks, lm_w
        self.norm_w, self.final_norm_w, self.eps = norm_w, final_norm_w, eps
        self.d_model, self.n_routed, self.top_k, self.d_ff = d_model, n_routed, top_k, d_ff
        self.vocab = vocab
        self.shared_gate = shared_gate
        dev = "cuda"
        n_sel = top_k + (1 if shared_gate is not None else 0)
        self.n_sel = n_sel
        self.x = torch.zeros(d_model, dtype=torch.float32, device=dev)  # the state
        self.xn = torch.zeros(d_model, dtype=torch.float32, device=dev)  # normalized state
        self.logits = torch.empty(n_routed, dtype=torch.float32, device=dev)
        self.ids = torch.empty(n_sel, dtype=torch.int32, device=dev)
        self.wts = torch.empty(n_sel, dtype=torch.float32, device=dev)
        self.ws_bytes = _zq.zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.y_lm = torch.empty(vocab, dtype=torch.float32, device=dev)
        self.idx = torch.empty(1, dtype=torch.int32, device=dev)
        self.lm_ws_bytes = _zq.zq_dmmv_f32_argmax_workspace_bytes()
        self.lm_ws = torch.empty(self.lm_ws_bytes, dtype=torch.uint8, device=dev)
        self.graph = None

    def step_layer(self, layer, stream=None):
        """Enqueue one layer: norm, router, the routed MoE block added onto
        the state (xn and the logits published)."""
        d, f = self.d_model, self.d_ff
        gu, gs, dn, ds, ne = self.moe_banks[layer]
        g = None if self.shared_gate is None else self.shared_gate[layer]
        _zq.zq_moe_ffn_norm_route(_zq.ZQ_Q4_0, gu, gs, dn, ds, ne, d, f, self.router_w[layer],
                                  self.norm_w[layer], self.eps, self.x, self.n_routed, self.top_k,
                                  g, self.xn, self.logits, self.ids, self.wts, self.ws,
                                  self.ws_bytes, self.x, _zq.ZQ_ACCUMULATE, stream=stream)

    def lm_head(self, stream=None):
        """Enqueue the final norm, the LM-head DMMV and the argmax."""
        _zq.zq_rms_norm_dmmv_f32_argmax(_zq.ZQ_Q4_0, self.lm_w, self.vocab, self.d_model, self.x,
                                        self.final_norm_w, self.eps, self.y_lm, self.idx,
                                        self.lm_ws, self.lm_ws_bytes, stream=stream)

    def step(self, stream=None):
        """Enqueue one token: every layer, then the LM head and argmax."""
        for layer in range(self.layers):
            self.step_layer(layer, stream)
        self.lm_head(stream)

    def launches_per_step(self) -> int:
        return 3 * self.layers + 2

    def capture(self):
        """Record step() into a graph (after one eager warm-up call made by
        the caller); replay() then submits the whole token at once."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.step()
        torch.cuda.current_stream().wait_stream(s)
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
