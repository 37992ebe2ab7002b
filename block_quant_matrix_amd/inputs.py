"""Seeded synthetic inputs for the block-quantized DMMV path.

This module only draws random numbers and lays them out as the raw input bytes
the path consumes (GGML-style blocks: little-endian fp16 scale first, then the
quants).  It does none of the method's arithmetic: no quantization, no dot
products, no scaling.  Both the CPU oracle's tests and the GPU path take their
inputs from here, so both sides see identical bytes.

Value distributions (the workloads' recipe):
  * Q8_0 weights: int8 values uniform in [-127, 127]; scales |N(0,1)|*0.01
    rounded once to fp16.
  * Q4_0 weights: nibbles uniform in 0..15 (so each packed byte is uniform in
    0..255); scales |N(0,1)|*0.02 rounded once to fp16.
  * K-quant weights (256-element super-blocks): every packed byte of codes,
    fifth bits, 6-bit sub-block scales/mins (Q4_K, Q5_K) uniform in 0..255;
    Q6_K sub-block scales int8 uniform in [-128, 127]; the super-block d and
    dmin |N(0,1)|*0.001 rounded once to fp16.
  * F16 / F32 weights: N(0,1)*0.02 rounded once to the weight type.
  * activations: fp32 N(0,1).
  * MoE router logits: fp32 N(0,1); shared-expert gate scalar: fp32 N(0,1).
Seeds: workload i (1-based, in the order below) uses 1000*i + s.
"""
from __future__ import annotations

import numpy as np

Q4_0 = 4
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
F16 = 16
F32 = 32
FLOAT_BYTES = {F16: 2, F32: 4}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}
SCALE_C = {Q8_0: 0.01, Q4_0: 0.02, Q4_K: 0.001, Q5_K: 0.001, Q6_K: 0.001}
# K-quant super-blocks: bytes per 256 elements
K_BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}


def seed_for(workload: int, s: int = 0) -> int:
    return 1000 * workload + s


def fp16_scales(rng: np.random.Generator, n: int, c: float) -> np.ndarray:
    """|N(0,1)| * c in fp64, rounded once (RNE) to fp16."""
    return (np.abs(rng.standard_normal(n, dtype=np.float64)) * c).astype(np.float16)


def layout_blocks(scales_f16: np.ndarray, quant_bytes: np.ndarray) -> np.ndarray:
    """Interleave per-block fp16 scales and quant bytes into one byte stream.

    scales_f16: [n] float16; quant_bytes: [n][q] uint8 -> [n*(2+q)] uint8.
    """
    n = scales_f16.size
    q = quant_bytes.reshape(n, -1)
    out = np.empty((n, 2 + q.shape[1]), np.uint8)
    out[:, :2] = np.ascontiguousarray(scales_f16.astype("<f2")).view(np.uint8).reshape(n, 2)
    out[:, 2:] = q
    return out.reshape(-1)


def gen_weights(wtype: int, rows: int, k: int, seed: int, scale_c: float | None = None) -> np.ndarray:
    """Random weight matrix [rows][k/32 blocks] as raw bytes (uint8)."""
    assert k % 32 == 0
    n = rows * (k // 32)
    rng = np.random.default_rng(seed)
    c = SCALE_C[wtype] if scale_c is None else scale_c
    d = fp16_scales(rng, n, c)
    if wtype == Q8_0:
        q = rng.integers(-127, 128, size=(n, 32), dtype=np.int8).view(np.uint8)
    elif wtype == Q4_0:
        q = rng.integers(0, 256, size=(n, 16), dtype=np.uint8)
    else:
        raise ValueError("unknown weight type %r" % wtype)
    return layout_blocks(d, q)


def gen_weights_k(wtype: int, rows: int, k: int, seed: int) -> np.ndarray:
    """Random K-quant weight matrix [rows][k/256 super-blocks] as raw bytes.

    Q4_K / Q5_K: fp16 d, fp16 dmin, then the rest of the super-block as
    uniform random bytes (12 bytes of packed 6-bit scales and mins, the fifth
    bits of Q5_K, the nibbles).  Q6_K: 208 uniform random bytes (low nibbles,
    2-bit highs, int8 sub-block scales) then fp16 d."""
    assert k % 256 == 0
    n = rows * (k // 256)
    bb = K_BLOCK_BYTES[wtype]
    rng = np.random.default_rng(seed)
    c = SCALE_C[wtype]
    out = np.empty((n, bb), np.uint8)
    if wtype in (Q4_K, Q5_K):
        d = fp16_scales(rng, n, c)
        dmin = fp16_scales(rng, n, c)
        out[:, 0:2] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(n, 2)
        out[:, 2:4] = np.ascontiguousarray(dmin.astype("<f2")).view(np.uint8).reshape(n, 2)
        out[:, 4:] = rng.integers(0, 256, size=(n, bb - 4), dtype=np.uint8)
    elif wtype == Q6_K:
        d = fp16_scales(rng, n, c)
        out[:, :208] = rng.integers(0, 256, size=(n, 208), dtype=np.uint8)
        out[:, 208:] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(n, 2)
    else:
        raise ValueError("not a K-quant type %r" % wtype)
    return out.reshape(-1)


def gen_weights_float(wtype: int, rows: int, k: int, seed: int, c: float = 0.02) -> np.ndarray:
    """Random float weight matrix [rows][k] (N(0,1)*c in fp64, rounded once to
    binary16 or binary32) as raw little-endian bytes (uint8)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, k), dtype=np.float64) * c
    dt = "<f2" if wtype == F16 else "<f4"
    return np.ascontiguousarray(v.astype(dt)).view(np.uint8).reshape(-1)


def gen_activation(n_tok: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_tok, k), dtype=np.float32)
    return x[0] if n_tok == 1 else x


def gen_router(n_routed: int, seed: int):
    """Router logits N(0,1)[n_routed] and the shared-expert gate scalar g ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(n_routed, dtype=np.float32)
    g = np.float32(rng.standard_normal(dtype=np.float32))
    return logits, g


# The workloads (shapes from the pages; distributions as above).
WORKLOADS = {
    1: dict(name="q8_0_dmmv_64x2048", wtype=Q8_0, rows=64, k=2048),
    2: dict(name="q4_0_dmmv_4096x4096", wtype=Q4_0, rows=4096, k=4096),
    3: dict(name="q4_0_lmhead_248320x2048_argmax", wtype=Q4_0, rows=248320, k=2048),
    4: dict(name="q4_0_moe_128e_top8_shared_2048x512", wtype=Q4_0, n_routed=128, top_k=8,
            d_model=2048, d_ff=512),
    5: dict(name="q4_0_prefill_gemm_m512_n5120_k5120", wtype=Q4_0, m=512, n=5120, k=5120),
    # K-quant DMMV: the headline shape over the format the pages' experts use
    6: dict(name="q4_k_dmmv_4096x4096", wtype=Q4_K, rows=4096, k=4096),
    # the LM head of the pages' model is Q6_K at the vocabulary shape
    7: dict(name="q6_k_lmhead_dmmv_248320x2048", wtype=Q6_K, rows=248320, k=2048),
    8: dict(name="q5_k_dmmv_4096x4096", wtype=Q5_K, rows=4096, k=4096),
    # small-M decode: eight tokens through one pass over the weights
    9: dict(name="q4_0_dmmv_8tok_4096x4096", wtype=Q4_0, rows=4096, k=4096, n_tok=8),
    # one token through 40 layers of the path (norm + router + routed MoE)
    # and the LM head, replayed as one graph; 4 distinct expert banks
    10: dict(name="decode_chain_40l_moe128e_top8_lmhead248320", layers=40, moe_banks=4,
             n_routed=128, top_k=8, d_model=2048, d_ff=512, vocab=248320),
    # the MoE block in the pages' model formats: routed gate/up Q4_K, down
    # Q5_K, shared expert Q8_0
    11: dict(name="moe_128e_top8_q4k_q5k_shared_q8_0_2048x512", n_routed=128, top_k=8,
             d_model=2048, d_ff=512, gu_wtype=Q4_K, down_wtype=Q5_K, sh_wtype=Q8_0),
    # small-M at the vocabulary shape: eight tokens through the LM head
    12: dict(name="q4_0_lmhead_8tok_248320x2048", wtype=Q4_0, rows=248320, k=2048, n_tok=8),
    13: dict(name="q8_0_lmhead_248320x2048_argmax", wtype=Q8_0, rows=248320, k=2048),
    # the F16 member of the DMMV family: the headline shape and the LM head
    14: dict(name="f16_dmmv_4096x4096", wtype=F16, rows=4096, k=4096),
    15: dict(name="f16_lmhead_dmmv_248320x2048", wtype=F16, rows=248320, k=2048),
    # small-M MoE: eight tokens, each with its own routing, in one call
    16: dict(name="q4_0_moe_8tok_128e_top8_shared_2048x512", wtype=Q4_0, n_routed=128, top_k=8,
             d_model=2048, d_ff=512, n_tok=8),
}


def moe_banks_k(seed: int, n_experts: int, d_model: int, d_ff: int, gu_wtype: int,
                down_wtype: int):
    """As moe_banks for K-quant experts (gate||up and down may differ in
    type, as in the pages' model: Q4_K gate/up, Q5_K down)."""
    gu = gen_weights_k(gu_wtype, n_experts * 2 * d_ff, d_model, seed)
    down = gen_weights_k(down_wtype, n_experts * d_model, d_ff, seed + 500)
    gu_stride = 2 * d_ff * (d_model // 256) * K_BLOCK_BYTES[gu_wtype]
    down_stride = d_model * (d_ff // 256) * K_BLOCK_BYTES[down_wtype]
    return gu, gu_stride, down, down_stride


def moe_banks(seed: int, n_experts: int, d_model: int, d_ff: int, wtype: int = Q4_0):
    """Gate||up bank [E][2*d_ff rows][d_model] (rows 0..d_ff-1 gate, d_ff..2*d_ff-1 up)
    and down bank [E][d_model rows][d_ff], as contiguous byte streams."""
    gu = gen_weights(wtype, n_experts * 2 * d_ff, d_model, seed)
    down = gen_weights(wtype, n_experts * d_model, d_ff, seed + 500)
    gu_stride = 2 * d_ff * (d_model // 32) * BLOCK_BYTES[wtype]
    down_stride = d_model * (d_ff // 32) * BLOCK_BYTES[wtype]
    return gu, gu_stride, down, down_stride
