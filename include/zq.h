/*
 * zq.h -- C ABI of libzq, block-quantized decode-path kernels for AMD MI355X
 * (gfx950).
 *
 * The path: GGML-style Q8_0 / Q4_0 weight blocks, an activation quantized to
 * int8 blocks of 32 with one fp32 scale each, and per-block int8 x int8 ->
 * int32 dot products scaled by d_w * d_x and summed into fp32 rows.
 *
 *   Q8_0 block (34 bytes): fp16 d (little-endian) then int8 q[32]; value q*d.
 *   Q4_0 block (18 bytes): fp16 d then uint8 qs[16]; element j (j < 16) is the
 *       low nibble of qs[j], element j+16 the high nibble; value (nib-8)*d.
 *   Both are the GGML layouts, which the pages state are identical bit for bit
 *   across ZINC's backends ("Bringing ZINC to NVIDIA: a CUDA backend ...",
 *   section "The reassuring result: ZINC's matmuls are __dp4a, not tensor
 *   cores"; "CUDA backend for ZINC", section 4 "Kernel port strategy").
 *   A weight matrix of `rows` x `k` is rows*(k/32) blocks, row-major, no
 *   padding; its row b-th block starts at byte (r*(k/32)+b)*block_bytes.
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or retains memory.  `stream` is a hipStream_t passed as
 *     void* (NULL = the default stream).  Calls are asynchronous on `stream`;
 *     the caller keeps every buffer alive until that work completes.
 *   - Arguments are checked before anything is launched.  On any error the
 *     call returns a negative zq_status and writes nothing.  0 = launched.
 *   - Alignment: weights 4-byte aligned; qx 16-byte aligned; x 16-byte aligned
 *     with a row stride that is a multiple of 4 elements; every other array
 *     4-byte aligned.  A Q4_0/Q8_0 kernel may read the two bytes that follow
 *     the last block of a weight buffer when they share that block's aligned
 *     4-byte word (never beyond it).
 *   - k must be a positive multiple of 32; sizes are element counts.
 *   - Only gfx950 devices are accepted (ZQ_EDEVICE otherwise).
 *   - The library keeps no mutable global state apart from a per-device
 *     capability cache filled once; calls are thread-safe.
 */
#ifndef ZQ_H
#define ZQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum zq_status {
    ZQ_OK = 0,
    ZQ_EINVAL = -1,  /* bad size, k % 32 != 0, unknown flag/type/mode, ranges    */
    ZQ_ENULL = -2,   /* a required pointer is NULL                              */
    ZQ_EALIGN = -3,  /* a pointer or stride violates the alignment rules above  */
    ZQ_ERANGE = -4,  /* an expert id outside [0, n_experts), found on the GPU   */
    ZQ_EDEVICE = -5, /* current device is not gfx950 / no device                */
    ZQ_ELAUNCH = -6  /* the HIP runtime refused the launch                      */
};

enum zq_flags { ZQ_ACCUMULATE = 1 /* y += W.x instead of y = W.x */ };
enum zq_wtype { ZQ_Q4_0 = 4, ZQ_Q8_0 = 8, ZQ_Q4_K = 12, ZQ_Q5_K = 13, ZQ_Q6_K = 14, ZQ_F16 = 16,
                ZQ_F32 = 32 };
enum zq_moe_mode { ZQ_MOE_GATHER = 0, ZQ_MOE_WEIGHTED_SUM = 1 };

int zq_version(void);
const char *zq_strerror(int status);
/* ZQ_OK when `device` is a gfx950 GPU, else ZQ_EDEVICE. */
int zq_device_check(int device);

/* Activation block quantization (the "quantize" shader family named in
 * "Bringing ZINC to NVIDIA", section "Porting the kernels"; formula: the
 * reading documented with the library).  For each token t and block b:
 *   amax = max|x|, d = amax/127 (IEEE fp32 division), id = d ? 1/d : 0,
 *   q = round_half_away_from_zero(x*id) clamped to [-127,127], s = sum q.
 * x:  [n_tok][x_stride] fp32 (first k used);  qx: [n_tok][k] int8;
 * dx: [n_tok][k/32] fp32;  sx: [n_tok][k/32] int32, may be NULL.
 * x must be finite (not checked). */
int zq_quantize_act(const float *x, int64_t n_tok, int64_t k, int64_t x_stride,
                    int8_t *qx, float *dx, int32_t *sx, void *stream);

/* Dequantizing matrix-vector product (habr "Как мы запустили 35B LLM ...",
 * section "Что такое DMMV": read the quantized weights, dequantize in
 * registers, multiply by the input vector, write the row):
 *   y[r] (+)= sum_b fp32(d_w[r][b]) * dx[b] * isum[r][b],
 *   isum[r][b] = sum_i w[r][b][i] * qx[32b+i]   (exact int32).
 * w: rows*(k/32) blocks; qx [k]; dx [k/32]; y [rows] fp32.
 * flags: 0 or ZQ_ACCUMULATE. */
int zq_dmmv_q8_0(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 float *y, uint32_t flags, void *stream);
/* As zq_dmmv_q8_0 for Q4_0 weights.  sx [k/32] (block sums of qx) may be NULL,
 * in which case the kernel sums qx itself. */
int zq_dmmv_q4_0(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream);

/* The same DMMV over GGML's K-quant super-blocks of 256 elements, bit for
 * bit ("Bringing ZINC to NVIDIA", section "The reassuring result"; "CUDA
 * backend for ZINC", section 5, dmmv_q4k / dmmv_q5k / dmmv_q6k; the pages'
 * model keeps its experts in Q4_K / Q5_K and its LM head in Q6_K):
 *   Q4_K, 144 bytes: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block scales
 *     and mins, 128 bytes of nibbles; element d*sc*q - dmin*m, q in 0..15;
 *   Q5_K, 176 bytes: as Q4_K with 32 bytes of fifth bits after the scales;
 *     q in 0..31;
 *   Q6_K, 210 bytes: 128 bytes of low nibbles, 64 bytes of 2-bit highs, 16
 *     int8 scales of 16-element sub-blocks, fp16 d; element d*sc*(q - 32).
 * With the int8 activation blocks of 32 (zq_quantize_act), which line up
 * with the sub-blocks:
 *   Q4_K / Q5_K: y[r] (+)= sum_b dx[b]*(d*sc_b*isum[r][b] - dmin*m_b*sx[b]),
 *     isum = sum q*qx;
 *   Q6_K: y[r] (+)= sum_b dx[b]*d*isum[r][b], isum = sum sc*(q-32)*qx over
 *     the block's two 16-element sub-blocks;
 * every isum an exact int32.  k a multiple of 256; w 16-byte aligned, rows
 * of k/256 super-blocks back to back; sx may be NULL (the kernel then sums
 * the codes).  zq_dmmv_isums with ZQ_Q4_K / ZQ_Q5_K / ZQ_Q6_K returns the
 * isum of every 32-element block. */
int zq_dmmv_q4_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream);
int zq_dmmv_q5_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 const int32_t *sx, float *y, uint32_t flags, void *stream);
int zq_dmmv_q6_k(const void *w, int64_t rows, int64_t k, const int8_t *qx, const float *dx,
                 float *y, uint32_t flags, void *stream);

/* The DMMV over a plain float weight matrix, the F16 and F32 members of the
 * DMMV shader family beside the block formats (habr "Как мы запустили 35B
 * LLM ...", section "Что такое DMMV", which lists separate shaders for the
 * K-quants, Q8_0, F16 and F32).  A float matrix has no blocks to pair with
 * int8 codes, so the activation is the fp32 vector itself:
 *   y[r] (+)= sum_j w[r][j] * x[j], accumulated in fp32.
 * wtype ZQ_F16 (little-endian binary16) or ZQ_F32 (binary32); w: rows x k,
 * row-major, 16-byte aligned; x [k] fp32, 16-byte aligned, finite; y [rows]
 * fp32; k a positive multiple of 8, at most 16384; flags 0 or
 * ZQ_ACCUMULATE. */
int zq_dmmv_float(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                  uint32_t flags, void *stream);

/* Multi-token DMMV: the DMMV above for n_tok = 1..8 activations sharing one
 * pass over the weights: the small-M matvec ("RTX 5090: Batched Prefill &
 * CUDA Graphs in ZINC", section "What's next", names a multi-row kernel for
 * the small-M expert matvecs; section "Prefill - a correction, and a better
 * GEMM" takes all tokens through one weight pass instead of one matvec per
 * token):
 *   y[t][r] (+)= sum_b fp32(d_w[r][b]) * dx[t][b] * isum_t[r][b].
 * wtype ZQ_Q4_0 or ZQ_Q8_0; qx [n_tok][k] int8 (16-byte aligned); dx
 * [n_tok][k/32]; sx [n_tok][k/32] for Q4_0, may be NULL (ignored for Q8_0);
 * y [n_tok][rows] fp32.  Tall matrices (rows >= 65536, e.g. the LM head)
 * with 3 or more tokens take the int8 matrix cores (one 16x16x32 MFMA per
 * 16 rows and block, all tokens at once) when their staged tokens fit the
 * workgroup's 64 KB of LDS (k = 2048: up to 8 tokens); so do shorter
 * matrices with 5 or more tokens, 64 to 128 blocks per row and at least 8 M
 * weights (their rows staged whole, 16 at a time).  The sums and the fp32
 * rescale are the same, only the association differs. */
int zq_dmmv_tokens(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                   const float *dx, const int32_t *sx, int32_t n_tok, float *y, uint32_t flags,
                   void *stream);

/* DMMV from the fp32 activation in one launch: y (+)= W . Q(x), where Q is
 * exactly the quantization of zq_quantize_act (same codes, scales, sums).
 * The input is the fp32 vector, as in the direct row-range DMMV slice of
 * "The first ZINC_RT model slices that actually count", section "The
 * one-wave workaround" (input fp32 vector, output fp32 rows, weight rows,
 * cols a multiple of 32, rows); each workgroup quantizes x into LDS while its
 * weight loads are in flight.
 * wtype: ZQ_Q4_0 or ZQ_Q8_0; w: rows x k blocks; x [k] fp32 (16-byte aligned,
 * finite); y [rows] fp32; flags: 0 or ZQ_ACCUMULATE; 32 <= k <= 16384.
 * qx_out [k] int8 (4-byte aligned), dx_out [k/32], sx_out [k/32]: when
 * qx_out is non-NULL the quantized activation is also stored there (dx_out
 * and sx_out may each be NULL); all three may be NULL. */
int zq_dmmv_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                uint32_t flags, int8_t *qx_out, float *dx_out, int32_t *sx_out, void *stream);

/* The K-quant DMMV from the fp32 activation in one launch: y (+)= W . Q(x),
 * Q exactly the quantization of zq_quantize_act, over Q4_K / Q5_K / Q6_K
 * super-blocks as zq_dmmv_q4_k / zq_dmmv_q5_k / zq_dmmv_q6_k read them.  The
 * fp32-input ABI of the direct DMMV slice ("The first ZINC_RT model slices
 * that actually count", section "The one-wave workaround"), with the
 * activation's quantization fused into the matvec kernel ("Как мы запустили
 * 35B LLM...", section "Фьюженные ядра"): each workgroup quantizes x into LDS
 * while its first weight loads are in flight.
 * wtype ZQ_Q4_K, ZQ_Q5_K or ZQ_Q6_K; w rows x k/256 super-blocks (16-byte
 * aligned); x [k] fp32 (16-byte aligned, finite); y [rows] fp32; flags 0 or
 * ZQ_ACCUMULATE; k a multiple of 256, 256 <= k <= 16384.  qx_out [k] int8
 * (4-byte aligned), dx_out [k/32], sx_out [k/32]: as for zq_dmmv_f32. */
int zq_dmmv_k_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                  uint32_t flags, int8_t *qx_out, float *dx_out, int32_t *sx_out, void *stream);

/* The multi-token DMMV from fp32 tokens: for t < n_tok,
 *   y[t] (+)= W . Q(x[t]),
 * the products of zq_dmmv_tokens on the codes of zq_quantize_act, which are
 * also stored in qx / dx / sx (always written; they may feed later products
 * against the same tokens).  The fp32-input ABI of the same slice ("The first
 * ZINC_RT model slices that actually count", section "The one-wave
 * workaround") for the multi-row matvec of "RTX 5090: Batched Prefill & CUDA
 * Graphs in ZINC", section "What's next".  Two launches: zq_quantize_act,
 * then zq_dmmv_tokens (every workgroup of the product needs every token's
 * codes, so quantizing inside it would repeat the whole quantization in each
 * workgroup; a producer that emits the codes, as zq_rms_norm_quantize does,
 * saves the first launch).  wtype ZQ_Q4_0 or ZQ_Q8_0; w rows x k blocks;
 * x [n_tok][k] fp32 (16-byte aligned, finite); qx [n_tok][k] int8 (16-byte
 * aligned); dx, sx [n_tok][k/32]; y [n_tok][rows]; 1 <= n_tok <= 8; flags 0
 * or ZQ_ACCUMULATE. */
int zq_dmmv_tokens_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                       int32_t n_tok, int8_t *qx, float *dx, int32_t *sx, float *y, uint32_t flags,
                       void *stream);

/* RMS normalization fused with the activation quantization (the
 * rms_norm_mul stage of "Bringing ZINC to NVIDIA: a CUDA backend, because
 * WSL2 only speaks CUDA", section "The roadmap: from 70 to a coherent
 * token", and the fused rms_norm_dmmv kernels of "CUDA backend for ZINC",
 * section 5, milestone M3; the formula is the reading documented with the
 * library).  Per token t, in fp32:
 *   ss = sum_i x[t][i]^2 (fused multiply-adds, order the kernel's),
 *   inv = 1 / sqrt(ss / k + eps)  (IEEE division and root),
 *   xn[t][i] = (x[t][i] * inv) * norm_w[i],
 * then qx/dx/sx = the zq_quantize_act quantization of xn.  norm_w [k] and
 * x (row stride x_stride, a multiple of 4) 16-byte aligned; eps finite and
 * >= 0; xn_out [n_tok][k] (16-byte aligned) receives xn when non-NULL; sx
 * may be NULL.  x must be finite and not all zero when eps = 0. */
int zq_rms_norm_quantize(const float *x, const float *norm_w, float eps, int64_t n_tok, int64_t k,
                         int64_t x_stride, int8_t *qx, float *dx, int32_t *sx, float *xn_out,
                         void *stream);
/* zq_dmmv_f32 with the RMS normalization in front: y (+)= W . Q(xn), xn as
 * in zq_rms_norm_quantize, in one launch (every workgroup reduces the sum of
 * squares of x while its weight loads are in flight).  xn_out [k] (16-byte
 * aligned, may be NULL) receives xn; qx_out / dx_out / sx_out as in
 * zq_dmmv_f32.  32 <= k <= 16384. */
int zq_rms_norm_dmmv_f32(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                         const float *norm_w, float eps, float *y, uint32_t flags, int8_t *qx_out,
                         float *dx_out, int32_t *sx_out, float *xn_out, void *stream);
/* The LM-head step with the final RMS normalization in front: as
 * zq_dmmv_f32_argmax on xn. */
int zq_rms_norm_dmmv_f32_argmax(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                                const float *norm_w, float eps, float *y, int32_t *out_idx,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Test hook: the per-block integer sums of the same DMMV inner loop,
 * isums[r][b] for every row r and block b (int32 [rows][k/32]). */
int zq_dmmv_isums(int wtype, const void *w, int64_t rows, int64_t k, const int8_t *qx,
                  const int32_t *sx, int32_t *isums, void *stream);

/* Index of the largest logit, ties to the lowest index (the exact argmax of the kernel library,
 * "CUDA backend for ZINC", section 5, M1 kernel library).  y [n] fp32 finite;
 * out_idx: one int32.  workspace: device scratch of at least
 * zq_argmax_workspace_bytes(n) bytes, 8-byte aligned. */
size_t zq_argmax_workspace_bytes(int64_t n);
int zq_argmax_f32(const float *y, int64_t n, int32_t *out_idx, void *workspace,
                  size_t workspace_bytes, void *stream);

/* The LM-head step in two launches: y = W . Q(x) over all rows, exactly as
 * zq_dmmv_f32 computes it (same codes, same rows, bit for bit), and out_idx
 * = the argmax of y with ties to the lowest row (the exact argmax of the kernel library, "CUDA
 * backend for ZINC", section 5; the vocab-output DMMV, "Как мы запустили
 * 35B LLM на видеокарте за $500", section "Утилизация полосы памяти по
 * операциям").  The DMMV launch is persistent: each workgroup quantizes the
 * activation once, walks several row groups and leaves the best (logit,
 * row) pair it wrote; one block then reduces those pairs.  k <= 16384 as
 * for zq_dmmv_f32.  x [k] fp32 16-byte aligned; y [rows] fp32 (written,
 * never accumulated); out_idx: one int32, or NULL to produce y only (one
 * launch; the partials are still written to the workspace).  workspace:
 * device scratch of at least zq_dmmv_f32_argmax_workspace_bytes() bytes,
 * 8-byte aligned, owned by the caller; its contents are undefined
 * afterwards.  1 <= rows <= INT32_MAX.  ZQ_EINVAL for k out of range or a
 * small workspace; nothing is launched then. */
size_t zq_dmmv_f32_argmax_workspace_bytes(void);
int zq_dmmv_f32_argmax(int wtype, const void *w, int64_t rows, int64_t k, const float *x, float *y,
                       int32_t *out_idx, void *workspace, size_t workspace_bytes, void *stream);

/* zq_dmmv_f32_argmax for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): the same two launches, the same rows and index bit for bit,
 * with no workspace argument.  The argmax partials live in a device array
 * of 16 KiB (2048 pairs) that the library holds on each GPU it runs on,
 * until the process ends; the call allocates and frees nothing.  Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (on
 * different streams, or from several threads) race: order them on one
 * stream.  Nothing in the array needs to start cleared: each call writes
 * every partial it reads.  Same arguments and limits as zq_dmmv_f32_argmax
 * (1 <= rows <= INT32_MAX, 32 <= k <= 16384, out_idx required); larger
 * sizes return ZQ_EINVAL, and ZQ_ELAUNCH if the runtime cannot resolve the
 * array on the current device. */
int zq_dmmv_f32_argmax_noalloc(int wtype, const void *w, int64_t rows, int64_t k, const float *x,
                               float *y, int32_t *out_idx, void *stream);

/* MoE router ("softmax_topk", "Bringing ZINC to NVIDIA", section "The roadmap:
 * from 70 to a coherent token"; "CUDA backend for ZINC", section 5): the
 * top_k largest of n_routed logits, largest first, ties to the lower id;
 * wts = softmax over the selected logits.  If shared_gate (one device fp32)
 * is non-NULL, a shared expert with id n_routed and weight sigmoid(g) is
 * appended (the pages' model adds one shared expert whose output is scaled
 * by a sigmoid gate: same page, section "The target model").  ids/wts: top_k (+1) entries.  1 <= top_k <= 64,
 * top_k <= n_routed <= 1024. */
int zq_moe_route(const float *logits, int32_t n_routed, int32_t top_k,
                 const float *shared_gate, int32_t *ids, float *wts, void *stream);

/* Expert-indexed DMMV over a list of selected experts (dmmv_*_moe and
 * moe_weighted_acc, "CUDA backend for ZINC", section 5; the selected experts
 * come from a GPU-resident work list, "RTX 5090: Batched Prefill & CUDA
 * Graphs in ZINC", section "Prefill -- a correction, and a better GEMM").
 * wtype: ZQ_Q4_0 / ZQ_Q8_0 (stride even), or ZQ_Q4_K / ZQ_Q5_K / ZQ_Q6_K (k a
 * multiple of 256, bank 16-byte aligned, stride a multiple of 16; the pages'
 * experts are Q4_K / Q5_K, "CUDA backend for ZINC", section 5).
 * bank: n_experts matrices of rows x k, expert e at bank + e*expert_stride_bytes.  ids [n_sel] int32, wts [n_sel] fp32 (device).  Activation
 * of slot s: qx + s*x_stride, dx/sx + s*(x_stride/32) (x_stride = 0 broadcasts
 * one activation; otherwise a multiple of 32).
 *   ZQ_MOE_GATHER:       y[s][r]   = (W[ids[s]] . x_s)[r]        y [n_sel][rows]
 *                        (wts unused, may be NULL; flags must be 0)
 *   ZQ_MOE_WEIGHTED_SUM: y[r]    (+)= sum_s wts[s]*(W[ids[s]] . x_s)[r]   y [rows]
 * An id outside [0, n_experts) is skipped (contributes nothing; in GATHER its
 * output row block is left untouched) and, if dev_status is non-NULL,
 * ZQ_ERANGE is stored to *dev_status (which is otherwise not written). */
int zq_dmmv_moe(int wtype, const void *bank, int64_t n_experts, int64_t expert_stride_bytes,
                int64_t rows, int64_t k, const int32_t *ids, const float *wts, int32_t n_sel,
                const int8_t *qx, const float *dx, const int32_t *sx, int64_t x_stride,
                int mode, float *y, uint32_t flags, int32_t *dev_status, void *stream);

/* SwiGLU then activation quantization ("swiglu", "CUDA backend for ZINC",
 * section 5): gu [n][2f] (gate in [.][0:f], up in [.][f:2f]);
 * h = silu(g)*u with silu(z) = z/(1+exp(-z)), evaluated in fp64 and rounded
 * once to fp32, then quantized exactly as zq_quantize_act:
 * qh [n][f] int8, dh [n][f/32] fp32, sh [n][f/32] int32 (may be NULL);
 * h_out [n][f] fp32 receives h when non-NULL.  f % 32 == 0. */
int zq_swiglu_quantize(const float *gu, int64_t n, int64_t f, int8_t *qh, float *dh,
                       int32_t *sh, float *h_out, void *stream);

/* The gate||up stage of the expert FFN with SwiGLU and the re-quantization
 * fused in (one launch): for every selected slot s and every 32-wide block
 * of the FFN width, the 32 gate rows and 32 up rows of expert ids[s] against
 * Q(x) (the quantization of zq_quantize_act), then h = silu(g)*u in fp64
 * rounded once to fp32, then h quantized exactly as zq_quantize_act.
 * ("dmmv_q4k_moe (gate/up)" and "swiglu", "CUDA backend for ZINC",
 * section 5; the fusion is that page's M3 "fused_gate_up" item.)
 * gu_bank: experts of [2*d_ff][d_model] (rows 0..d_ff-1 gate, d_ff.. up),
 * expert e at gu_bank + e*gu_stride_bytes; ids [n_sel]; x [d_model] fp32
 * (16-byte aligned); outputs qh [n_sel][d_ff] int8 (16-byte aligned),
 * dh [n_sel][d_ff/32] fp32, sh [n_sel][d_ff/32] int32 (may be NULL).
 * Optional (may be NULL) debug outputs: h_out [n_sel][d_ff] fp32 (16-byte
 * aligned) and gu_out [n_sel][2*d_ff] fp32, the gate||up rows.
 * wtype: ZQ_Q4_0 / ZQ_Q8_0 with d_model <= 4096, or ZQ_Q4_K / ZQ_Q5_K /
 * ZQ_Q6_K with d_model of 1024, 2048 or 4096 (the pages' routed experts are
 * Q4_K gate/up: "dmmv_q4k_moe"; K-quant banks 16-byte aligned with
 * gu_stride_bytes % 16 == 0; the row dot products are those of
 * zq_dmmv_q4_k and its kin).  d_ff % 32 == 0.  A bad id is skipped (its
 * outputs are left untouched) and reported through dev_status as in
 * zq_dmmv_moe. */
int zq_moe_gate_up(int wtype, const void *gu_bank, int64_t gu_stride_bytes, int64_t n_experts,
                   int64_t d_model, int64_t d_ff, const int32_t *ids, int32_t n_sel,
                   const float *x, int8_t *qh, float *dh, int32_t *sh, float *h_out,
                   float *gu_out, int32_t *dev_status, void *stream);

/* The same stage with the router folded in (the router of zq_moe_route, in
 * every workgroup): slot s < top_k takes the expert of rank s among the
 * n_routed logits, slot top_k the shared expert (id n_routed) when
 * shared_gate is non-NULL; ids / wts (top_k (+1) entries) receive the
 * router's output, bit for bit, for the down pass.  Outputs as
 * zq_moe_gate_up with n_sel = top_k (+1), for the same weight types and
 * d_model.  1 <= top_k <= 64, top_k <= n_routed <= 1024,
 * n_experts >= n_routed (+1). */
int zq_moe_gate_up_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                         int64_t n_experts, int64_t d_model, int64_t d_ff, const float *logits,
                         int32_t n_routed, int32_t top_k, const float *shared_gate,
                         const float *x, int32_t *ids, float *wts, int8_t *qh, float *dh,
                         int32_t *sh, float *h_out, float *gu_out, void *stream);

/* The gate/up stage of zq_moe_ffn_mixed in one launch: the routed experts
 * (gu_wtype, gu_bank at gu_stride_bytes) with the router folded in, as
 * zq_moe_gate_up_route, and the shared expert's own [2*d_ff][d_model]
 * matrix sh_gu in sh_wtype as slot top_k (id n_routed).  Any of the five
 * weight types each; d_model of 1024 or 2048; shared_gate required.
 * Outputs as zq_moe_gate_up_route with n_sel = top_k + 1, bit for bit
 * those of zq_moe_gate_up run on each matrix.  ("CUDA backend for ZINC",
 * section 5: dmmv_q4k_moe gate/up beside the Q8_0 shared expert.) */
int zq_moe_gate_up_mixed(int gu_wtype, const void *gu_bank, int64_t gu_stride_bytes,
                         int sh_wtype, const void *sh_gu, int64_t d_model, int64_t d_ff,
                         const float *logits, int32_t n_routed, int32_t top_k,
                         const float *shared_gate, const float *x, int32_t *ids, float *wts,
                         int8_t *qh, float *dh, int32_t *sh, void *stream);

/* One token through the selected experts in two launches: zq_moe_gate_up
 * (quantize x, gate||up rows, swiglu, re-quantize), then the down DMMV with
 * the weighted sum over the selected experts fused in.  (The expert chain of
 * "Bringing ZINC to NVIDIA", section "The roadmap: from 70 to a coherent
 * token": expert gate/up, swiglu, expert down, weighted accumulate; fused
 * as the gate/up and down-accumulate kernels of "CUDA backend for ZINC",
 * section 5, milestone M3.)  gu_bank: experts of [2*d_ff][d_model]
 * (rows 0..d_ff-1 gate, d_ff..2*d_ff-1 up); down_bank: [d_model][d_ff].
 * workspace: at least zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel) bytes,
 * 256-byte aligned.  y [d_model] (+)= sum_s wts[s] * down_s.
 * flags: 0 or ZQ_ACCUMULATE.  y may be x itself (the residual add of a
 * decode step): x is read only by the launches before y is written. */
size_t zq_moe_ffn_workspace_bytes(int64_t d_model, int64_t d_ff, int32_t n_sel);
int zq_moe_ffn(int wtype, const void *gu_bank, int64_t gu_stride_bytes, const void *down_bank,
               int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
               const int32_t *ids, const float *wts, int32_t n_sel, const float *x,
               void *workspace, size_t workspace_bytes, float *y, uint32_t flags,
               int32_t *dev_status, void *stream);

/* zq_moe_route followed by zq_moe_ffn, with the router folded into the
 * gate/up pass: the whole MoE block of one token in two launches, the expert
 * list never leaving the GPU ("RTX 5090: Batched Prefill & CUDA Graphs in
 * ZINC", sections "Prefill -- a correction, and a better GEMM" and "What's
 * next": GPU-side expert routing with no router round-trip).  Every gate/up
 * workgroup ranks the n_routed logits itself; the selection and weights are
 * those of zq_moe_route, bit for bit, and are written to ids / wts
 * (top_k + 1 entries with a shared gate, else top_k), which the down pass
 * then reads.  n_sel = top_k (+ 1): the workspace is
 * zq_moe_ffn_workspace_bytes(d_model, d_ff, n_sel).  n_experts >= n_routed
 * (+ 1 for the shared expert, id n_routed).  1 <= top_k <= 64,
 * top_k <= n_routed <= 1024.  Wide models (d_model > 4096) run the router,
 * quantize, gather and swiglu launches instead, with the same results.
 * flags: 0 or ZQ_ACCUMULATE. */
int zq_moe_ffn_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                     const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                     int64_t d_model, int64_t d_ff, const float *logits, int32_t n_routed,
                     int32_t top_k, const float *shared_gate, const float *x, int32_t *ids,
                     float *wts, void *workspace, size_t workspace_bytes, float *y,
                     uint32_t flags, void *stream);

/* One token through routed experts and a shared expert stored in different
 * formats, as the pages' model keeps them: routed gate/up Q4_K, routed down
 * Q5_K, shared expert Q8_0 ("CUDA backend for ZINC", section 5, "The target
 * model & milestone ordering": dmmv_q4k_moe gate/up, dmmv_q5k_moe down, the
 * Q8_0 shared expert with sigmoid_scale_acc).  gu_wtype / down_wtype /
 * sh_wtype: any of ZQ_Q4_0, ZQ_Q8_0, ZQ_Q4_K, ZQ_Q5_K, ZQ_Q6_K (K-quant
 * matrices need d_model resp. d_ff a multiple of 256; banks and matrices
 * 16-byte aligned for K-quants, 4 otherwise).  gu_bank: n_routed experts of
 * [2*d_ff][d_model] (rows 0..d_ff-1 gate) at gu_stride_bytes; down_bank:
 * n_routed experts of [d_model][d_ff]; sh_gu / sh_down: the shared expert's
 * two matrices (used when shared_gate is non-NULL).  The router is
 * zq_moe_route's (ids / wts receive top_k (+1) entries, the shared one with
 * id n_routed).  Gate/up: at d_model 1024 or 2048 one launch
 * (zq_moe_gate_up_mixed); at other widths that zq_moe_gate_up takes for
 * both types, the routed pass with the router folded in and the shared
 * expert's pass; otherwise five launches (router, quantize x, the routed and
 * the shared gate||up gathers, SwiGLU + re-quantize).  Down: with K-quant
 * routed experts, a Q4_0 / Q8_0 shared expert and d_ff of 256, 512, 1024 or
 * 2048, one launch that sums every term in one reduction; otherwise the
 * routed weighted sum, then the shared term added on.
 * y [d_model] (+)= the weighted sum; workspace >=
 * zq_moe_ffn_workspace_bytes(d_model, d_ff, top_k (+1)) bytes, 256-byte
 * aligned.  y may be x itself. */
int zq_moe_ffn_mixed(int gu_wtype, const void *gu_bank, int64_t gu_stride_bytes, int down_wtype,
                     const void *down_bank, int64_t down_stride_bytes, int sh_wtype,
                     const void *sh_gu, const void *sh_down, int64_t d_model, int64_t d_ff,
                     const float *logits, int32_t n_routed, int32_t top_k,
                     const float *shared_gate, const float *x, int32_t *ids, float *wts,
                     void *workspace, size_t workspace_bytes, float *y, uint32_t flags,
                     void *stream);

/* The MoE block of 1..8 tokens at once, each with its own router logits,
 * through one pass over the union of the experts they touch: the multi-row
 * expert kernel for the small-M matvecs of "RTX 5090: Batched Prefill & CUDA
 * Graphs in ZINC", section "What's next", with the expert list kept on the
 * GPU (same page, section "Prefill -- a correction, and a better GEMM").
 * For every token t it computes what zq_moe_ffn_route computes for that
 * token alone: the router of zq_moe_route on logits[t] (ids[t], wts[t]:
 * top_k (+1) entries each, the shared expert id n_routed with weight
 * sigmoid(shared_gate[t]) when shared_gate is non-NULL), then
 *   y[t] (+)= sum_s wts[t][s] * down_{ids[t][s]}(Q(swiglu(gate||up_{ids[t][s]}(Q(x[t]))))),
 * the gate/up codes and scales bit for bit those of the single-token stages,
 * the weighted sum taken over the slots in order.  Three launches: route
 * (every token's router and quantized activation), gate/up (each distinct
 * expert's rows read once for all tokens that selected it; it also records
 * which tokens share each expert), and down with the per-token weighted sums
 * (each distinct expert's rows read once).
 * wtype ZQ_Q4_0 or ZQ_Q8_0; banks as zq_moe_ffn (n_experts >= n_routed + 1
 * with a shared expert); d_model a multiple of 32 up to 4096; d_ff 256, 512,
 * 1024 or 2048.  logits [n_tok][n_routed]; shared_gate [n_tok] or NULL;
 * x [n_tok][d_model] fp32 (16-byte aligned); ids [n_tok][n_sel], wts
 * [n_tok][n_sel] receive the router's output (n_sel = top_k (+1)); y
 * [n_tok][d_model] (may be x itself: x is read only by launches before y is
 * written).  workspace >= zq_moe_ffn_tokens_workspace_bytes(d_model, d_ff,
 * n_tok, n_sel) bytes, 256-byte aligned.  1 <= n_tok <= 8, 1 <= top_k <= 64,
 * top_k <= n_routed <= 1024; flags 0 or ZQ_ACCUMULATE. */
size_t zq_moe_ffn_tokens_workspace_bytes(int64_t d_model, int64_t d_ff, int32_t n_tok,
                                         int32_t n_sel);
int zq_moe_ffn_tokens(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                      const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                      int64_t d_model, int64_t d_ff, const float *logits, int32_t n_routed,
                      int32_t top_k, const float *shared_gate, const float *x, int32_t n_tok,
                      int32_t *ids, float *wts, void *workspace, size_t workspace_bytes, float *y,
                      uint32_t flags, void *stream);

/* One decode layer's MoE block from the un-normalized state, the layer's
 * RMS norm and router matvec included:
 *   xn = rms_norm(x) * norm_w, as zq_rms_norm_dmmv_f32 computes it,
 *   logits = R . Q(xn), R the Q8_0 router matrix [n_routed][d_model],
 *   then the routed MoE block of zq_moe_ffn_route on xn and those logits:
 *   y (+)= sum_s wts[s] * down_{ids[s]}(Q(swiglu(gate||up_{ids[s]}(Q(xn))))).
 * The per-token order of "Bringing ZINC to NVIDIA: a CUDA backend, because
 * WSL2 only speaks CUDA", section "The roadmap: from 70 to a coherent token"
 * (router DMMV, softmax_topk, expert gate/up, swiglu, expert down with the
 * weighted accumulate, residual accumulate), in three launches:
 * zq_rms_norm_dmmv_f32, then zq_moe_ffn_route.  (Running the norm and the
 * router inside every gate/up workgroup instead, two launches, measured
 * slower at the pages' widths: each of the 144 workgroups then reads the
 * whole 278 KB router.)  xn_out [d_model] (16-byte aligned) and logits_out
 * [n_routed] receive xn and the logits (always written); xn_out must not
 * overlap x.  Other arguments as zq_moe_ffn_route; norm_w [d_model] 16-byte
 * aligned, eps finite and >= 0, d_model <= 16384; y may be x itself (the
 * residual add, with ZQ_ACCUMULATE). */
int zq_moe_ffn_norm_route(int wtype, const void *gu_bank, int64_t gu_stride_bytes,
                          const void *down_bank, int64_t down_stride_bytes, int64_t n_experts,
                          int64_t d_model, int64_t d_ff, const void *router_w,
                          const float *norm_w, float eps, const float *x, int32_t n_routed,
                          int32_t top_k, const float *shared_gate, float *xn_out,
                          float *logits_out, int32_t *ids, float *wts, void *workspace,
                          size_t workspace_bytes, float *y, uint32_t flags, void *stream);

/* Batched prefill GEMM (all prompt tokens through one tiled GEMM rather than
 * one matvec per token: "RTX 5090: Batched Prefill & CUDA Graphs in ZINC", opening answer
 * and section "Prefill -- a correction, and a better GEMM"; the dequant is
 * fused into the GEMM as the same page's closing paragraph recommends):
 *   Y[m][n] (+)= sum_b dx[m][b] * d_w[n][b] * isum(m, n, b),
 * with each block's integer sum taken on int8 matrix cores.
 * w: n x k weight matrix; qx [m][k] int8; dx [m][k/32]; sx [m][k/32] (may be
 * NULL); y [m][n] fp32 row-major.  flags: 0 or ZQ_ACCUMULATE. */
int zq_gemm_prefill(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx,
                    const float *dx, const int32_t *sx, int64_t m, float *y, uint32_t flags,
                    void *stream);

/* Test hook: the per-block integer sums of the same GEMM tile loop for
 * tokens [m0, m1) and weight rows [n0, n1): isums[(mm-m0)][(nn-n0)][b],
 * int32 [(m1-m0)][(n1-n0)][k/32]. */
int zq_gemm_isums(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx,
                  const int32_t *sx, int64_t m, int64_t m0, int64_t m1, int64_t n0, int64_t n1,
                  int32_t *isums, void *stream);

/* Measurement hook: a plain streaming read of `bytes` bytes of buf with
 * 16-byte loads spread over the whole chip, nothing computed from them but a
 * fold that decides whether the one word *sink is written (practically
 * never).  Its rate is the read ceiling the weight-streaming kernels are
 * reported against beside the chip's nominal HBM peak.  buf 16-byte aligned,
 * bytes a multiple of 16; sink one uint32. */
int zq_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ZQ_H */
