/*
 * zqref.c -- the CPU oracle for the block-quantized decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; it reads the same raw input bytes and nothing else.
 *
 * Plain, scalar, deliberately slow C.  Build with
 *     gcc -O2 -ffp-contract=off -fno-fast-math -std=c11 -fPIC -shared
 * so that every fp32 step below is one IEEE round-to-nearest-even operation
 * and no multiply-add is fused.
 *
 * What it computes and where the pages say so:
 *   - int8 x int8 -> int32 dot products of packed quants: "Bringing ZINC to
 *     NVIDIA", section "The reassuring result: ZINC's matmuls are __dp4a, not
 *     tensor cores" (dotPacked4x8AccSatEXT / v_dot4_i32_i8 / __dp4a, and the
 *     1*5+2*6+3*7+4*8 = 70 check).
 *   - GGML block layouts, unchanged in every backend: the same section (it
 *     names Q8_0 and its 32-element blocks and says the layouts match GGML's
 *     exactly), and "CUDA backend for ZINC", section 4 "Kernel port
 *     strategy".  Q8_0 = {fp16 d; int8 q[32]} (34 bytes), value
 *     q*d.  Q4_0 = {fp16 d; uint8 qs[16]} (18 bytes), value (nib-8)*d, element
 *     j<16 in the low nibble of qs[j], element j+16 in the high nibble.
 *   - DMMV = read quantized weights, dequantize in registers, multiply by the
 *     input vector, write the row result: habr "Как мы запустили 35B LLM ...",
 *     section "Что такое DMMV".
 *   - MoE chain softmax_topk -> expert gate/up DMMV -> swiglu -> expert down
 *     DMMV -> weighted accumulate, plus a sigmoid-gated shared expert:
 *     "Bringing ZINC to NVIDIA", section "The roadmap: from 70 to a coherent
 *     token", and "CUDA backend for ZINC", section 5 (milestone M1).
 *   - an exact argmax: "CUDA backend for ZINC", section 5 (the M1 kernel library).
 *   - the K-quant super-blocks Q4_K / Q5_K / Q6_K (256 elements), also GGML's
 *     layouts unchanged: "Bringing ZINC to NVIDIA", section "The reassuring
 *     result" (the three K-quant formats and their super-blocks of 256), and
 *     "CUDA backend for ZINC", section 5 (the Q4_K matvec there follows
 *     GGML's dequantization, scale/min unpacking included).  Layouts, as
 *     published with GGML:
 *       Q4_K (144 B): fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block scales
 *         and mins, 128 bytes of nibbles.  Eight sub-blocks of 32; element e
 *         of 64-group g (e < 32: low nibble, else high nibble of byte
 *         16 + 32g + e%32) belongs to sub-block 2g + e/32; value
 *         d*sc*q - dmin*m with q in 0..15.
 *       Q5_K (176 B): as Q4_K, plus 32 bytes of fifth bits after the scales
 *         (bit 2g for the low-nibble element, 2g+1 for the high-nibble one,
 *         in byte e%32), the nibbles following; q in 0..31.
 *       Q6_K (210 B): 128 bytes of low nibbles, 64 bytes of 2-bit highs, 16
 *         int8 sub-block scales, fp16 d last.  Sixteen sub-blocks of 16
 *         (element index / 16); value d*scale*(q - 32), q in 0..63.
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *   - activation block scale d = amax/127 in fp32, no zero point; quantize by
 *     multiplying with the fp32 reciprocal and rounding half away from zero;
 *     clamp to [-127,127]; an all-zero block gives d = 0 and q = 0;
 *   - per-block activation sum s = sum(q) is part of the quantized activation;
 *   - routing: top-k by logit (ties to the lower id), weights = softmax over
 *     the selected k; shared expert weight = sigmoid(g);
 *   - swiglu h = silu(g)*u with silu(z) = z/(1+exp(-z)), evaluated in fp64
 *     and rounded once to fp32;
 *   - rms_norm_mul ("Bringing ZINC to NVIDIA", section "The roadmap: from 70
 *     to a coherent token"; fused rms_norm_dmmv kernels in "CUDA backend for
 *     ZINC", section 5, milestone M3): xn_i = x_i / sqrt(mean_j x_j^2 + eps)
 *     * w_i, the root-mean-square normalization with an elementwise weight,
 *     eps an argument; evaluated in fp64.
 *
 * Every fp32 row output of the path is compared against the fp64 reference
 * y_ref computed here together with its error scale S = sum_b |t_b|.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ZQREF_OK 0
#define ZQREF_EINVAL (-1)
#define ZQREF_ENONFINITE (-2)
#define ZQREF_EOVERFLOW (-3)
#define ZQREF_EIDENTITY (-4)

#define ZQREF_Q4_0 4
#define ZQREF_Q8_0 8
#define ZQREF_Q4_K 12
#define ZQREF_Q5_K 13
#define ZQREF_Q6_K 14

int zqref_version(void) { return 1; }

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE binary16 -> double by bit manipulation: sign, 5-bit exponent with
 * bias 15, 10-bit mantissa; exponent 0 is subnormal (m * 2^-24). */
double zqref_fp16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);
    }
    return sign ? -v : v;
}

void zqref_fp16_to_f64_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = zqref_fp16_to_f64(h[i]);
}

/* ------------------------------------------------------- block layout -- */

static int64_t block_bytes(int wtype)
{
    if (wtype == ZQREF_Q8_0) return 34;
    if (wtype == ZQREF_Q4_0) return 18;
    return -1;
}

int64_t zqref_block_bytes(int wtype) { return block_bytes(wtype); }

static double block_scale(const uint8_t *blk)
{
    uint16_t h = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8)); /* little-endian */
    return zqref_fp16_to_f64(h);
}

/* The integer weight value of element i (0..31) of one block. */
static int block_value(int wtype, const uint8_t *blk, int i)
{
    if (wtype == ZQREF_Q8_0) {
        return (int)(int8_t)blk[2 + i];
    } else {
        int nib = (i < 16) ? (blk[2 + i] & 0x0F) : (blk[2 + (i - 16)] >> 4);
        return nib - 8;
    }
}

/* Unsigned nibble of element i of a Q4_0 block (0..15). */
static int q4_nibble(const uint8_t *blk, int i)
{
    return (i < 16) ? (blk[2 + i] & 0x0F) : (blk[2 + (i - 16)] >> 4);
}

/* Decode one block: d (double) and the 32 integer values. */
int zqref_decode_block(int wtype, const uint8_t *blk, double *d, int32_t *vals)
{
    if (block_bytes(wtype) < 0) return ZQREF_EINVAL;
    *d = block_scale(blk);
    for (int i = 0; i < 32; i++) vals[i] = block_value(wtype, blk, i);
    return ZQREF_OK;
}

/* ------------------------------------------------ activation quantizer -- */

/* One block of 32 fp32 activations -> 32 int8 codes, scale d, sum s.
 * amax = max|x|; d = amax/127 (fp32 division); id = 1/d (0 if d == 0);
 * q = round_half_away(x*id), clamped to [-127,127]; s = sum(q). */
int zqref_quantize_block(const float *x, int8_t *q, float *d_out, int32_t *s_out)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(x[i])) return ZQREF_ENONFINITE;
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    int32_t s = 0;
    for (int i = 0; i < 32; i++) {
        float v = x[i] * id;
        int qi = (int)roundf(v);
        if (qi > 127) qi = 127;
        if (qi < -127) qi = -127;
        q[i] = (int8_t)qi;
        s += qi;
    }
    *d_out = d;
    *s_out = s;
    return ZQREF_OK;
}

/* x[t][k] with row stride x_stride (elements) -> qx[t][k], dx[t][k/32],
 * sx[t][k/32] (sx may be NULL). */
int zqref_quantize_act(const float *x, int64_t n_tok, int64_t k, int64_t x_stride,
                       int8_t *qx, float *dx, int32_t *sx)
{
    if (k <= 0 || k % 32 != 0 || n_tok < 0 || x_stride < k) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t t = 0; t < n_tok; t++) {
        for (int64_t b = 0; b < nb; b++) {
            int32_t s;
            int rc = zqref_quantize_block(x + t * x_stride + b * 32, qx + t * k + b * 32,
                                          dx + t * nb + b, &s);
            if (rc != ZQREF_OK) return rc;
            if (sx) sx[t * nb + b] = s;
        }
    }
    return ZQREF_OK;
}

/* --------------------------------------------------------- block dots -- */

/* isum = sum_i w_i * qx_i over one block, exact in int64; it must fit int32.
 * For Q4_0 the second form sum_i nib_i*qx_i - 8*sum_i qx_i is also evaluated
 * and must agree (an exact integer identity). */
int zqref_block_isum(int wtype, const uint8_t *blk, const int8_t *qx, int32_t *isum)
{
    if (block_bytes(wtype) < 0) return ZQREF_EINVAL;
    int64_t acc = 0;
    for (int i = 0; i < 32; i++) acc += (int64_t)block_value(wtype, blk, i) * (int64_t)qx[i];
    if (acc > INT32_MAX || acc < INT32_MIN) return ZQREF_EOVERFLOW;
    if (wtype == ZQREF_Q4_0) {
        int64_t raw = 0, s = 0;
        for (int i = 0; i < 32; i++) {
            raw += (int64_t)q4_nibble(blk, i) * (int64_t)qx[i];
            s += qx[i];
        }
        if (raw - 8 * s != acc) return ZQREF_EIDENTITY;
    }
    *isum = (int32_t)acc;
    return ZQREF_OK;
}

/* ------------------------------------------------------ row references -- */

/* For each evaluated row r (row_idx[i], or i when row_idx is NULL):
 *   t_rb = (double)d_w[r][b] * (double)dx[b] * (double)isum[r][b]
 *   y_ref[i] = sum_b t_rb  (sequential, fp64)      S[i] = sum_b |t_rb|
 * With y_prev (accumulate): y_ref += y_prev[r], S += |y_prev[r]|.
 * isums (optional) receives isum[i][b]. */
int zqref_dmmv_rows(int wtype, const uint8_t *w, int64_t rows, int64_t k,
                    const int8_t *qx, const float *dx, const float *y_prev,
                    const int64_t *row_idx, int64_t n_eval,
                    double *y_ref, double *S, int32_t *isums)
{
    int64_t bb = block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 32 != 0 || rows < 0 || n_eval < 0) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0, s = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + (r * nb + b) * bb;
            int32_t isum;
            int rc = zqref_block_isum(wtype, blk, qx + b * 32, &isum);
            if (rc != ZQREF_OK) return rc;
            if (isums) isums[i * nb + b] = isum;
            double t = block_scale(blk) * (double)dx[b] * (double)isum;
            y += t;
            s += fabs(t);
        }
        if (y_prev) {
            y += (double)y_prev[r];
            s += fabs((double)y_prev[r]);
        }
        y_ref[i] = y;
        if (S) S[i] = s;
    }
    return ZQREF_OK;
}

/* Brute force: dequantize every weight (d_w * value) and every activation
 * (dx * qx) to fp64 and take the plain dot product, element by element. */
int zqref_dmmv_bruteforce(int wtype, const uint8_t *w, int64_t rows, int64_t k,
                          const int8_t *qx, const float *dx,
                          const int64_t *row_idx, int64_t n_eval, double *y_bf)
{
    int64_t bb = block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 32 != 0) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0;
        for (int64_t j = 0; j < k; j++) {
            const uint8_t *blk = w + (r * nb + j / 32) * bb;
            double wv = block_scale(blk) * (double)block_value(wtype, blk, (int)(j % 32));
            double xv = (double)dx[j / 32] * (double)qx[j];
            y += wv * xv;
        }
        y_bf[i] = y;
    }
    return ZQREF_OK;
}

/* ------------------------------------------------------ float weights -- */

#define ZQREF_F16 16
#define ZQREF_F32 32

/* DMMV over a matrix of plain floats, the F16 / F32 members of the DMMV
 * shader family beside the block formats (habr "Как мы запустили 35B LLM
 * ...", section "Что такое DMMV"; the same read-dequantize-multiply-write
 * operation with a float weight).  A float matrix has no blocks to pair with
 * int8 codes, so the activation is the fp32 vector itself (the reading
 * documented with the library):
 *   y_ref[i] = sum_j (double)w[r][j] * (double)x[j]  (sequential, fp64)
 *   S[i]     = sum_j |w[r][j] * x[j]|
 * w: rows x k, row-major, little-endian binary16 (ZQREF_F16) or binary32
 * (ZQREF_F32).  With y_prev (accumulate): y_ref += y_prev[r], S += |y_prev[r]|.
 * Non-finite weights or activations are refused. */
static double float_weight(int wtype, const uint8_t *w, int64_t idx)
{
    if (wtype == ZQREF_F16) return zqref_fp16_to_f64((uint16_t)(w[2 * idx] | (w[2 * idx + 1] << 8)));
    float f;
    memcpy(&f, w + 4 * idx, 4);
    return (double)f;
}

int zqref_float_dmmv_rows(int wtype, const uint8_t *w, int64_t rows, int64_t k, const float *x,
                          const float *y_prev, const int64_t *row_idx, int64_t n_eval,
                          double *y_ref, double *S)
{
    if ((wtype != ZQREF_F16 && wtype != ZQREF_F32) || k <= 0 || rows < 0 || n_eval < 0)
        return ZQREF_EINVAL;
    for (int64_t j = 0; j < k; j++)
        if (!isfinite(x[j])) return ZQREF_ENONFINITE;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0, s = 0.0;
        for (int64_t j = 0; j < k; j++) {
            double wv = float_weight(wtype, w, r * k + j);
            if (!isfinite(wv)) return ZQREF_ENONFINITE;
            double t = wv * (double)x[j];
            y += t;
            s += fabs(t);
        }
        if (y_prev) {
            y += (double)y_prev[r];
            s += fabs((double)y_prev[r]);
        }
        y_ref[i] = y;
        if (S) S[i] = s;
    }
    return ZQREF_OK;
}

/* The unquantized-activation product sum_j w_deq[r][j] * x[j] (report only). */
int zqref_dmmv_true(int wtype, const uint8_t *w, int64_t rows, int64_t k, const float *x,
                    const int64_t *row_idx, int64_t n_eval, double *y_true)
{
    int64_t bb = block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 32 != 0) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0;
        for (int64_t j = 0; j < k; j++) {
            const uint8_t *blk = w + (r * nb + j / 32) * bb;
            y += block_scale(blk) * (double)block_value(wtype, blk, (int)(j % 32)) * (double)x[j];
        }
        y_true[i] = y;
    }
    return ZQREF_OK;
}

/* Bound on |y_ref - y_true| from rounding the activation: each |x - d*q| is at
 * most d/2, so the row error is at most sum_b |d_w| * (dx_b/2) * sum_i |w_i|. */
int zqref_quant_error_bound(int wtype, const uint8_t *w, int64_t rows, int64_t k,
                            const float *dx, const int64_t *row_idx, int64_t n_eval,
                            double *bound)
{
    int64_t bb = block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 32 != 0) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double e = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + (r * nb + b) * bb;
            double sw = 0.0;
            for (int j = 0; j < 32; j++) sw += fabs((double)block_value(wtype, blk, j));
            e += fabs(block_scale(blk)) * ((double)dx[b] / 2.0) * sw;
        }
        bound[i] = e;
    }
    return ZQREF_OK;
}

/* ------------------------------------------------- K-quant super-blocks -- */

int64_t zqref_k_block_bytes(int wtype)
{
    if (wtype == ZQREF_Q4_K) return 144;
    if (wtype == ZQREF_Q5_K) return 176;
    if (wtype == ZQREF_Q6_K) return 210;
    return ZQREF_EINVAL;
}

static uint16_t le16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* The 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes s:
 * sub-blocks 0-3 keep their scale in the low 6 bits of s[j] and their min in
 * the low 6 bits of s[j+4]; sub-blocks 4-7 keep the low 4 bits of scale and
 * min in the two nibbles of s[j+4] and their top 2 bits in the top 2 bits of
 * s[j-4] (scale) and s[j] (min). */
static void k_scale_min(const uint8_t *s, int j, int32_t *sc, int32_t *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Decode one super-block: d, dmin (0 for Q6_K), the sub-block scales and
 * mins (8 of each for Q4_K / Q5_K, 16 scales for Q6_K with mins 0), and the
 * 256 unsigned codes q in element order. */
int zqref_k_decode(int wtype, const uint8_t *sb, double *d, double *dmin, int32_t *sc,
                   int32_t *mn, int32_t *q)
{
    if (wtype == ZQREF_Q4_K || wtype == ZQREF_Q5_K) {
        *d = zqref_fp16_to_f64(le16(sb));
        *dmin = zqref_fp16_to_f64(le16(sb + 2));
        for (int j = 0; j < 8; j++) k_scale_min(sb + 4, j, &sc[j], &mn[j]);
        const uint8_t *qh = sb + 16;
        const uint8_t *qs = sb + (wtype == ZQREF_Q4_K ? 16 : 48);
        for (int e = 0; e < 256; e++) {
            int g = e / 64, l = e % 32, hi = (e % 64) >= 32;
            int v = hi ? (qs[32 * g + l] >> 4) : (qs[32 * g + l] & 15);
            if (wtype == ZQREF_Q5_K) v |= ((qh[l] >> (2 * g + hi)) & 1) << 4;
            q[e] = v;
        }
        return ZQREF_OK;
    }
    if (wtype == ZQREF_Q6_K) {
        const uint8_t *ql = sb, *qh = sb + 128;
        const int8_t *scales = (const int8_t *)(sb + 192);
        *d = zqref_fp16_to_f64(le16(sb + 208));
        *dmin = 0.0;
        for (int j = 0; j < 16; j++) {
            sc[j] = scales[j];
            mn[j] = 0;
        }
        for (int e = 0; e < 256; e++) {
            int h = e / 128, c = (e % 128) / 32, l = e % 32;
            int lo = ql[64 * h + 32 * (c & 1) + l];
            lo = (c < 2) ? (lo & 15) : (lo >> 4);
            int top = (qh[32 * h + l] >> (2 * c)) & 3;
            q[e] = lo | (top << 4);
        }
        return ZQREF_OK;
    }
    return ZQREF_EINVAL;
}

/* Row references over K-quant weights against the int8 activation blocks of
 * 32.  Each activation block b lines up with one 32-element sub-block of
 * Q4_K / Q5_K, or with two 16-element sub-blocks of Q6_K.  Per block:
 *   Q4_K / Q5_K: isum_b = sum q*qx, s_b = sum qx (exact integers),
 *     t_b = dx_b * (d*sc*isum_b - dmin*m*s_b),
 *     S += |dx_b| * (|d*sc*isum_b| + |dmin*m*s_b|);
 *   Q6_K: isum_b = sum sc(e) * (q - 32) * qx (the scale of each element's
 *     16-element sub-block; an exact integer), t_b = dx_b * d * isum_b,
 *     S += |t_b|.
 * y_ref = sum_b t_b in fp64, sequentially; y_prev / row_idx / isums as in
 * zqref_dmmv_rows. */
int zqref_k_dmmv_rows(int wtype, const uint8_t *w, int64_t rows, int64_t k, const int8_t *qx,
                      const float *dx, const float *y_prev, const int64_t *row_idx,
                      int64_t n_eval, double *y_ref, double *S, int32_t *isums)
{
    int64_t bb = zqref_k_block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 256 != 0 || rows < 0 || n_eval < 0) return ZQREF_EINVAL;
    int64_t nsb = k / 256, nb = k / 32;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0, sabs = 0.0;
        for (int64_t u = 0; u < nsb; u++) {
            double d, dmin;
            int32_t sc[16], mn[16], q[256];
            int rc = zqref_k_decode(wtype, w + (r * nsb + u) * bb, &d, &dmin, sc, mn, q);
            if (rc != ZQREF_OK) return rc;
            for (int j = 0; j < 8; j++) {
                int64_t b = u * 8 + j;
                const int8_t *xb = qx + b * 32;
                int64_t is = 0, sx = 0;
                for (int e = 0; e < 32; e++) {
                    int64_t code = q[32 * j + e];
                    if (wtype == ZQREF_Q6_K) is += (int64_t)sc[(32 * j + e) / 16] * (code - 32) * xb[e];
                    else is += code * xb[e];
                    sx += xb[e];
                }
                if (is > INT32_MAX || is < INT32_MIN) return ZQREF_EOVERFLOW;
                if (isums) isums[i * nb + b] = (int32_t)is;
                double t, tabs;
                if (wtype == ZQREF_Q6_K) {
                    t = (double)dx[b] * d * (double)is;
                    tabs = fabs(t);
                } else {
                    double a1 = d * (double)sc[j] * (double)is;
                    double a2 = dmin * (double)mn[j] * (double)sx;
                    t = (double)dx[b] * (a1 - a2);
                    tabs = fabs((double)dx[b]) * (fabs(a1) + fabs(a2));
                }
                y += t;
                sabs += tabs;
            }
        }
        if (y_prev) {
            y += (double)y_prev[r];
            sabs += fabs((double)y_prev[r]);
        }
        y_ref[i] = y;
        if (S) S[i] = sabs;
    }
    return ZQREF_OK;
}

/* Brute force: every weight dequantized to fp64 on its own (d*sc*q - dmin*m,
 * or d*sc*(q-32)), every activation element dx*qx, plain dot product. */
int zqref_k_bruteforce(int wtype, const uint8_t *w, int64_t rows, int64_t k, const int8_t *qx,
                       const float *dx, const int64_t *row_idx, int64_t n_eval, double *y_bf)
{
    int64_t bb = zqref_k_block_bytes(wtype);
    if (bb < 0 || k <= 0 || k % 256 != 0) return ZQREF_EINVAL;
    int64_t nsb = k / 256;
    for (int64_t i = 0; i < n_eval; i++) {
        int64_t r = row_idx ? row_idx[i] : i;
        if (r < 0 || r >= rows) return ZQREF_EINVAL;
        double y = 0.0;
        for (int64_t u = 0; u < nsb; u++) {
            double d, dmin;
            int32_t sc[16], mn[16], q[256];
            int rc = zqref_k_decode(wtype, w + (r * nsb + u) * bb, &d, &dmin, sc, mn, q);
            if (rc != ZQREF_OK) return rc;
            for (int e = 0; e < 256; e++) {
                double wv;
                if (wtype == ZQREF_Q6_K) wv = d * (double)sc[e / 16] * (double)(q[e] - 32);
                else wv = d * (double)sc[e / 32] * (double)q[e] - dmin * (double)mn[e / 32];
                int64_t j = u * 256 + e;
                y += wv * ((double)dx[j / 32] * (double)qx[j]);
            }
        }
        y_bf[i] = y;
    }
    return ZQREF_OK;
}

/* ------------------------------------------------------------- argmax -- */

/* Lowest index holding the maximum (strict '>' scan).  -1 for n <= 0. */
int64_t zqref_argmax_f32(const float *y, int64_t n)
{
    if (n <= 0) return -1;
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (y[i] > y[best]) best = i;
    return best;
}

/* ------------------------------------------------------------ MoE -------- */

/* Routing: pick top_k of n_routed logits, largest first, ties to the lower id;
 * weights = softmax over the selected logits (max-subtracted, fp64).  When
 * shared_gate is non-NULL a shared expert with id n_routed and weight
 * sigmoid(*shared_gate) is appended.  ids/wts hold top_k (+1) entries. */
int zqref_moe_route(const float *logits, int n_routed, int top_k, const float *shared_gate,
                    int32_t *ids, double *wts)
{
    if (n_routed <= 0 || top_k <= 0 || top_k > n_routed || n_routed > 4096) return ZQREF_EINVAL;
    unsigned char taken[4096];
    memset(taken, 0, sizeof(taken));
    for (int j = 0; j < n_routed; j++)
        if (!isfinite(logits[j])) return ZQREF_ENONFINITE;
    for (int s = 0; s < top_k; s++) {
        int best = -1;
        for (int j = 0; j < n_routed; j++) {
            if (taken[j]) continue;
            if (best < 0 || logits[j] > logits[best]) best = j;
        }
        taken[best] = 1;
        ids[s] = best;
    }
    double m = (double)logits[ids[0]];
    double z = 0.0;
    for (int s = 0; s < top_k; s++) {
        wts[s] = exp((double)logits[ids[s]] - m);
        z += wts[s];
    }
    for (int s = 0; s < top_k; s++) wts[s] /= z;
    if (shared_gate) {
        ids[top_k] = n_routed;
        wts[top_k] = 1.0 / (1.0 + exp(-(double)*shared_gate));
    }
    return ZQREF_OK;
}

/* gu[s][0:f] = gate rows, gu[s][f:2f] = up rows; h[s][i] = silu(g)*u,
 * silu(z) = z / (1 + exp(-z)), fp64, one rounding to fp32. */
int zqref_swiglu(const float *gu, int64_t n, int64_t f, float *h)
{
    if (n < 0 || f <= 0) return ZQREF_EINVAL;
    for (int64_t s = 0; s < n; s++) {
        for (int64_t i = 0; i < f; i++) {
            double g = (double)gu[s * 2 * f + i];
            double u = (double)gu[s * 2 * f + f + i];
            if (!isfinite(g) || !isfinite(u)) return ZQREF_ENONFINITE;
            double silu = g / (1.0 + exp(-g));
            h[s * f + i] = (float)(silu * u);
        }
    }
    return ZQREF_OK;
}

/* RMS normalization with an elementwise weight, per token t:
 *   xn[t][i] = x[t][i] / sqrt((sum_j x[t][j]^2) / k + eps) * w[i],
 * every step in fp64 (the sum sequential), the result kept in fp64.
 * x: [n_tok][x_stride] (first k used); w: [k]; eps >= 0. */
int zqref_rms_norm(const float *x, const float *w, double eps, int64_t n_tok, int64_t k,
                   int64_t x_stride, double *xn)
{
    if (n_tok < 0 || k <= 0 || x_stride < k || !(eps >= 0.0) || !isfinite(eps)) return ZQREF_EINVAL;
    for (int64_t i = 0; i < k; i++)
        if (!isfinite(w[i])) return ZQREF_ENONFINITE;
    for (int64_t t = 0; t < n_tok; t++) {
        const float *xt = x + t * x_stride;
        double ss = 0.0;
        for (int64_t i = 0; i < k; i++) {
            if (!isfinite(xt[i])) return ZQREF_ENONFINITE;
            ss += (double)xt[i] * (double)xt[i];
        }
        double ms = ss / (double)k + eps;
        if (!(ms > 0.0)) return ZQREF_EINVAL;  /* all-zero x with eps = 0 */
        double r = sqrt(ms);
        for (int64_t i = 0; i < k; i++) xn[t * k + i] = (double)xt[i] / r * (double)w[i];
    }
    return ZQREF_OK;
}

/* ------------------------------------------------------------- GEMM ----- */

/* Prefill GEMM entries: Y[m][n] = sum_b dx[m][b] * d_w[n][b] * isum(m,n,b),
 * i.e. row n of W against token m's quantized activation, evaluated for the
 * listed (m, n) pairs.  W is [n_rows][k/32] blocks, qx [m_tok][k]. */
int zqref_gemm_entries(int wtype, const uint8_t *w, int64_t n_rows, int64_t k,
                       const int8_t *qx, const float *dx, int64_t m_tok,
                       const int64_t *mi, const int64_t *ni, int64_t n_pairs,
                       double *y, double *S)
{
    if (k <= 0 || k % 32 != 0) return ZQREF_EINVAL;
    int64_t nb = k / 32;
    for (int64_t p = 0; p < n_pairs; p++) {
        if (mi[p] < 0 || mi[p] >= m_tok || ni[p] < 0 || ni[p] >= n_rows) return ZQREF_EINVAL;
        int rc = zqref_dmmv_rows(wtype, w, n_rows, k, qx + mi[p] * k, dx + mi[p] * nb, NULL,
                                 &ni[p], 1, &y[p], &S[p], NULL);
        if (rc != ZQREF_OK) return rc;
    }
    return ZQREF_OK;
}
