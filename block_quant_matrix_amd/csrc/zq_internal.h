// zq_internal.h -- host-side launchers shared between the libzq translation
// units (argument checking lives in zq_api.hip; these assume valid input).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

enum DmmvMode { MODE_PLAIN = 0, MODE_ISUMS = 1, MODE_GATHER = 2, MODE_WEIGHTED = 3 };

// Everything one DMMV-family launch needs, passed by value.
struct DmmvArgs {
  const uint8_t *w;     // matrix, or bank of matrices (MoE)
  const int8_t *qx;     // activation codes (slot s at qx + s * x_stride)
  const float *dx;      // activation scales (slot s at dx + s * x_stride / 32)
  const int32_t *sx;    // activation block sums, may be null (Q4_0 then sums qx)
  float *y;             // output rows
  int32_t *isums;       // MODE_ISUMS output [rows][nb]
  const int32_t *ids;   // MoE: selected expert ids [n_sel]
  const float *wts;     // MoE weighted sum: weights [n_sel]
  int32_t *status;      // MoE: receives ZQ_ERANGE on a bad id (may be null)
  int64_t rows;
  int64_t row_bytes;
  int64_t expert_stride;
  int64_t x_stride;
  int64_t n_groups;     // row groups per slot
  int32_t nb;           // blocks per row
  int32_t n_experts;
  int32_t n_sel;
  uint32_t flags;
  // last, so that the fields above keep their kernel-argument offsets
  int32_t id_base;      // MoE: expert e = ids[s] - id_base (a bank holding experts id_base..)
  // K-quant weighted sum with a shared expert folded in: w2 [rows][k] in a
  // block format, taken with slot n_sel's activation and weight wts[n_sel]
  const uint8_t *w2;
  int64_t row_bytes2;   // filled in by the launcher
};

// Kernel arguments in SGPRs.  The library is built with kernel-argument
// preloading: a kernel's leading scalar arguments (up to 14 SGPRs' worth)
// are in SGPRs when its waves start, while a struct argument stays in the
// argument segment in memory, a round trip away, and every load whose
// address needs one of its fields waits for that round trip.  So a kernel
// takes the fields its first loads need as leading scalars and the whole
// struct after them, and puts the scalars back into its local copy of the
// struct, so the rest of its code reads one struct.  Pointers come first and
// 32-bit fields last, so that no SGPR is lost to alignment.
//
// DmmvArgs for the single-matrix and gathered forms: the weights, the
// activation and the row groups.
__device__ __forceinline__ void dmmv_hot(DmmvArgs &a, const uint8_t *w, const int8_t *qx,
                                         const float *dx, int64_t rows, int64_t row_bytes,
                                         int64_t n_groups, int32_t nb, int32_t id_base) {
  a.w = w;
  a.qx = qx;
  a.dx = dx;
  a.rows = rows;
  a.row_bytes = row_bytes;
  a.n_groups = n_groups;
  a.nb = nb;
  a.id_base = id_base;
}
#define ZQ_DMMV_HOT(a) (a).w, (a).qx, (a).dx, (a).rows, (a).row_bytes, (a).n_groups, (a).nb, (a).id_base

// The multi-token DMMV: T <= 8 activations, token t at qx + t*k,
// dx / sx + t*nb, output rows at y + t*rows.
struct DmmvTokArgs {
  const uint8_t *w;
  const int8_t *qx;
  const float *dx;
  const int32_t *sx;    // may be null (the kernel then sums the codes)
  float *y;
  int64_t rows;
  int64_t row_bytes;    // filled in by the launcher
  int64_t n_groups;     // filled in by the launcher
  int32_t k;
  int32_t nb;
  int32_t n_tok;
  uint32_t flags;
};
int launch_dmmv_tok(int wtype, DmmvTokArgs a, hipStream_t stream);

// The K-quant weighted sum over n_sel routed slots (wtype) plus the shared
// expert a.w2 in sh_wtype (ZQ_Q4_0 / ZQ_Q8_0) at slot n_sel, in one launch:
// y (+)= sum_s wts[s] W[e_s] x_s + wts[n_sel] W2 x_{n_sel}.
bool dmmv_k_wsum_shared_fits(int wtype, int sh_wtype, int64_t k);
int launch_dmmv_k_wsum_shared(int wtype, int sh_wtype, DmmvArgs a, hipStream_t stream);

// RMS normalization + quantization, one workgroup per token.
struct RmsNormArgs {
  const float *x;       // [n_tok][x_stride]
  const float *w;       // [k]
  int8_t *qx;           // [n_tok][k]
  float *dx;            // [n_tok][k/32]
  int32_t *sx;          // may be null
  float *xn_out;        // [n_tok][k], may be null
  int64_t n_tok;
  int64_t x_stride;
  int32_t k;
  float eps;
};
int launch_rms_norm_quantize(RmsNormArgs a, hipStream_t stream);

// The fused quantize + DMMV launch.
struct DmmvF32Args {
  const uint8_t *w;
  const float *x;       // fp32 activation [k]
  float *y;
  int8_t *qx_out;       // optional copy of the quantized activation
  float *dx_out;
  int32_t *sx_out;
  void *part;           // argmax partials, one (value, index) per workgroup, or null
  int32_t *out_idx;     // argmax of y (needs part), or null
  int64_t rows;
  int64_t row_bytes;    // filled in by the launcher
  int32_t k;
  int32_t nb;
  uint32_t flags;
  // last, so that the fields above keep their offsets in the kernel arguments
  const float *norm_w;  // RMS-norm weight [k]: x is normalized before quantizing, or null
  float *xn_out;        // optional copy of the normalized activation (with norm_w)
  float eps;
};

// With a.part set, the launch is persistent (at most kArgmaxMaxParts
// workgroups walk the row groups) and leaves one argmax partial per
// workgroup; with a.out_idx also set, the final argmax follows.
constexpr int kArgmaxMaxParts = 2048;
int launch_dmmv_f32x(int wtype, DmmvF32Args a, hipStream_t stream);

// DMMV over K-quant super-blocks, wtype ZQ_Q4_K / ZQ_Q5_K / ZQ_Q6_K
// (a.nb = k/32, k a multiple of 256); isums selects the per-32-block integer
// sums instead of rows.
int launch_dmmv_k(int wtype, int mode, DmmvArgs a, hipStream_t stream);
// Reduce nparts (value, index) partials to the argmax index.
int launch_argmax_final(const void *part, int nparts, int32_t *out_idx, hipStream_t stream);

// MoE gate/up pass fused with swiglu + re-quantization.
struct MoeGateUpArgs {
  const uint8_t *bank;  // experts of [2*d_ff rows][k]
  int64_t expert_stride;
  int32_t n_experts;
  const int32_t *ids;
  int32_t n_sel;
  const float *x;       // fp32 activation [k]
  int32_t k;
  int32_t nb;           // filled in by the launcher
  int64_t row_bytes;    // filled in by the launcher
  int32_t d_ff;
  int8_t *qh;           // [n_sel][d_ff]
  float *dh;            // [n_sel][d_ff/32]
  int32_t *sh;          // [n_sel][d_ff/32] or null
  float *h_out;         // [n_sel][d_ff] or null
  float *gu_out;        // [n_sel][2*d_ff] or null
  int32_t *status;
  // With logits set, the workgroups select the experts themselves (the
  // router of zq_moe_route) instead of reading ids: slot s < top_k takes the
  // expert of rank s, slot top_k the shared expert (id n_routed); the
  // workgroup of slot 0, block 0 also writes ids_out / wts_out.
  const float *logits;  // [n_routed] or null
  int32_t n_routed;
  int32_t top_k;
  const float *shared_gate;
  int32_t *ids_out;
  float *wts_out;
  // last, so that the fields above keep their kernel-argument offsets
  int32_t id_base;      // without logits: expert e = ids[s] - id_base
  // the mixed launch: the shared expert's [2*d_ff][k] matrix in its own
  // format (slot top_k)
  const uint8_t *bank2;
  int64_t row_bytes2;   // filled in by the launcher
};

// MoE down pass with the weighted sum over the selected experts fused in.
struct MoeDownArgs {
  const uint8_t *bank;  // experts of [rows][k]
  int64_t expert_stride;
  int32_t n_experts;
  const int32_t *ids;
  const float *wts;
  int32_t n_sel;
  const int8_t *qx;     // slot s at qx + s * x_stride
  const float *dx;
  const int32_t *sx;
  int64_t x_stride;
  int32_t k;
  int32_t nb;           // filled in by the launcher
  int64_t rows;
  int64_t row_bytes;    // filled in by the launcher
  float *y;
  uint32_t flags;
  int32_t *status;
  // last, so that the fields above keep their kernel-argument offsets
  int32_t id_base;      // expert e = ids[s] - id_base
};

int launch_moe_gate_up(int wtype, MoeGateUpArgs a, hipStream_t stream);
int launch_moe_down(int wtype, MoeDownArgs a, hipStream_t stream);
// The gate/up pass over K-quant experts (wtype ZQ_Q4_K / ZQ_Q5_K / ZQ_Q6_K):
// d_model of 1024, 2048 or 4096 (one 64-element unit per lane, one pass).
bool moe_gate_up_k_fits(int64_t d_model);
int launch_moe_gate_up_k(int wtype, MoeGateUpArgs a, hipStream_t stream);
// Routed experts (wtype, a.bank, router folded in: a.logits set) and the
// shared expert (sh_wtype, one matrix at a.bank2) in one gate/up launch of
// top_k + 1 slots; any of the five formats each, d_model of 1024 or 2048.
bool moe_gate_up_mix_fits(int64_t d_model);
int launch_moe_gate_up_mix(int wtype, int sh_wtype, MoeGateUpArgs a, hipStream_t stream);
size_t moe_down_lds_bytes(int64_t n_sel, int64_t k);
bool moe_gate_up_fits(int64_t d_model);
bool moe_down_fits(int64_t n_sel, int64_t k);
int launch_quantize_act(const float *x, int64_t n_tok, int64_t k, int64_t x_stride, int8_t *qx,
                        float *dx, int32_t *sx, hipStream_t stream);
int launch_swiglu_quantize(const float *gu, int64_t n, int64_t f, int8_t *qh, float *dh,
                           int32_t *sh, float *h_out, hipStream_t stream);
// mode: DmmvMode; a.n_groups and a.row_bytes are filled in by the launcher.
int launch_dmmv(int wtype, int mode, DmmvArgs a, hipStream_t stream);
int launch_argmax(const float *y, int64_t n, int32_t *out_idx, void *ws, hipStream_t stream);
size_t argmax_workspace(int64_t n);
int launch_moe_route(const float *logits, int32_t n_routed, int32_t top_k, const float *shared_gate,
                     int32_t *ids, float *wts, hipStream_t stream);
int launch_gemm(int wtype, const void *w, int64_t n, int64_t k, const int8_t *qx, const float *dx,
                int64_t m, float *y, uint32_t flags, int32_t *isums, int64_t m0, int64_t m1,
                int64_t n0, int64_t n1, hipStream_t stream);

}  // namespace zq
