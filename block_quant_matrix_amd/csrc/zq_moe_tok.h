// zq_moe_tok.h -- the several-token MoE block's launcher, shared by moe.hip
// and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zq_internal.h"

namespace zq {

constexpr int kTokMax = 8;  // tokens per several-token MoE call

// The route launch: every token's router and activation codes.
struct MoeTokArgs {
  const float *logits;        // [n_tok][n_routed]
  int32_t n_routed;
  int32_t top_k;
  const float *shared_gate;   // [n_tok] or null
  int32_t n_tok;
  int32_t *ids;               // [n_tok][n_sel]
  float *wts;                 // [n_tok][n_sel]
  const float *x;             // [n_tok][d_model], 16-byte aligned
  int32_t d_model;
  int8_t *qx;                 // [n_tok][d_model]: every token's codes
  float *dx;                  // [n_tok][d_model / 32]
  int32_t *sx;                // [n_tok][d_model / 32]
};

// The down launch and the final sum.
struct MoeDownTokArgs {
  const uint8_t *bank;        // experts of [rows][k]
  int64_t expert_stride;
  int32_t n_experts;
  int32_t *mem;               // [J][kTokMax]: when slot j is the first use of its
                              // expert, the slots of every token that selected that
                              // expert in token order, then -1; all -1 otherwise
                              // (written by the gate/up launch)
  const int32_t *ids;         // [J]: the router's expert ids (filled in by the launcher)
  int32_t n_sel;              // J = n_tok * (top_k (+1)): flattened slots
  int32_t n_tok;
  const int8_t *qh;           // [J][k]
  const float *dh;            // [J][k/32]
  const int32_t *sh;          // [J][k/32]
  const float *wts;           // [J]: the router's weights
  int32_t n_sel_tok;          // slots per token (J / n_tok)
  float *y;                   // [n_tok][rows]
  int64_t rows;               // d_model
  int64_t row_bytes;          // filled in by the launcher
  int32_t k;                  // d_ff
  int32_t nb;                 // filled in by the launcher
  uint32_t flags;
  int32_t *status;
};

bool moe_tok_fits(int64_t d_model, int64_t d_ff);
// route, gate/up (g: bank, stride, n_experts, k = d_model, d_ff, qh / dh /
// sh of J slots, n_sel = J), down with the weighted sums.
int launch_moe_ffn_tok(int wtype, const MoeTokArgs &p, MoeGateUpArgs g, MoeDownTokArgs d,
                       hipStream_t stream);

}  // namespace zq
