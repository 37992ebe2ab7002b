// zq_f32in.h -- the fp32-input form of the K-quant DMMV: its argument block
// and launcher, shared by the kernel and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

// K-quant DMMV from the fp32 activation, y (+)= W . Q(x), Q the activation
// quantizer of zq_quantize_act.
struct DmmvKF32Args {
  const uint8_t *w;     // rows x k/256 super-blocks
  const float *x;       // [k], 16-byte aligned
  float *y;             // [rows]
  int8_t *qx_out;       // [k] or null: the quantized activation (workgroup 0)
  float *dx_out;        // [k/32] or null
  int32_t *sx_out;      // [k/32] or null
  int64_t rows;
  int64_t row_bytes;    // filled in by the launcher
  int64_t n_groups;     // filled in by the launcher
  int32_t k;            // a multiple of 256, at most 16384
  int32_t nb;           // k / 32
  uint32_t flags;
};
int launch_dmmv_k_f32(int wtype, DmmvKF32Args a, hipStream_t stream);

}  // namespace zq
