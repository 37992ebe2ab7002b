// zq_float.h -- the float-weight (F16 / F32) DMMV's launcher, shared by
// dmmv_float.hip and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

struct FloatDmmvArgs {
  const uint8_t *w;     // rows x k weights, row-major, 16-byte aligned
  const float *x;       // fp32 activation [k], 16-byte aligned
  float *y;             // output rows
  int64_t rows;
  int64_t row_bytes;    // filled in by the launcher
  int32_t k;            // a multiple of 16 bytes of weights; at most 16384
  uint32_t flags;
};

// wtype ZQ_F16 or ZQ_F32 (arguments already checked).
int launch_dmmv_float(int wtype, FloatDmmvArgs a, hipStream_t stream);

}  // namespace zq
