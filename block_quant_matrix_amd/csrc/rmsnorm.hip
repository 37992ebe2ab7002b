// rmsnorm.hip -- RMS normalization fused with the activation block
// quantization (gfx950): per token,
//   xn = x * (1 / sqrt(sum(x^2) / k + eps)) * w,   then Q(xn) as quantize.hip.
//
// One 256-thread workgroup per token.  Pass 1: each thread sums the squares
// of its float4 chunks (fused multiply-adds) and the workgroup adds the
// partial sums.  Pass 2: eight lanes per 32-element block normalize four
// elements each ((x * inv) * w, two roundings), optionally store the fp32
// xn, and quantize the block (quantize_block<8>: the same codes, scale and
// sum as zq_quantize_act would give for that xn).
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

__global__ __launch_bounds__(256) void rms_norm_quantize_kernel(const float *x_in, const float *w,
                                                                int64_t x_stride, int32_t k,
                                                                const RmsNormArgs a_in) {
#pragma clang fp contract(off)
  // leading scalars: preloaded kernel arguments (as dmmv_hot in zq_internal.h)
  RmsNormArgs a = a_in;
  a.x = x_in;
  a.w = w;
  a.x_stride = x_stride;
  a.k = k;
  const int64_t t = blockIdx.x;
  const int tid = static_cast<int>(threadIdx.x);
  const float *x = a.x + t * a.x_stride;
  const int nc = a.k / 4;  // float4 chunks; a multiple of 8
  float ss = 0.0f;
  for (int c = tid; c < nc; c += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(x + 4 * c);
    ss = __builtin_fmaf(v.x, v.x, ss);
    ss = __builtin_fmaf(v.y, v.y, ss);
    ss = __builtin_fmaf(v.z, v.z, ss);
    ss = __builtin_fmaf(v.w, v.w, ss);
  }
  ss = block_sum_all<4>(ss);
  const float inv = rms_inv(ss, a.k, a.eps);
  // chunk c is lane c & 7 of block c >> 3: the eight lanes of a group share
  // a block and leave the loop together (nc is a multiple of 8)
  for (int c = tid; c < nc; c += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(x + 4 * c);
    const float4 wv = *reinterpret_cast<const float4 *>(a.w + 4 * c);
    const float xn[4] = {(v.x * inv) * wv.x, (v.y * inv) * wv.y, (v.z * inv) * wv.z,
                         (v.w * inv) * wv.w};
    if (a.xn_out)
      *reinterpret_cast<float4 *>(a.xn_out + t * a.k + 4 * c) = make_float4(xn[0], xn[1], xn[2], xn[3]);
    float d;
    int32_t s;
    const uint32_t packed = quantize_block8(xn, d, s);
    *reinterpret_cast<uint32_t *>(a.qx + t * a.k + 4 * c) = packed;
    if ((c & 7) == 0) {
      const int64_t blk = t * (a.k / 32) + (c >> 3);
      a.dx[blk] = d;
      if (a.sx) a.sx[blk] = s;
    }
  }
}

int launch_rms_norm_quantize(RmsNormArgs a, hipStream_t stream) {
  if (a.n_tok == 0) return ZQ_OK;
  hipLaunchKernelGGL(rms_norm_quantize_kernel, dim3(static_cast<unsigned>(a.n_tok)), dim3(256), 0,
                     stream, a.x, a.w, a.x_stride, a.k, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
