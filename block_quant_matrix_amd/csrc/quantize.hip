// quantize.hip -- activation block quantization and the fused SwiGLU +
// re-quantization of the MoE expert FFN (gfx950).
//
// Eight lanes own one 32-element block (four elements each, one 16-byte load
// per lane, so a wave quantizes 8 blocks = 1 KB of fp32 per instruction).  The
// block amax, the scale and the code sum are reduced with DPP inside the
// 8-lane group.
#include "zq_common.h"
#include "zq_internal.h"

namespace zq {

__global__ __launch_bounds__(256) void quantize_act_kernel(const float *__restrict__ x,
                                                           int64_t n_blocks, int32_t nb,
                                                           int64_t k, int64_t x_stride,
                                                           int8_t *__restrict__ qx,
                                                           float *__restrict__ dx,
                                                           int32_t *__restrict__ sx) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int g = static_cast<int>(gid & 7);
  if (blk >= n_blocks) return;  // whole 8-lane groups leave together
  const int64_t t = blk / nb;
  const int32_t b = static_cast<int32_t>(blk - t * nb);
  const float4 v = *reinterpret_cast<const float4 *>(x + t * x_stride + b * 32 + g * 4);
  const float xv[4] = {v.x, v.y, v.z, v.w};
  float d;
  int32_t s;
  const uint32_t packed = quantize_block8(xv, d, s);
  *reinterpret_cast<uint32_t *>(qx + t * k + b * 32 + g * 4) = packed;
  if (g == 0) {
    dx[blk] = d;
    if (sx) sx[blk] = s;
  }
}

// h = silu(g) * u in fp64 (silu(z) = z / (1 + exp(-z))), rounded once to
// fp32, then quantized like the activation.
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(const float *__restrict__ gu,
                                                              int64_t n_blocks, int32_t nbf,
                                                              int64_t f, int8_t *__restrict__ qh,
                                                              float *__restrict__ dh,
                                                              int32_t *__restrict__ sh,
                                                              float *__restrict__ h_out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int g = static_cast<int>(gid & 7);
  if (blk >= n_blocks) return;
  const int64_t s = blk / nbf;
  const int32_t b = static_cast<int32_t>(blk - s * nbf);
  const int64_t i0 = b * 32 + g * 4;
  const float4 gv = *reinterpret_cast<const float4 *>(gu + s * 2 * f + i0);
  const float4 uv = *reinterpret_cast<const float4 *>(gu + s * 2 * f + f + i0);
  const float ga[4] = {gv.x, gv.y, gv.z, gv.w};
  const float ua[4] = {uv.x, uv.y, uv.z, uv.w};
  float h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double gd = static_cast<double>(ga[e]);
    const double silu = gd / (1.0 + exp(-gd));
    h[e] = static_cast<float>(silu * static_cast<double>(ua[e]));
  }
  if (h_out) *reinterpret_cast<float4 *>(h_out + s * f + i0) = make_float4(h[0], h[1], h[2], h[3]);
  float d;
  int32_t sum;
  const uint32_t packed = quantize_block8(h, d, sum);
  *reinterpret_cast<uint32_t *>(qh + s * f + i0) = packed;
  if (g == 0) {
    dh[blk] = d;
    if (sh) sh[blk] = sum;
  }
}

int launch_quantize_act(const float *x, int64_t n_tok, int64_t k, int64_t x_stride, int8_t *qx,
                        float *dx, int32_t *sx, hipStream_t stream) {
  const int32_t nb = static_cast<int32_t>(k / 32);
  const int64_t n_blocks = n_tok * nb;
  if (n_blocks == 0) return ZQ_OK;
  const int64_t threads = n_blocks * 8;
  const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
  hipLaunchKernelGGL(quantize_act_kernel, dim3(grid), dim3(256), 0, stream, x, n_blocks, nb, k,
                     x_stride, qx, dx, sx);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

int launch_swiglu_quantize(const float *gu, int64_t n, int64_t f, int8_t *qh, float *dh,
                           int32_t *sh, float *h_out, hipStream_t stream) {
  const int32_t nbf = static_cast<int32_t>(f / 32);
  const int64_t n_blocks = n * nbf;
  if (n_blocks == 0) return ZQ_OK;
  const unsigned grid = static_cast<unsigned>((n_blocks * 8 + 255) / 256);
  hipLaunchKernelGGL(swiglu_quantize_kernel, dim3(grid), dim3(256), 0, stream, gu, n_blocks, nbf,
                     f, qh, dh, sh, h_out);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

}  // namespace zq
