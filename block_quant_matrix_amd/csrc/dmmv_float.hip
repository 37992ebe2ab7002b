// dmmv_float.hip -- DMMV over plain float weight matrices (F16 / F32) against
// the fp32 activation (gfx950).
//
//   y[r] (+)= sum_j w[r][j] * x[j]
//
// A float matrix has no blocks to pair with int8 codes, so the activation
// stays fp32; every product is an fp16 (or fp32) weight times an fp32 value,
// accumulated in fp32 (v_fma_mix_f32 converts the half operand inside the
// fused multiply-add, one instruction per element).
//
// Mapping: the row is cut into 16-byte chunks (8 F16 or 4 F32 weights) and
// lane l of a wave owns chunks l, l + 64, l + 128, ... of every row it
// visits, so one load instruction of a wave covers 1 KB of one row,
// coalesced.  A wave takes RB rows at a time and requests all of their
// chunks of one step (RB x U 16-byte loads per lane) before any arithmetic;
// the activation is staged once per workgroup in LDS and read as 16-byte
// pieces beside the weights.  The RB rows are folded across the wave by the
// permlane-swap halvings and a DPP sum (RowReduce).  Waves walk row groups
// with a grid stride, so a workgroup's staged activation serves every row
// group it visits.
#include "zq_common.h"
#include "zq_float.h"
#include "zq_internal.h"

namespace zq {

namespace {

constexpr int kFloatMaxGrid = 4096;  // workgroups of a persistent launch

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
// global-address-space views, so the loads are global_load (vmcnt only)
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

}  // namespace

template <int WT, int RB, int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void dmmv_float_kernel(const uint8_t *w, const float *x,
                                                                   int64_t rows, int64_t row_bytes,
                                                                   int32_t k,
                                                                   const FloatDmmvArgs a_in) {
  // leading scalars: preloaded kernel arguments (as dmmv_hot in zq_internal.h)
  FloatDmmvArgs a = a_in;
  a.w = w;
  a.x = x;
  a.rows = rows;
  a.row_bytes = row_bytes;
  a.k = k;
  extern __shared__ __attribute__((aligned(16))) float xs[];
  constexpr int EPC = WT == ZQ_F16 ? 8 : 4;   // weights per 16-byte chunk
  const int nch = a.k / EPC;
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int wave = static_cast<int>(threadIdx.x >> 6);
  const int64_t n_groups = (a.rows + RB - 1) / RB;
  const int64_t wstride = static_cast<int64_t>(gridDim.x) * WPB;
  int64_t grp = static_cast<int64_t>(blockIdx.x) * WPB + wave;

  // Request the first row group's weights before staging the activation.
  u32x4 wv[RB][U];
  auto load_group = [&](int64_t g, int c0) {
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      int64_t row = g * RB + t;
      row = row < a.rows ? row : a.rows - 1;
      const uint8_t *base = a.w + row * a.row_bytes;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int c = c0 + lane + 64 * u;
        c = c < nch ? c : nch - 1;
        wv[t][u] = *(const g_u32x4 *)(base + 16 * static_cast<int64_t>(c));
      }
    }
  };
  if (grp < n_groups) load_group(grp, 0);
  for (int i = static_cast<int>(threadIdx.x) * 4; i < a.k; i += 64 * WPB * 4)
    *reinterpret_cast<u32x4 *>(xs + i) = *(const g_u32x4 *)(a.x + i);
  __syncthreads();

  for (; grp < n_groups; grp += wstride) {
    float acc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) acc[t] = 0.0f;
    for (int c0 = 0;;) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + lane + 64 * u;
        if (c < nch) {
          if constexpr (WT == ZQ_F16) {
            const float4 x0 = *reinterpret_cast<const float4 *>(xs + 8 * c);
            const float4 x1 = *reinterpret_cast<const float4 *>(xs + 8 * c + 4);
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int t = 0; t < RB; ++t) {
              const uint32_t d[4] = {wv[t][u].x, wv[t][u].y, wv[t][u].z, wv[t][u].w};
              float s = acc[t];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const h2 h = __builtin_bit_cast(h2, d[e]);
                s = __builtin_fmaf(static_cast<float>(h.x), xv[2 * e], s);
                s = __builtin_fmaf(static_cast<float>(h.y), xv[2 * e + 1], s);
              }
              acc[t] = s;
            }
          } else {
            const float4 x0 = *reinterpret_cast<const float4 *>(xs + 4 * c);
            const float xv[4] = {x0.x, x0.y, x0.z, x0.w};
#pragma unroll
            for (int t = 0; t < RB; ++t) {
              const uint32_t d[4] = {wv[t][u].x, wv[t][u].y, wv[t][u].z, wv[t][u].w};
              float s = acc[t];
#pragma unroll
              for (int e = 0; e < 4; ++e) s = __builtin_fmaf(__builtin_bit_cast(float, d[e]), xv[e], s);
              acc[t] = s;
            }
          }
        }
      }
      c0 += 64 * U;
      if (c0 >= nch) break;
      load_group(grp, c0);
    }
    // the next row group's first step is requested before this group's
    // reduction and stores
    const int64_t next = grp + wstride;
    if (next < n_groups) load_group(next, 0);

    using R = RowReduce<64, RB>;
    float res[R::NOUT];
    R::run(acc, res);
    if (R::writer(lane)) {
#pragma unroll
      for (int m = 0; m < R::NOUT; ++m) {
        const int64_t row = grp * RB + R::rowstep(m, lane);
        if (row < a.rows) {
          float *yp = a.y + row;
          *yp = (a.flags & ZQ_ACCUMULATE) ? *yp + res[m] : res[m];
        }
      }
    }
  }
}

namespace {

template <int WT, int RB, int U, int WPB = 4>
int launch_fl(const FloatDmmvArgs &a, hipStream_t stream) {
  const int64_t n_groups = (a.rows + RB - 1) / RB;
  int64_t grid = (n_groups + WPB - 1) / WPB;
  if (grid > kFloatMaxGrid) grid = kFloatMaxGrid;
  const size_t lds = static_cast<size_t>(a.k) * 4;
  hipLaunchKernelGGL((dmmv_float_kernel<WT, RB, U, WPB>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WPB), lds, stream, a.w, a.x, a.rows, a.row_bytes, a.k, a);
  ZQ_LAUNCH_CHECK();
  return ZQ_OK;
}

// U 16-byte chunks per lane and step (at most 8, enough for one pass over
// rows of up to 512 chunks) and RB rows per wave, RB * U <= 16 loads in
// flight per lane; 8 waves per workgroup, so each workgroup's staged
// activation serves twice the rows of 4 waves.  From a sweep of 1/2/4 rows
// x 4/8/16 waves (F16, us per launch):
//   8 or more chunks per lane: one row per step, 4096 x 4096 8.02 (2 rows,
//     4 waves: 8.35), 14336 x 4096 22.99 (23.84), 4096 x 14336 23.77
//     (25.16), F32 4096 x 4096 13.27 (14.13);
//   4 chunks per lane: 4 rows per step on the LM head, 248 320 x 2048
//     156.6 (4 waves: 170.2), one row elsewhere, 2048 x 2048 3.94 (4.21).
template <int WT>
int launch_fw(const FloatDmmvArgs &a, hipStream_t stream) {
  constexpr int EPC = WT == ZQ_F16 ? 8 : 4;
  const int cpl = (a.k / EPC + 63) / 64;
  if (cpl <= 1) return launch_fl<WT, 4, 1>(a, stream);
  if (cpl <= 2) return launch_fl<WT, 4, 2>(a, stream);
  if (cpl <= 4) {
    if (a.rows >= 65536) return launch_fl<WT, 4, 4, 8>(a, stream);
    return launch_fl<WT, 1, 4, 8>(a, stream);
  }
  return launch_fl<WT, 1, 8, 8>(a, stream);
}

}  // namespace

int launch_dmmv_float(int wtype, FloatDmmvArgs a, hipStream_t stream) {
  if (a.rows == 0) return ZQ_OK;
  a.row_bytes = static_cast<int64_t>(a.k) * (wtype == ZQ_F16 ? 2 : 4);
  if (wtype == ZQ_F16) return launch_fw<ZQ_F16>(a, stream);
  return launch_fw<ZQ_F32>(a, stream);
}

}  // namespace zq
